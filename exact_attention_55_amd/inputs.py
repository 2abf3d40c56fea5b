"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This module only draws random numbers and rounds them to the input dtype; it
holds none of the attention arithmetic, so both the GPU path and the CPU
oracle can take their inputs from here without sharing any of the method.

Recipe (the pages measure on synthetic data only: head dim 128 and sequence
length 8K in the ping-pong ablation of "FlashAttention-3: Fast & Accurate
Attention with Asynchrony & Low-Precision", section "Overlapping GEMM and
Softmax", and 0.1% large outliers in its section "Incoherent Processing for
FP8 Accuracy"):

* numpy.random.default_rng(seed); float32 standard normals of shape
  [B, H, N, d], drawn in the order Q, K, V;
* with outliers: after the three base draws, for each of Q, K, V in turn a
  mask (uniform < p, p = 0.001) and values N(0, sigma^2) with sigma = 10 are
  drawn and added where the mask is set;
* the float32 values are rounded once to the 16-bit input dtype (round to
  nearest even, torch CPU cast). Every consumer reads the rounded values.
* Hadamard sign vectors: default_rng(seed + 1000), +-1 int8 of shape [H, d].
"""

import numpy as np
import torch

# Workloads: (name, B, H, N, d, causal, dtype, seed, outliers)
CONFIGS = {
    "tiny_fp16": dict(B=1, H=1, N=256, d=64, causal=False, dtype="fp16", seed=0),
    "b8h16n2k_d128": dict(B=8, H=16, N=2048, d=128, causal=False, dtype="bf16", seed=1),
    "b8h16n2k_d128_causal": dict(B=8, H=16, N=2048, d=128, causal=True, dtype="bf16", seed=1),
    "b4h32n4k_d64": dict(B=4, H=32, N=4096, d=64, causal=False, dtype="bf16", seed=2),
    "b2h16n8k_d128_causal": dict(B=2, H=16, N=8192, d=128, causal=True, dtype="bf16", seed=5),
    # the same shape and inputs without the mask (the long-context d = 128
    # regime, non-causal)
    "b2h16n8k_d128": dict(B=2, H=16, N=8192, d=128, causal=False, dtype="bf16", seed=5),
    "b2h8n16k_d256_causal": dict(B=2, H=8, N=16384, d=256, causal=True, dtype="bf16", seed=3),
    "fp8_b4h16n4k_d128": dict(B=4, H=16, N=4096, d=128, causal=False, dtype="bf16", seed=4,
                              outliers=True),
}

# Decode workloads (few new query rows against a long key/value history; the
# pages name autoregressive sampling but give no shapes): B sequences, H query
# heads sharing Hkv key/value heads, Nq new rows, Nk cached keys; with
# ragged=True the key count of each sequence is drawn uniformly from
# [Nk/8, Nk].
DECODE_CONFIGS = {
    "decode_b8h16_nk16k_d128": dict(B=8, H=16, Hkv=16, Nq=1, Nk=16384, d=128, causal=True,
                                    dtype="bf16", seed=6),
    "decode_gqa_b16h64kv8_nk8k_ragged": dict(B=16, H=64, Hkv=8, Nq=1, Nk=8192, d=128, causal=True,
                                             dtype="bf16", seed=7, ragged=True),
}

TORCH_DTYPES = {"bf16": torch.bfloat16, "fp16": torch.float16}


def make_qkv(B, H, N, d, seed, dtype="bf16", outliers=False, p_outlier=1e-3,
             sigma_outlier=10.0, **_):
    """Return q, k, v as CPU torch tensors of the 16-bit dtype, [B,H,N,d]."""
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    base = [rng.standard_normal(shape, dtype=np.float32) for _ in range(3)]
    if outliers:
        for x in base:
            mask = rng.random(shape, dtype=np.float32) < p_outlier
            vals = rng.normal(0.0, sigma_outlier, size=shape).astype(np.float32)
            x += np.where(mask, vals, np.float32(0.0))
    tdt = TORCH_DTYPES[dtype]
    return tuple(torch.from_numpy(x).to(tdt) for x in base)


def make_dout(B, H, N, d, seed, dtype="bf16"):
    """Upstream gradient dL/dO for the backward: float32 standard normals
    [B,H,N,d] from default_rng(seed), one RNE cast to the 16-bit dtype."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, N, d), dtype=np.float32)
    return torch.from_numpy(x).to(TORCH_DTYPES[dtype])


def make_decode(B, H, Hkv, Nq, Nk, d, seed, dtype="bf16", ragged=False, **_):
    """Decode inputs: q [B,H,Nq,d], k and v [B,Hkv,Nk,d] (float32 standard
    normals drawn in the order q, k, v from default_rng(seed), one RNE cast to
    the 16-bit dtype), and seqlens (int32 [B] drawn afterwards from
    [Nk // 8, Nk] when ragged, else None)."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, Nq, d), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Nk, d), dtype=np.float32)
    lens = rng.integers(Nk // 8, Nk + 1, size=B).astype(np.int32) if ragged else None
    tdt = TORCH_DTYPES[dtype]
    out = tuple(torch.from_numpy(x).to(tdt) for x in (q, k, v))
    return out + (None if lens is None else torch.from_numpy(lens),)


def make_signs(H, d, seed):
    """+-1 sign vectors [H, d] int8 for the random-sign Hadamard."""
    rng = np.random.default_rng(seed + 1000)
    return (rng.integers(0, 2, size=(H, d), dtype=np.int8) * 2 - 1).astype(np.int8)


def to_f64(t):
    """Exact float64 copy of a CPU tensor (for the oracle)."""
    return t.to(torch.float64).numpy()


def attention_flops(B, H, N, d, causal):
    """The metric's work count: 4*B*H*N^2*d, halved for causal."""
    f = 4.0 * B * H * N * N * d
    return f / 2 if causal else f
