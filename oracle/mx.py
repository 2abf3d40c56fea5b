"""Microscaled (MX) fp8 e4m3 quantisation in float64 (test infrastructure only).

Source: the block quantisation of FP8 attention in "FlashAttention-3: почему
внимание стало быстрее" (review), section «Метод», item 3, and the random
orthogonal rotation of "FlashAttention-3: Fast & Accurate Attention with
Asynchrony & Low-Precision" (Embodied AI 101 transcript), section
"Incoherent Processing for FP8 Accuracy". The pages fix neither the block
shape nor the scale format; this module is the finer-grained variant with
the block shape and power-of-two scales of the OCP Microscaling (MX)
formats, which the gfx950 scaled matrix instructions consume directly.

Readings (listed in the design notes):
* a block is 32 consecutive elements along one axis: along d for Q and K
  (one scale per row and 32 columns), along the sequence for V (one scale per
  column and 32 rows; the last block of a head may be shorter);
* the shared scale is X = 2^e with e = floor(log2(amax)) - 8 (8 = the
  exponent of the largest e4m3 normal, 448 = 1.75 * 2^8), clamped to the
  E8M0 range [-127, 127]; an all-zero block has e = -127;
* element code = e4m3 round-to-nearest-even of x / X, saturated to +-448
  (x / X lies in [256, 512) for the largest element of a block, so the top
  of that range clamps);
* the value is decode(code) * X; the stored scale byte is e + 127;
* optionally (along d only, prescale = p) the rotated float32 values are
  multiplied by p in float32 before the block maximum, so the codes and
  exponents represent x * p (the form in which Q carries
  softmax_scale * log2(e) for the fp8 forward).
The rotated values are formed in float64 and rounded once to float32 before
the block maximum (the GPU's precision, as for the per-128-row quantiser);
x / X is exact in float32 because X is a power of two.
"""

import numpy as np

from .fp8 import E4M3_MAX, e4m3_encode, e4m3_decode
from .hadamard import random_sign_hadamard

MX_BLOCK = 32
EMAX_E4M3 = 8


def _block_exponents(amax):
    """e = floor(log2(amax)) - 8 clamped to [-127, 127]; -127 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - EMAX_E4M3
    e = np.where(amax > 0, e, -127.0)
    return np.clip(e, -127, 127).astype(np.int32)


def mx_quantize(x, axis, signs=None, prescale=None):
    """MX e4m3 quantisation of x [B, H, N, d].

    axis: "d" (blocks of 32 columns of a row: Q, K) or "n" (blocks of 32
    rows of a column: V). signs: [H, d] of +-1 to apply the random-sign
    Hadamard along d first (Q and K), or None. prescale: None, or a float32
    factor applied to the rotated values (axis "d" only).
    Returns (codes uint8 [B,H,N,d], exponents int32: [B,H,N,d/32] for "d",
    [B,H,ceil(N/32),d] for "n").
    """
    x = np.asarray(x, dtype=np.float64)
    if signs is not None:
        x = random_sign_hadamard(x, signs)
    y = x.astype(np.float32)
    if prescale is not None:
        if axis != "d":
            raise ValueError("prescale is defined along d only")
        y = (y * np.float32(prescale)).astype(np.float32)
    y = y.astype(np.float64)
    B, H, N, d = y.shape
    if axis == "d":
        if d % MX_BLOCK:
            raise ValueError("d must be a multiple of 32")
        blocks = y.reshape(B, H, N, d // MX_BLOCK, MX_BLOCK)
        e = _block_exponents(np.max(np.abs(blocks), axis=-1))         # [B,H,N,d/32]
        scaled = blocks * np.exp2(-e.astype(np.float64))[..., None]
        codes = e4m3_encode(np.clip(scaled, -E4M3_MAX, E4M3_MAX)).reshape(B, H, N, d)
        return codes, e
    if axis == "n":
        nb = (N + MX_BLOCK - 1) // MX_BLOCK
        pad = np.zeros((B, H, nb * MX_BLOCK, d))
        pad[:, :, :N] = y
        blocks = pad.reshape(B, H, nb, MX_BLOCK, d)
        e = _block_exponents(np.max(np.abs(blocks), axis=3))           # [B,H,nb,d]
        scaled = blocks * np.exp2(-e.astype(np.float64))[:, :, :, None, :]
        codes = e4m3_encode(np.clip(scaled, -E4M3_MAX, E4M3_MAX)).reshape(B, H, nb * MX_BLOCK, d)
        return codes[:, :, :N], e
    raise ValueError("axis must be 'd' or 'n'")


def mx_dequantize(codes, exps, axis):
    """decode(code) * 2^e in float64, inverse layout of mx_quantize."""
    v = e4m3_decode(codes)
    B, H, N, d = v.shape
    s = np.exp2(np.asarray(exps, dtype=np.float64))
    if axis == "d":
        return (v.reshape(B, H, N, d // MX_BLOCK, MX_BLOCK) * s[..., None]).reshape(B, H, N, d)
    rows = np.repeat(s, MX_BLOCK, axis=2)[:, :, :N]
    return v * rows


def fake_quant_attention_mx(q, k, v, signs=None, causal=False, scale=None, prescaled=False):
    """Exact float64 attention of the MX-dequantised inputs (Q, K along d
    after the optional random-sign Hadamard; V along the sequence).
    prescaled: Q quantised as x * float32(scale * log2(e)); the dequantised
    logits are then base-2 exponents and the attention takes the softmax
    scale ln(2). Returns (O, LSE)."""
    from .attention import attention
    d = np.asarray(q).shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    pq = np.float32(scale * np.log2(np.e)) if prescaled else None
    qc, qe = mx_quantize(q, "d", signs, prescale=pq)
    kc, ke = mx_quantize(k, "d", signs)
    vc, ve = mx_quantize(v, "n", None)
    return attention(mx_dequantize(qc, qe, "d"), mx_dequantize(kc, ke, "d"),
                     mx_dequantize(vc, ve, "n"), causal, np.log(2.0) if prescaled else scale)
