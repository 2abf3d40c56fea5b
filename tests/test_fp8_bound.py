"""CPU check of fp8_p_rounding_bound (the elementwise bound the fp8 GPU
tests use on rows with few keys): a float64 emulation of P' = 8 p w rounded
to e4m3 with the oracle's e4m3 rounding stays within it, and the bound is
not vacuous (the emulated error reaches a fair part of it)."""

import numpy as np
import pytest

import oracle
from exact_attention_55_amd.inputs import make_qkv, make_signs, to_f64

from helpers import fp8_p_rounding_bound


def emulate(qd, kd, vd, rows, causal, w):
    """O with P' = 8 p w rounded to e4m3 (p against the row maximum), the V
    factor 1/w undone after the product and the row sum from the unrounded p."""
    q = qd[0, 0][rows]
    k, v = kd[0, 0], vd[0, 0]
    N, d = k.shape
    s = (q @ k.T) / np.sqrt(d)
    if causal:
        s = np.where(np.arange(N)[None, :] <= np.asarray(rows)[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    pq = oracle.e4m3_round(8.0 * p * w[None, :])
    return (pq @ (v / w[:, None])) / (8.0 * p.sum(axis=1, keepdims=True))


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("blocks", [False, True])
def test_bound_covers_emulated_rounding(causal, blocks):
    N, d = 300, 64
    q, k, v = make_qkv(1, 1, N, d, seed=5, dtype="bf16", outliers=True)
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    signs = make_signs(1, d, 5)
    qc, qs = oracle.fp8_quantize(q64, signs, 128)
    kc, ks = oracle.fp8_quantize(k64, signs, 128)
    vc, vs = oracle.fp8_quantize(v64, None, 128)
    qd, kd, vd = (oracle.fp8_dequantize(c, sc) for c, sc in ((qc, qs), (kc, ks), (vc, vs)))
    w = np.repeat(vs[0, 0] / vs[0, 0].max(), 128)[:N] if blocks else np.ones(N)
    rows = np.arange(N)
    o_fq, _ = oracle.attention(qd, kd, vd, causal)
    o_em = emulate(qd, kd, vd, rows, causal, w)
    err = np.abs(o_em - o_fq[0, 0])
    bound = fp8_p_rounding_bound(qd, kd, vd, 0, 0, rows, causal, None if not blocks else w)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    assert np.max(err / np.maximum(bound, 1e-30)) > 0.05


def _bf16(x):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("scale", [0.125, 1.5])
def test_p16_bound_covers_emulated_rounding(causal, scale):
    """p16_rounding_bound (the elementwise bound the bf16 GPU tests use where
    one to three keys carry a row) holds for a float64 emulation of weights
    rounded to bf16 and normalised by their rounded sum, reaches a fair part
    of the emulated error, and fails a planted mistake (normalising by the
    unrounded sum with weights rounded to bf16 after scaling by 1.01)."""
    from helpers import p16_rounding_bound
    N, d = 200, 64
    q, k, v = make_qkv(1, 1, N, d, seed=9, dtype="bf16")
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o_ref, _ = oracle.attention(q64, k64, v64, causal, scale)
    s = scale * (q64[0, 0] @ k64[0, 0].T)
    if causal:
        s = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    r = _bf16(p)
    o_em = (r @ v64[0, 0]) / r.sum(axis=1, keepdims=True)
    bound = p16_rounding_bound(q64, k64, v64, 0, 0, causal, scale)
    err = np.abs(o_em - o_ref[0, 0])
    assert np.all(err <= bound)
    assert np.max(err / bound) > 0.05
    bad = (_bf16(1.01 * p) @ v64[0, 0]) / p.sum(axis=1, keepdims=True)
    assert np.any(np.abs(bad - o_ref[0, 0]) > bound)
