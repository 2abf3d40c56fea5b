"""GPU parity of the microscaled FP8 path: fa_mx_prep (E8M0 scale per 32
elements, along d for Q/K after the optional random-sign Hadamard, along the
sequence for V) against the oracle quantiser, and fa_fwd with FA_FP8_MX
against the exact attention of the unquantised inputs and the attention of
the oracle's own dequantised inputs.

Codes and exponents: without the Hadamard every float32 step is reproduced
(x * 2^-e is exact), so both must be identical. With it, the GPU's float32
butterflies round differently from the float64 transform: a block whose
maximum sits at a power of two may take the neighbouring exponent, and a
value at an e4m3 rounding boundary the neighbouring code; both must be rare.
"""

import sys

import numpy as np
import pytest
import torch

import oracle
import exact_attention_55_amd as fa
from exact_attention_55_amd.inputs import CONFIGS, make_qkv, make_signs, to_f64
from oracle.mx import fake_quant_attention_mx, mx_dequantize, mx_quantize

from helpers import FP8_RMSE, check_lse, errors, fp8_p_rounding_bound, half_ulp, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_mx(x, signs, axis):
    B, H, N, d = x.shape
    sd = None if signs is None else torch.from_numpy(signs).to(DEV)
    packed = fa.mx_prep(x.to(DEV), sd, axis)
    torch.cuda.synchronize()
    codes = packed[: B * H * N * d].view(B, H, N, d).cpu().numpy()
    sc = fa.mx_scales_view(packed, B, H, N, d, axis).cpu().numpy().astype(np.int32) - 127
    if axis == "n":   # [B,H,nb,32,d/32] -> [B,H,nb,d] with column c at [c % 32, c // 32]
        nb = sc.shape[2]
        sc = sc.transpose(0, 1, 2, 4, 3).reshape(B, H, nb, d)
    return packed, codes, sc


def compare_mx(codes, exps, rc, re, axis, exact):
    if exact:
        np.testing.assert_array_equal(exps, re)
        np.testing.assert_array_equal(codes, rc)
        return
    bad_blocks = exps != re
    assert bad_blocks.mean() <= 1e-3, f"{bad_blocks.mean():.2e} of block exponents differ"
    B, H, N, d = codes.shape
    if axis == "d":
        same = np.repeat(~bad_blocks, 32, axis=-1)
    else:
        same = np.repeat(~bad_blocks, 32, axis=2)[:, :, :N]
    diff = (codes != rc) & same
    assert diff.mean() <= 1e-3, f"{diff.mean():.2e} of codes differ"
    if diff.any():
        a = oracle.e4m3_decode(codes[diff])
        b = oracle.e4m3_decode(rc[diff])
        mag = np.maximum(np.maximum(np.abs(a), np.abs(b)), 2.0 ** -6)
        assert np.all(np.abs(a - b) <= 2.0 ** (np.floor(np.log2(mag)) - 3))


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("had", [False, True])
def test_prep_along_d(d, had):
    say(f"mx prep along d, d={d} had={had}")
    B, H, N = 2, 3, 300
    x, _, _ = make_qkv(B, H, N, d, seed=61 + d, dtype="bf16", outliers=True)
    signs = make_signs(H, d, 61) if had else None
    _, codes, exps = gpu_mx(x, signs, "d")
    rc, re = mx_quantize(to_f64(x), "d", signs)
    compare_mx(codes, exps, rc, re, "d", exact=not had)


@pytest.mark.parametrize("d,N,dtype", [(64, 300, "bf16"), (128, 257, "fp16"), (256, 96, "bf16")])
def test_prep_along_n(d, N, dtype):
    say(f"mx prep along n, d={d} N={N} {dtype}")
    x, _, _ = make_qkv(2, 2, N, d, seed=67 + d, dtype=dtype, outliers=True)
    x[0, 1, 32:64] = 0                          # an all-zero block
    _, codes, exps = gpu_mx(x, None, "n")
    rc, re = mx_quantize(to_f64(x), "n")
    compare_mx(codes, exps, rc, re, "n", exact=True)
    assert np.all(exps[0, 1, 1] == -127)


def mx_run(q, k, v, signs, causal, out_f32=True):
    B, H, N, d = q.shape
    q8, _, _ = gpu_mx(q, signs, "d")
    k8, _, _ = gpu_mx(k, signs, "d")
    v8, _, _ = gpu_mx(v, None, "n")
    o, lse = fa.fwd_fp8(q8, k8, v8, B, H, N, d, causal=causal, out_f32=out_f32, mx=True)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("B,H,N,d,causal", [
    (1, 2, 300, 64, False), (1, 2, 300, 64, True), (2, 2, 640, 128, False),
    (1, 2, 520, 128, True), (1, 1, 384, 256, False), (1, 1, 200, 256, True), (2, 3, 33, 128, False),
])
def test_mx_forward_vs_oracles(B, H, N, d, causal):
    say(f"mx forward B={B} H={H} N={N} d={d} causal={causal}")
    q, k, v = make_qkv(B, H, N, d, seed=71 + N, dtype="bf16")
    signs = make_signs(H, d, 71)
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o, lse = mx_run(q, k, v, signs, causal)
    assert np.all(np.isfinite(o))
    o_ref, _ = oracle.attention(q64, k64, v64, causal)
    _, rmse = errors(o, o_ref)
    assert rmse <= FP8_RMSE, f"fp8 MX RMSE {rmse:.3e}"
    o_fq, lse_fq = fake_quant_attention_mx(q64, k64, v64, signs, causal)
    check_lse(lse, lse_fq)
    _, rmse_fq = errors(o, o_fq)
    assert rmse_fq <= FP8_RMSE / 2, f"RMSE vs fake-quant {rmse_fq:.3e}"


@pytest.mark.parametrize("causal,d", [(False, 128), (True, 128), (False, 256)])
def test_mx_late_score_jump(causal, d):
    """As the block-scaled case: keys eight times longer than the rest in
    tiles after the first push P' past the e4m3 maximum against the first
    tile's maximum, so those tiles take the exact-maximum redo. Every row is
    held elementwise to exact attention of the oracle's own MX-quantised
    inputs within the bound on the e4m3 rounding of P' = 8 p, and the LSE
    to it within 1e-3."""
    B, H, N = 1, 2, 600
    say(f"mx late score jump causal={causal} d={d}")
    q, k, v = make_qkv(B, H, N, d, seed=59, dtype="bf16")
    k = k.clone()
    k[:, :, [300, 301, 455]] *= 8
    signs = make_signs(H, d, 59)
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o, lse = mx_run(q, k, v, signs, causal)
    assert np.all(np.isfinite(o))
    qc, qe = mx_quantize(q64, "d", signs)
    kc, ke = mx_quantize(k64, "d", signs)
    vc, ve = mx_quantize(v64, "n", None)
    qd, kd, vd = mx_dequantize(qc, qe, "d"), mx_dequantize(kc, ke, "d"), mx_dequantize(vc, ve, "n")
    o_fq, lse_fq = oracle.attention(qd, kd, vd, causal)
    s = np.einsum("bhid,bhjd->bhij", qd, kd) / np.sqrt(d)
    assert np.max(lse_fq - s[..., :64].max(-1)) * np.log2(np.e) > 8
    check_lse(lse, lse_fq)
    rows = np.arange(N)
    for h in range(H):
        bound = fp8_p_rounding_bound(qd, kd, vd, 0, h, rows, causal) + 1e-5
        err = np.abs(o[0, h] - o_fq[0, h])
        assert np.all(err <= bound), f"head {h}: worst excess {np.max(err - bound):.3e}"


@pytest.mark.parametrize("d", [64, 128, 256])
def test_mx_single_key(d):
    """N = 1: the one quantised weight is exactly P' = 8, undone by the 2^-3
    PV scale, so O is the dequantised V row times 1/l, where l differs from 1
    only by the float32 rounding of the logit and of exp2 (relative 1e-5 is
    far below the e4m3 step 2^-4); the LSE is the one logit of the
    dequantised Q and K."""
    say(f"mx single key d={d}")
    q, k, v = make_qkv(2, 2, 1, d, seed=73 + d, dtype="bf16")
    signs = make_signs(2, d, 73)
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    for causal in (False, True):
        o, lse = mx_run(q, k, v, signs, causal)
        o_fq, lse_fq = fake_quant_attention_mx(q64, k64, v64, signs, causal)
        np.testing.assert_allclose(o, o_fq, rtol=1e-5, atol=0)
        check_lse(lse, lse_fq)


def test_mx_outlier_workload():
    """The fp8 outlier workload at full size with microscaling and the
    Hadamard: within the RMSE bound and below plain per-tensor fp8 (sampled
    rows); LSE against the oracle's own MX-quantised inputs on one head."""
    cfg = CONFIGS["fp8_b4h16n4k_d128"]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    say("mx outlier workload")
    q, k, v = make_qkv(**cfg)
    signs = make_signs(H, d, cfg["seed"])
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o_mx, lse_mx = mx_run(q, k, v, signs, False)
    # plain per-tensor baseline through the block-scaled path
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    q8, k8, v8 = (fa.fp8_prep(t, None, 0) for t in (qd, kd, vd))
    o_pt, _ = fa.fwd_fp8(q8, k8, v8, B, H, N, d, False, out_f32=True)
    o_pt = o_pt.cpu().numpy()
    sq_mx, sq_pt = [], []
    for b, h in ((0, 0), (B - 1, H - 1), (1, 7)):
        rows = sample_rows(N, seed=b * 50 + h)
        o_ref, _ = oracle.attention_rows(q64, k64, v64, b, h, rows, False)
        sq_mx.append((o_mx[b, h, rows] - o_ref) ** 2)
        sq_pt.append((o_pt[b, h, rows] - o_ref) ** 2)
    r_mx = float(np.sqrt(np.mean(np.concatenate(sq_mx))))
    r_pt = float(np.sqrt(np.mean(np.concatenate(sq_pt))))
    say(f"mx sampled RMSE {r_mx:.3e}, per-tensor {r_pt:.3e}")
    assert r_mx <= FP8_RMSE and r_mx < r_pt
    _, lse_fq = fake_quant_attention_mx(q64[:1, :1], k64[:1, :1], v64[:1, :1], signs[:1], False)
    rows = sample_rows(N, seed=3)
    check_lse(lse_mx[0, 0, rows], lse_fq[0, 0, rows])


def test_mx_causal_workload():
    """The fp8 outlier workload at full size with microscaling, causal, bf16
    output: every row of two whole heads against exact causal attention (the
    RMSE bound is over all elements; see the block-scaled causal test);
    against the oracle's own MX-quantised inputs (one head): RMSE over all
    rows, tile-boundary and random rows elementwise within the bound on the
    e4m3 rounding of P' (fp8_p_rounding_bound), LSE within 1e-3."""
    cfg = CONFIGS["fp8_b4h16n4k_d128"]
    B, H, N, d = cfg["B"], cfg["H"], cfg["N"], cfg["d"]
    say("mx causal workload")
    q, k, v = make_qkv(**cfg)
    signs = make_signs(H, d, cfg["seed"])
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    o, lse = mx_run(q, k, v, signs, True, out_f32=False)
    sq = []
    for b, h in ((0, 0), (B - 1, H - 1)):
        o_ref, _ = oracle.attention(q64[b:b + 1, h:h + 1], k64[b:b + 1, h:h + 1], v64[b:b + 1, h:h + 1],
                                    True)
        sq.append((o[b, h] - o_ref[0, 0]) ** 2)
    rmse = float(np.sqrt(np.mean(np.concatenate(sq))))
    say(f"mx causal RMSE over two heads {rmse:.3e}")
    assert rmse <= FP8_RMSE
    qc, qe = mx_quantize(q64[:1, :1], "d", signs[:1])
    kc, ke = mx_quantize(k64[:1, :1], "d", signs[:1])
    vc, ve = mx_quantize(v64[:1, :1], "n")
    qd, kd, vd = mx_dequantize(qc, qe, "d"), mx_dequantize(kc, ke, "d"), mx_dequantize(vc, ve, "n")
    o_fq, lse_fq = oracle.attention(qd, kd, vd, True)
    _, rmse_fq = errors(o[0, 0], o_fq[0, 0])
    say(f"mx causal RMSE vs fake-quant over a head {rmse_fq:.3e}")
    assert rmse_fq <= FP8_RMSE / 2, f"RMSE vs fake-quant {rmse_fq:.3e}"
    rows = sample_rows(N, seed=11)
    bound = fp8_p_rounding_bound(qd, kd, vd, 0, 0, rows, True)
    bound += half_ulp(np.abs(o_fq[0, 0, rows]) + bound, "bf16") + 1e-6
    err = np.abs(o[0, 0, rows] - o_fq[0, 0, rows])
    assert np.all(err <= bound), f"worst excess {np.max(err - bound):.3e}"
    check_lse(lse[0, 0, rows], lse_fq[0, 0, rows])
