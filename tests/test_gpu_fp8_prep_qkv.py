"""GPU parity of fa_fp8_prep_qkv and fa_mx_prep_qkv, the three fp8 preps
of one attention call in a single launch: q rotated by the random-sign
Hadamard and multiplied by its prescale, k rotated, v plain; block-scaled
(128-row blocks, power-of-two scales) or microscaled (q, k along d, v along
the sequence).

* every code and scale against the oracle's quantisers (fp8_quantize with
  power-of-two scales, mx_quantize; q with the prescale): bit-identical for
  v and without the rotation, adjacent and rare with it (the prep's float32
  butterflies);
* byte for byte what the three separate preps each one replaces write;
* the outlier workload B=4 H=16 N=4096 d=128, and the prescaled fp8
  forward on its outputs against exact attention.
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import exact_attention_55_amd as fa
from exact_attention_55_amd.inputs import CONFIGS, make_qkv, make_signs, to_f64

from helpers import FP8_RMSE, errors, sample_rows

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def views(packed, shape):
    B, H, N, d = shape
    return (fa.fp8_codes_view(packed, B, H, N, d).cpu().numpy(),
            fa.fp8_scales_view(packed, B, H, N, d).cpu().numpy())


def check_against_oracle(codes, scales, ref_codes, ref_scales, exact):
    """Codes and scales equal; with the rotation, codes may sit one e4m3 step
    apart on at most 1e-3 of the elements."""
    if exact:
        np.testing.assert_array_equal(scales, ref_scales)
        np.testing.assert_array_equal(codes, ref_codes)
        return
    np.testing.assert_allclose(scales, ref_scales, rtol=2e-6, atol=0)
    diff = codes != ref_codes
    assert diff.mean() <= 1e-3, f"{diff.mean():.2e} of codes differ"
    if diff.any():
        a = oracle.e4m3_decode(codes[diff])
        b = oracle.e4m3_decode(ref_codes[diff])
        mag = np.maximum(np.maximum(np.abs(a), np.abs(b)), 2.0 ** -6)
        assert np.all(np.abs(a - b) <= 2.0 ** (np.floor(np.log2(mag)) - 3))


SHAPES = [
    # B, H, N, d, dtype, rotation, prescaled
    (2, 3, 300, 64, "bf16", True, True),      # ragged last block
    (1, 2, 129, 128, "bf16", True, True),     # a one-row last block
    (2, 3, 300, 128, "fp16", True, False),
    (2, 3, 300, 128, "bf16", False, True),
    (1, 2, 1000, 256, "bf16", True, True),
    (3, 1, 1, 128, "bf16", True, True),       # one row per head
]


@pytest.mark.parametrize("B,H,N,d,dt,rot,scaled", SHAPES)
def test_prep_qkv_matches_oracle_and_separate_preps(B, H, N, d, dt, rot, scaled):
    say(f"prep qkv B={B} H={H} N={N} d={d} {dt} rotation={rot} prescaled={scaled}")
    q, k, v = make_qkv(B, H, N, d, seed=90 + N + d, dtype=dt, outliers=True)
    signs = make_signs(H, d, 90 + d) if rot else None
    sd = None if signs is None else torch.from_numpy(signs).to(DEV)
    p = fa.qk_prescale(1.0 / math.sqrt(d)) if scaled else 1.0
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    q8, k8, v8 = fa.fp8_prep_qkv(qd, kd, vd, sd, q_prescale=p)
    sep = (fa.fp8_prep(qd, sd, 128, prescale=p),
           fa.fp8_prep(kd, sd, 128, pow2_scale=True),
           fa.fp8_prep(vd, None, 128, pow2_scale=True))
    torch.cuda.synchronize()
    shape = (B, H, N, d)
    p32 = float(np.float32(p))
    for name, x, got, other, sg, ps in (("q", q, q8, sep[0], signs, p32), ("k", k, k8, sep[1], signs, None),
                                        ("v", v, v8, sep[2], None, None)):
        codes, scales = views(got, shape)
        c2, s2 = views(other, shape)
        np.testing.assert_array_equal(codes, c2, err_msg=f"{name} codes differ from the separate prep")
        np.testing.assert_array_equal(scales, s2, err_msg=f"{name} scales differ from the separate prep")
        rc, rs = oracle.fp8_quantize(to_f64(x), sg, 128, pow2=True, prescale=ps)
        check_against_oracle(codes, scales, rc, rs, exact=sg is None)
        assert np.all(np.frexp(scales)[0] == 0.5)


def test_prep_qkv_workload_and_forward():
    """The outlier workload: v every code against the oracle, q and k on
    two heads, all three byte for byte as the separate preps; then the
    prescaled forward on the outputs against exact attention (RMSE) on
    sampled rows of two heads."""
    c = CONFIGS["fp8_b4h16n4k_d128"]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    say(f"prep qkv workload B={B} H={H} N={N} d={d}")
    q, k, v = make_qkv(**c)
    signs = make_signs(H, d, c["seed"])
    sd = torch.from_numpy(signs).to(DEV)
    p = fa.qk_prescale(1.0 / math.sqrt(d))
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    q8, k8, v8 = fa.fp8_prep_qkv(qd, kd, vd, sd, q_prescale=p)
    sep = (fa.fp8_prep(qd, sd, 128, prescale=p),
           fa.fp8_prep(kd, sd, 128, pow2_scale=True),
           fa.fp8_prep(vd, None, 128, pow2_scale=True))
    o, lse = fa.fwd_fp8(q8, k8, v8, B, H, N, d, causal=False, out_f32=True, qscaled=True)
    torch.cuda.synchronize()
    shape = (B, H, N, d)
    for got, other in zip((q8, k8, v8), sep):
        for a, b in zip(views(got, shape), views(other, shape)):
            np.testing.assert_array_equal(a, b)
    codes, scales = views(v8, shape)
    rc, rs = oracle.fp8_quantize(to_f64(v), None, 128, pow2=True)
    check_against_oracle(codes, scales, rc, rs, exact=True)
    p32 = float(np.float32(p))
    for name, x, got, ps in (("q", q, q8, p32), ("k", k, k8, None)):
        codes, scales = views(got, shape)
        for h in (0, H - 1):
            rc, rs = oracle.fp8_quantize(to_f64(x[:1, h:h + 1]), signs[h:h + 1], 128, pow2=True,
                                         prescale=ps)
            check_against_oracle(codes[:1, h:h + 1], scales[:1, h:h + 1], rc, rs, exact=False)
    o = o.cpu().numpy()
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = sample_rows(N, seed=h)
        o_ref, _ = oracle.attention_rows(q64, k64, v64, b, h, rows, False)
        _, rmse = errors(o[b, h, rows], o_ref)
        say(f"prep qkv workload forward head {b},{h}: RMSE {rmse:.2e}")
        assert rmse <= FP8_RMSE


# ---- microscaled: fa_mx_prep_qkv (q, k along d; v along the sequence) ----

def mx_views(packed, shape, axis):
    """Codes [B,H,N,d] and block exponents ([B,H,N,d/32] along d,
    [B,H,ceil(N/32),d] along the sequence) of a packed microscaled tensor."""
    B, H, N, d = shape
    codes = packed[: B * H * N * d].view(B, H, N, d).cpu().numpy()
    sc = fa.mx_scales_view(packed, B, H, N, d, axis).cpu().numpy().astype(np.int32) - 127
    if axis == "n":   # [B,H,nb,32,d/32] -> [B,H,nb,d] with column c at [c % 32, c // 32]
        sc = sc.transpose(0, 1, 2, 4, 3).reshape(B, H, sc.shape[2], d)
    return codes, sc


def check_mx_against_oracle(codes, exps, ref_codes, ref_exps, axis, exact):
    """Exponents and codes equal; with the rotation, block exponents and
    codes may differ on at most 1e-3 of them, codes by one e4m3 step."""
    if exact:
        np.testing.assert_array_equal(exps, ref_exps)
        np.testing.assert_array_equal(codes, ref_codes)
        return
    bad = exps != ref_exps
    assert bad.mean() <= 1e-3, f"{bad.mean():.2e} of block exponents differ"
    same = np.repeat(~bad, 32, axis=-1) if axis == "d" else np.repeat(~bad, 32, axis=2)[:, :, :codes.shape[2]]
    diff = (codes != ref_codes) & same
    assert diff.mean() <= 1e-3, f"{diff.mean():.2e} of codes differ"
    if diff.any():
        a = oracle.e4m3_decode(codes[diff])
        b = oracle.e4m3_decode(ref_codes[diff])
        mag = np.maximum(np.maximum(np.abs(a), np.abs(b)), 2.0 ** -6)
        assert np.all(np.abs(a - b) <= 2.0 ** (np.floor(np.log2(mag)) - 3))


MX_SHAPES = [
    # B, H, N, d, dtype, rotation, prescaled
    (2, 3, 300, 64, "bf16", True, True),
    (1, 2, 257, 128, "fp16", True, False),
    (2, 3, 300, 128, "bf16", False, True),
    (2, 2, 96, 256, "bf16", True, True),
    (3, 1, 1, 128, "bf16", True, True),
]


@pytest.mark.parametrize("B,H,N,d,dt,rot,scaled", MX_SHAPES)
def test_mx_prep_qkv_matches_oracle_and_separate_preps(B, H, N, d, dt, rot, scaled):
    say(f"mx prep qkv B={B} H={H} N={N} d={d} {dt} rotation={rot} prescaled={scaled}")
    from oracle.mx import mx_quantize
    q, k, v = make_qkv(B, H, N, d, seed=95 + N + d, dtype=dt, outliers=True)
    if N > 64:
        v[0, 0, 32:64] = 0                      # an all-zero V block
    signs = make_signs(H, d, 95 + d) if rot else None
    sd = None if signs is None else torch.from_numpy(signs).to(DEV)
    p = fa.qk_prescale(1.0 / math.sqrt(d)) if scaled else 1.0
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    q8, k8, v8 = fa.mx_prep_qkv(qd, kd, vd, sd, q_prescale=p)
    sep = (fa.mx_prep(qd, sd, "d", prescale=p), fa.mx_prep(kd, sd, "d"), fa.mx_prep(vd, None, "n"))
    torch.cuda.synchronize()
    shape = (B, H, N, d)
    p32 = float(np.float32(p))
    for name, x, got, other, sg, ps, axis in (("q", q, q8, sep[0], signs, p32, "d"),
                                              ("k", k, k8, sep[1], signs, None, "d"),
                                              ("v", v, v8, sep[2], None, None, "n")):
        codes, exps = mx_views(got, shape, axis)
        c2, e2 = mx_views(other, shape, axis)
        np.testing.assert_array_equal(codes, c2, err_msg=f"{name} codes differ from the separate prep")
        np.testing.assert_array_equal(exps, e2, err_msg=f"{name} scales differ from the separate prep")
        rc, re = mx_quantize(to_f64(x), axis, sg, prescale=ps)
        check_mx_against_oracle(codes, exps, rc, re, axis, exact=sg is None)


def test_mx_prep_qkv_workload_and_forward():
    """The outlier workload through fa_mx_prep_qkv: byte for byte the three
    separate preps, v every code against the oracle, and the prescaled
    microscaled forward on the outputs against exact attention (RMSE) on
    sampled rows of two heads."""
    from oracle.mx import mx_quantize
    c = CONFIGS["fp8_b4h16n4k_d128"]
    B, H, N, d = c["B"], c["H"], c["N"], c["d"]
    say(f"mx prep qkv workload B={B} H={H} N={N} d={d}")
    q, k, v = make_qkv(**c)
    signs = make_signs(H, d, c["seed"])
    sd = torch.from_numpy(signs).to(DEV)
    p = fa.qk_prescale(1.0 / math.sqrt(d))
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    q8, k8, v8 = fa.mx_prep_qkv(qd, kd, vd, sd, q_prescale=p)
    sep = (fa.mx_prep(qd, sd, "d", prescale=p), fa.mx_prep(kd, sd, "d"), fa.mx_prep(vd, None, "n"))
    o, _ = fa.fwd_fp8(q8, k8, v8, B, H, N, d, causal=False, out_f32=True, mx=True, qscaled=True)
    torch.cuda.synchronize()
    shape = (B, H, N, d)
    for got, other, axis in zip((q8, k8, v8), sep, ("d", "d", "n")):
        for a, b in zip(mx_views(got, shape, axis), mx_views(other, shape, axis)):
            np.testing.assert_array_equal(a, b)
    codes, exps = mx_views(v8, shape, "n")
    rc, re = mx_quantize(to_f64(v), "n")
    check_mx_against_oracle(codes, exps, rc, re, "n", exact=True)
    o = o.cpu().numpy()
    q64, k64, v64 = to_f64(q), to_f64(k), to_f64(v)
    for b, h in ((0, 0), (B - 1, H - 1)):
        rows = sample_rows(N, seed=h)
        o_ref, _ = oracle.attention_rows(q64, k64, v64, b, h, rows, False)
        _, rmse = errors(o[b, h, rows], o_ref)
        say(f"mx prep qkv workload forward head {b},{h}: RMSE {rmse:.2e}")
        assert rmse <= FP8_RMSE
