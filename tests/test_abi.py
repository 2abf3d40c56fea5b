"""The C ABI on any host: the library loads, exports every symbol include/fa.h
declares, and rejects bad arguments with the documented status codes before
making any HIP call (so these run without a GPU)."""

import ctypes
import os
import re

import pytest

import exact_attention_55_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fa.lib_path()):
        pytest.fail("libfa.so is not built; run __graft_entry__.build()")
    return fa.lib()


def test_exports_every_declared_symbol(L):
    names = header_functions()
    assert {"fa_fwd", "fa_fp8_prep", "fa_fp8_packed_bytes", "fa_fp8_scales_offset",
            "fa_status_string"} <= set(names)
    for n in names:
        assert hasattr(L, n), f"{n} not exported"


def test_status_strings(L):
    for code in (0, 1, 2, 3, 4):
        assert fa.status_string(code) != "unknown status"
    assert L.fa_status_string(99).decode() == "unknown status"


def test_packed_sizes(L):
    B, H, N, d = 2, 3, 300, 128
    off = L.fa_fp8_scales_offset(B, H, N, d)
    assert off % 256 == 0 and off >= B * H * N * d
    size = L.fa_fp8_packed_bytes(B, H, N, d)
    assert size % 256 == 0 and size >= off + 4 * B * H * 3
    assert L.fa_fp8_packed_bytes(-1, 1, 1, 64) == 0


FAKE = 0x10000   # aligned non-null fake device pointer; never dereferenced


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, B=1, H=1, N=128, d=128, causal=0,
             scale=0.088, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.fwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["H"], a["N"], a["d"],
                      a["causal"], a["scale"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=7), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_BF16 | 0x200), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_BF16 | fa.FA_FWD_PIPELINED | 0x800), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    # one head's K/V past 2^31 - 2^16 - 1 bytes (31-bit buffer offsets)
    (dict(N=8388352, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 23, d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(N=-1), fa.FA_ERR_INVALID_ARG),
    (dict(B=-2), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(lse=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=FAKE + 8), fa.FA_ERR_INVALID_ARG),
    (dict(k=FAKE + 2), fa.FA_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_FP8_E4M3, q=FAKE + 16), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
    (dict(N=0, q=None), fa.FA_OK),
])
def test_fwd_validation(L, kw, status):
    assert fwd(**kw) == status


def prep(**kw):
    a = dict(x=FAKE, x8=FAKE, signs=None, B=1, H=1, N=128, d=128, block_rows=128,
             in_dtype=fa.FA_BF16)
    a.update(kw)
    return fa.fp8_prep_raw(a["x"], a["x8"], a["signs"], a["B"], a["H"], a["N"], a["d"],
                           a["block_rows"], a["in_dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_FP8_E4M3 | fa.FA_SCALE_POW2), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_BF16 | fa.FA_SCALE_POW2, block_rows=64), fa.FA_ERR_UNSUPPORTED),
    (dict(in_dtype=fa.FA_BF16 | fa.FA_OUT_F32), fa.FA_ERR_INVALID_ARG),
    (dict(block_rows=64), fa.FA_ERR_UNSUPPORTED),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(N=-5), fa.FA_ERR_INVALID_ARG),
    (dict(x=None), fa.FA_ERR_INVALID_ARG),
    (dict(x8=FAKE + 16), fa.FA_ERR_INVALID_ARG),
    (dict(x=FAKE + 4), fa.FA_ERR_INVALID_ARG),
    (dict(H=0), fa.FA_OK),
])
def test_prep_validation(L, kw, status):
    assert prep(**kw) == status


def test_binding_raises_without_library(monkeypatch, tmp_path):
    """The binding never falls back to CPU code: a missing library is an error."""
    from exact_attention_55_amd import _lib
    monkeypatch.setattr(_lib, "_LIB", None)
    monkeypatch.setattr(_lib, "lib_path", lambda: str(tmp_path / "missing.so"))
    with pytest.raises(fa.FaError):
        _lib.lib()


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, do=FAKE, dq=FAKE, dk=FAKE, dv=FAKE,
             delta=FAKE, B=1, H=1, N=128, d=128, causal=0, scale=0.088, dtype=fa.FA_BF16)
    a.update(kw)
    return fa.bwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                      a["delta"], a["B"], a["H"], a["N"], a["d"], a["causal"], a["scale"],
                      a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(dtype=fa.FA_BF16 | 0x400), fa.FA_ERR_INVALID_ARG),
    (dict(d=32), fa.FA_ERR_UNSUPPORTED),
    (dict(N=1 << 23, d=256), fa.FA_ERR_UNSUPPORTED),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=8388352, d=128), fa.FA_ERR_UNSUPPORTED),
    (dict(N=-1), fa.FA_ERR_INVALID_ARG),
    (dict(scale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(do=None), fa.FA_ERR_INVALID_ARG),
    (dict(delta=None), fa.FA_ERR_INVALID_ARG),
    (dict(dv=FAKE + 8), fa.FA_ERR_INVALID_ARG),
    (dict(delta=FAKE + 4), fa.FA_ERR_INVALID_ARG),
    (dict(lse=FAKE + 2), fa.FA_ERR_INVALID_ARG),
    (dict(H=0, q=None), fa.FA_OK),
])
def test_bwd_validation(L, kw, status):
    assert bwd(**kw) == status


def decode(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, o=FAKE, lse=FAKE, seqlens=None, ws=FAKE, ws_bytes=1 << 30,
             B=2, H=8, H_kv=2, Nq=1, Nk=4096, d=128, causal=0, scale=0.088, splits=4,
             dtype=fa.FA_BF16)
    a.update(kw)
    return fa.decode_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["seqlens"], a["ws"],
                         a["ws_bytes"], a["B"], a["H"], a["H_kv"], a["Nq"], a["Nk"], a["d"],
                         a["causal"], a["scale"], a["splits"], a["dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(H_kv=3), fa.FA_ERR_INVALID_ARG),          # H not a multiple of H_kv
    (dict(H_kv=0), fa.FA_ERR_INVALID_ARG),
    (dict(Nq=-1), fa.FA_ERR_INVALID_ARG),
    (dict(Nk=-1), fa.FA_ERR_INVALID_ARG),
    (dict(splits=0), fa.FA_ERR_INVALID_ARG),
    (dict(splits=257), fa.FA_ERR_INVALID_ARG),
    (dict(scale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(Nk=8388352), fa.FA_ERR_UNSUPPORTED),
    (dict(ws=None), fa.FA_ERR_INVALID_ARG),           # splits > 1 needs a workspace
    (dict(ws_bytes=1024), fa.FA_ERR_INVALID_ARG),     # too small
    (dict(ws=FAKE + 8), fa.FA_ERR_INVALID_ARG),
    (dict(seqlens=FAKE + 2), fa.FA_ERR_INVALID_ARG),
    (dict(k=None), fa.FA_ERR_INVALID_ARG),
    (dict(o=FAKE + 4), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
    (dict(Nq=0, q=None), fa.FA_OK),
])
def test_decode_validation(L, kw, status):
    assert decode(**kw) == status


def test_decode_sizes(L):
    # workspace: partial O (fp32) then partial LSE, each rounded to 256 bytes
    B, H, Nq, d, S = 2, 8, 3, 128, 5
    rows = B * H * Nq
    o_bytes = -(-rows * S * d * 4 // 256) * 256
    l_bytes = -(-rows * S * 4 // 256) * 256
    assert fa.decode_workspace_bytes(B, H, Nq, d, S) == o_bytes + l_bytes
    assert fa.decode_workspace_bytes(B, H, Nq, d, 1) == 0
    assert fa.decode_workspace_bytes(B, H, Nq, d, 300) == 0
    # suggested splits: at least 1, at most 64, and short histories are not split
    assert fa.decode_splits(8, 16, 16, 1, 16384, 128) > 1
    assert fa.decode_splits(8, 16, 16, 1, 200, 128) == 1
    assert 1 <= fa.decode_splits(1, 1, 1, 1, 1 << 20, 64) <= 64
    assert fa.decode_splits(1, 3, 2, 1, 100, 128) == 1


def prep_rope(**kw):
    a = dict(x=FAKE, x8=FAKE, signs=None, B=1, H=1, N=128, d=128, block_rows=128,
             in_dtype=fa.FA_BF16, style=fa.FA_ROPE_HALF, base=10000.0, pos0=0)
    a.update(kw)
    return fa.fp8_prep_rope_raw(a["x"], a["x8"], a["signs"], a["B"], a["H"], a["N"], a["d"],
                                a["block_rows"], a["in_dtype"], a["style"], a["base"], a["pos0"],
                                None)


@pytest.mark.parametrize("kw,status", [
    (dict(style=3), fa.FA_ERR_INVALID_ARG),
    (dict(style=-1), fa.FA_ERR_INVALID_ARG),
    (dict(base=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(base=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(pos0=-1), fa.FA_ERR_INVALID_ARG),
    (dict(pos0=(1 << 24) - 100), fa.FA_ERR_INVALID_ARG),     # positions past 2^24
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(block_rows=64), fa.FA_ERR_UNSUPPORTED),
    (dict(x8=FAKE + 16), fa.FA_ERR_INVALID_ARG),
    (dict(x=None), fa.FA_ERR_INVALID_ARG),
    (dict(N=0), fa.FA_OK),
    (dict(style=fa.FA_ROPE_NONE, base=0.0, pos0=-5, N=0), fa.FA_OK),   # no rotary: not checked
])
def test_prep_rope_validation(L, kw, status):
    assert prep_rope(**kw) == status


def mx(**kw):
    a = dict(x=FAKE, x8=FAKE, signs=None, B=1, H=1, N=128, d=128, axis=fa.FA_MX_ALONG_D,
             in_dtype=fa.FA_BF16)
    a.update(kw)
    return fa.mx_prep_raw(a["x"], a["x8"], a["signs"], a["B"], a["H"], a["N"], a["d"], a["axis"],
                          a["in_dtype"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(axis=2), fa.FA_ERR_INVALID_ARG),
    (dict(axis=fa.FA_MX_ALONG_N, signs=FAKE), fa.FA_ERR_INVALID_ARG),   # no Hadamard for V
    (dict(in_dtype=fa.FA_FP8_MX), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_BF16 | fa.FA_SCALE_POW2), fa.FA_ERR_INVALID_ARG),   # E8M0 scales already
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(N=-1), fa.FA_ERR_INVALID_ARG),
    (dict(x8=FAKE + 64), fa.FA_ERR_INVALID_ARG),
    (dict(x=None), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
])
def test_mx_prep_validation(L, kw, status):
    assert mx(**kw) == status


def test_mx_sizes_and_fwd_dtype(L):
    B, H, N, d = 2, 3, 100, 128
    off = L.fa_fp8_scales_offset(B, H, N, d)
    size = fa.mx_packed_bytes(B, H, N, d)
    assert size % 256 == 0
    assert size >= off + max(B * H * N * d // 32, B * H * 4 * d)
    assert fa.mx_packed_bytes(1, 1, 1, 80) == 0
    # the microscaled dtype is accepted by fa_fwd's validation (alignment 256)
    assert fwd(dtype=fa.FA_FP8_MX, q=FAKE + 16) == fa.FA_ERR_INVALID_ARG
    assert fwd(dtype=fa.FA_FP8_MX | 0x200) == fa.FA_ERR_INVALID_ARG
    assert fwd(dtype=fa.FA_FP8_MX, B=0) == fa.FA_OK


def prep_scaled(**kw):
    a = dict(x=FAKE, x8=FAKE, signs=None, B=1, H=1, N=128, d=128, block_rows=128,
             in_dtype=fa.FA_BF16, style=fa.FA_ROPE_NONE, base=10000.0, pos0=0, prescale=0.1275)
    a.update(kw)
    return fa.fp8_prep_scaled_raw(a["x"], a["x8"], a["signs"], a["B"], a["H"], a["N"], a["d"],
                                  a["block_rows"], a["in_dtype"], a["style"], a["base"], a["pos0"],
                                  a["prescale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(prescale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(prescale=-0.5), fa.FA_ERR_INVALID_ARG),
    (dict(prescale=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(prescale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(style=3), fa.FA_ERR_INVALID_ARG),
    (dict(style=fa.FA_ROPE_HALF, base=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(block_rows=64), fa.FA_ERR_UNSUPPORTED),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(x8=FAKE + 16), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_BF16 | fa.FA_SCALE_POW2, N=0), fa.FA_OK),
    (dict(style=fa.FA_ROPE_NONE, base=0.0, pos0=-5, N=0), fa.FA_OK),
])
def test_prep_scaled_validation(L, kw, status):
    assert prep_scaled(**kw) == status


def mx_scaled(**kw):
    a = dict(x=FAKE, x8=FAKE, signs=None, B=1, H=1, N=128, d=128, axis=fa.FA_MX_ALONG_D,
             in_dtype=fa.FA_BF16, prescale=0.1275)
    a.update(kw)
    return fa.mx_prep_scaled_raw(a["x"], a["x8"], a["signs"], a["B"], a["H"], a["N"], a["d"],
                                 a["axis"], a["in_dtype"], a["prescale"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(axis=fa.FA_MX_ALONG_N), fa.FA_ERR_INVALID_ARG),         # prescale defined along d only
    (dict(axis=fa.FA_MX_ALONG_N, prescale=1.0), fa.FA_ERR_INVALID_ARG),
    (dict(prescale=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(prescale=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(x8=FAKE + 64), fa.FA_ERR_INVALID_ARG),
    (dict(B=0), fa.FA_OK),
])
def test_mx_prep_scaled_validation(L, kw, status):
    assert mx_scaled(**kw) == status


def test_qscaled_flag_only_for_fp8(L):
    for base in (fa.FA_BF16, fa.FA_F16):
        assert fwd(dtype=base | fa.FA_FP8_QSCALED) == fa.FA_ERR_INVALID_ARG
    for base in (fa.FA_FP8_E4M3, fa.FA_FP8_MX):
        assert fwd(dtype=base | fa.FA_FP8_QSCALED, B=0) == fa.FA_OK
        assert fwd(dtype=base | fa.FA_FP8_QSCALED | fa.FA_OUT_F32, B=0) == fa.FA_OK
        assert fwd(dtype=base | fa.FA_FP8_QSCALED, q=FAKE + 16) == fa.FA_ERR_INVALID_ARG


P8 = 1 << 24   # spacing of the fake packed outputs: apart, they do not overlap


def prep_qkv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, q8=FAKE, k8=FAKE + P8, v8=FAKE + 2 * P8, signs=None, B=1, H=1,
             N=128, d=128, in_dtype=fa.FA_BF16, p=0.1275)
    a.update(kw)
    return fa.fp8_prep_qkv_raw(a["q"], a["k"], a["v"], a["q8"], a["k8"], a["v8"], a["signs"], a["B"],
                               a["H"], a["N"], a["d"], a["in_dtype"], a["p"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(p=-1.0), fa.FA_ERR_INVALID_ARG),
    (dict(p=float("inf")), fa.FA_ERR_INVALID_ARG),
    (dict(p=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_FP8_E4M3), fa.FA_ERR_INVALID_ARG),
    (dict(d=80), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 14, H=1 << 10, N=1 << 13), fa.FA_ERR_UNSUPPORTED),   # 3 x 2^30 workgroups
    (dict(q8=FAKE + 16), fa.FA_ERR_INVALID_ARG),
    (dict(k=FAKE + 4), fa.FA_ERR_INVALID_ARG),
    (dict(v=None), fa.FA_ERR_INVALID_ARG),
    (dict(v8=None), fa.FA_ERR_INVALID_ARG),
    (dict(k8=FAKE), fa.FA_ERR_INVALID_ARG),                 # k8 is q8
    (dict(v8=FAKE + P8 + 256), fa.FA_ERR_INVALID_ARG),      # v8 inside k8
    (dict(B=0, k8=FAKE), fa.FA_OK),
    (dict(N=0, in_dtype=fa.FA_F16 | fa.FA_SCALE_POW2), fa.FA_OK),
])
def test_prep_qkv_validation(L, kw, status):
    assert prep_qkv(**kw) == status


def mx_prep_qkv(**kw):
    a = dict(q=FAKE, k=FAKE, v=FAKE, q8=FAKE, k8=FAKE + P8, v8=FAKE + 2 * P8, signs=None, B=1, H=1,
             N=128, d=128, in_dtype=fa.FA_BF16, p=0.1275)
    a.update(kw)
    return fa.mx_prep_qkv_raw(a["q"], a["k"], a["v"], a["q8"], a["k8"], a["v8"], a["signs"], a["B"],
                              a["H"], a["N"], a["d"], a["in_dtype"], a["p"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(p=0.0), fa.FA_ERR_INVALID_ARG),
    (dict(p=float("nan")), fa.FA_ERR_INVALID_ARG),
    (dict(in_dtype=fa.FA_FP8_MX), fa.FA_ERR_INVALID_ARG),
    (dict(d=96), fa.FA_ERR_UNSUPPORTED),
    (dict(B=1 << 14, H=1 << 10, N=1 << 13), fa.FA_ERR_UNSUPPORTED),   # 2^32 V blocks
    (dict(q8=FAKE + 64), fa.FA_ERR_INVALID_ARG),
    (dict(v=FAKE + 2), fa.FA_ERR_INVALID_ARG),
    (dict(q=None), fa.FA_ERR_INVALID_ARG),
    (dict(v8=FAKE), fa.FA_ERR_INVALID_ARG),                 # v8 is q8
    (dict(k8=FAKE + 2 * P8 - 256), fa.FA_ERR_INVALID_ARG),  # k8 runs into v8
    (dict(H=0, v8=FAKE), fa.FA_OK),
])
def test_mx_prep_qkv_validation(L, kw, status):
    assert mx_prep_qkv(**kw) == status
