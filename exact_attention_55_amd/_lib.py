"""ctypes binding for libfa.so (argument marshalling only).

Every step of the attention path runs in the library's HIP kernels; this file
only turns torch tensors into device pointers, picks the current HIP stream,
and maps status codes to exceptions. If the library is missing the calls
raise: there is no CPU fallback.
"""

import ctypes
import math
import os

import torch

FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE = 0, 1, 2, 3, 4
FA_NOALLOC_SCRATCH_BYTES = 16 << 20
FA_F16, FA_BF16, FA_FP8_E4M3, FA_FP8_MX = 0, 1, 2, 3
FA_MX_ALONG_D, FA_MX_ALONG_N = 0, 1
FA_OUT_F32 = 0x100
FA_SCALE_POW2 = 0x200
FA_FWD_PIPELINED = 0x400
FA_FP8_QSCALED = 0x800
FA_ROPE_NONE, FA_ROPE_INTERLEAVED, FA_ROPE_HALF = 0, 1, 2
ROPE_STYLES = {"interleaved": FA_ROPE_INTERLEAVED, "half": FA_ROPE_HALF}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class FaError(RuntimeError):
    def __init__(self, status, what):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


def lib_path():
    """The library this process loads: libfa.so beside this file, or the
    build FA_LIB names (an ablation variant from build.py --variant)."""
    return os.environ.get("FA_LIB") or os.path.join(_HERE, "libfa.so")


def lib():
    """Load the library once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = lib_path()
    if not os.path.exists(path):
        raise FaError(FA_ERR_HIP, f"{path} not built (run __graft_entry__.build())")
    L = ctypes.CDLL(path)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.fa_fwd.restype = i
    L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, i, vp]
    L.fa_bwd.restype = i
    L.fa_fwd_decode.argtypes = [vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t,
                                i, i, i, i, i, i, i, f, i, i, vp]
    L.fa_fwd_decode.restype = i
    L.fa_fwd_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, i, i, vp]
    L.fa_fwd_decode_noalloc.restype = i
    L.fa_decode_splits.argtypes = [i, i, i, i, i, i]
    L.fa_decode_splits.restype = i
    L.fa_decode_workspace_bytes.argtypes = [i, i, i, i, i]
    L.fa_decode_workspace_bytes.restype = ctypes.c_size_t
    L.fa_fp8_prep.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    L.fa_mx_prep.argtypes = [vp, vp, vp, i, i, i, i, i, i, vp]
    L.fa_mx_prep.restype = i
    L.fa_mx_packed_bytes.argtypes = [i, i, i, i]
    L.fa_mx_packed_bytes.restype = ctypes.c_size_t
    L.fa_fp8_prep_rope.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, i, vp]
    L.fa_fp8_prep_rope.restype = i
    L.fa_fp8_prep_scaled.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, f, i, f, vp]
    L.fa_fp8_prep_scaled.restype = i
    L.fa_mx_prep_scaled.argtypes = [vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.fa_mx_prep_scaled.restype = i
    L.fa_fp8_prep_qkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    L.fa_fp8_prep_qkv.restype = i
    L.fa_mx_prep_qkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
    L.fa_mx_prep_qkv.restype = i
    L.fa_fp8_prep.restype = i
    L.fa_fp8_packed_bytes.argtypes = [i, i, i, i]
    L.fa_fp8_packed_bytes.restype = ctypes.c_size_t
    L.fa_fp8_scales_offset.argtypes = [i, i, i, i]
    L.fa_fp8_scales_offset.restype = ctypes.c_size_t
    L.fa_status_string.argtypes = [i]
    L.fa_status_string.restype = ctypes.c_char_p
    _LIB = L
    return L


def status_string(status):
    if _LIB is not None:
        return _LIB.fa_status_string(int(status)).decode()
    return {0: "ok", 1: "invalid argument", 2: "unsupported configuration",
            3: "HIP runtime error"}.get(status, "unknown status")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device):
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def fwd_raw(q, k, v, o, lse, B, H, N, d, causal, softmax_scale, dtype, stream=None):
    """Direct call with integer pointers; returns the status code."""
    return lib().fa_fwd(q, k, v, o, lse, B, H, N, d, int(causal), float(softmax_scale),
                        int(dtype), stream)


def bwd_raw(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, causal, softmax_scale, dtype,
            stream=None):
    """Direct call with integer pointers; returns the status code."""
    return lib().fa_bwd(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, N, d, int(causal),
                        float(softmax_scale), int(dtype), stream)


def decode_raw(q, k, v, o, lse, seqlens_k, workspace, workspace_bytes, B, H, H_kv, Nq, Nk, d,
               causal, softmax_scale, num_splits, dtype, stream=None):
    """Direct call with integer pointers; returns the status code."""
    return lib().fa_fwd_decode(q, k, v, o, lse, seqlens_k, workspace, workspace_bytes, B, H, H_kv,
                               Nq, Nk, d, int(causal), float(softmax_scale), int(num_splits),
                               int(dtype), stream)


def decode_noalloc_raw(q, k, v, o, lse, seqlens_k, B, H, H_kv, Nq, Nk, d, causal, softmax_scale,
                       num_splits, dtype, stream=None):
    """Direct call of the allocation-free decode entry point; returns the
    status code."""
    return lib().fa_fwd_decode_noalloc(q, k, v, o, lse, seqlens_k, B, H, H_kv, Nq, Nk, d,
                                       int(causal), float(softmax_scale), int(num_splits),
                                       int(dtype), stream)


def decode_splits(B, H, H_kv, Nq, Nk, d):
    return int(lib().fa_decode_splits(B, H, H_kv, Nq, Nk, d))


def decode_workspace_bytes(B, H, Nq, d, num_splits):
    return int(lib().fa_decode_workspace_bytes(B, H, Nq, d, num_splits))


def fp8_prep_raw(x, x8, signs, B, H, N, d, block_rows, in_dtype, stream=None):
    return lib().fa_fp8_prep(x, x8, signs, B, H, N, d, block_rows, in_dtype, stream)


def fp8_prep_rope_raw(x, x8, signs, B, H, N, d, block_rows, in_dtype, rope_style, rope_base, pos0,
                      stream=None):
    return lib().fa_fp8_prep_rope(x, x8, signs, B, H, N, d, block_rows, in_dtype, int(rope_style),
                                  float(rope_base), int(pos0), stream)


def fp8_prep_scaled_raw(x, x8, signs, B, H, N, d, block_rows, in_dtype, rope_style, rope_base,
                        pos0, prescale, stream=None):
    return lib().fa_fp8_prep_scaled(x, x8, signs, B, H, N, d, block_rows, in_dtype,
                                    int(rope_style), float(rope_base), int(pos0), float(prescale),
                                    stream)


def fp8_prep_qkv_raw(q, k, v, q8, k8, v8, signs, B, H, N, d, in_dtype, q_prescale, stream=None):
    return lib().fa_fp8_prep_qkv(q, k, v, q8, k8, v8, signs, B, H, N, d, in_dtype,
                                 float(q_prescale), stream)


def mx_prep_qkv_raw(q, k, v, q8, k8, v8, signs, B, H, N, d, in_dtype, q_prescale, stream=None):
    return lib().fa_mx_prep_qkv(q, k, v, q8, k8, v8, signs, B, H, N, d, in_dtype,
                                float(q_prescale), stream)


def mx_prep_raw(x, x8, signs, B, H, N, d, axis, in_dtype, stream=None):
    return lib().fa_mx_prep(x, x8, signs, B, H, N, d, int(axis), in_dtype, stream)


def mx_prep_scaled_raw(x, x8, signs, B, H, N, d, axis, in_dtype, prescale, stream=None):
    return lib().fa_mx_prep_scaled(x, x8, signs, B, H, N, d, int(axis), in_dtype,
                                   float(prescale), stream)


def qk_prescale(softmax_scale):
    """The prescale that makes a prepared q carry softmax_scale * log2(e)
    (for fwd_fp8(..., qscaled=True))."""
    return softmax_scale * math.log2(math.e)


def mx_packed_bytes(B, H, N, d):
    return int(lib().fa_mx_packed_bytes(B, H, N, d))


def fp8_packed_bytes(B, H, N, d):
    return int(lib().fa_fp8_packed_bytes(B, H, N, d))


def _check(cond, what):
    if not cond:
        raise FaError(FA_ERR_INVALID_ARG, what)


def _check_device(*ts):
    dev = ts[0].device
    _check(dev.type == "cuda", "tensors must be on a HIP device")
    for t in ts:
        _check(t.device == dev, "tensors on different devices")
        _check(t.is_contiguous(), "tensors must be contiguous")


def _dtype_code(t):
    if t.dtype == torch.bfloat16:
        return FA_BF16
    if t.dtype == torch.float16:
        return FA_F16
    raise FaError(FA_ERR_UNSUPPORTED, f"dtype {t.dtype}")


def fwd(q, k, v, causal=False, softmax_scale=None, out=None, lse=None, out_f32=False,
        pipelined=False):
    """Attention forward on 16-bit [B,H,N,d] device tensors.

    Returns (o, lse): o has q's dtype (float32 with out_f32=True), lse is
    float32 [B,H,N]. pipelined: at d = 128, run the 64-rows-per-wave kernel
    with the in-wave pipeline instead of the default one (non-causal
    forwards with N >= 8192 run it without the flag).
    """
    B, H, N, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    odt = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    if out_f32:
        code |= FA_OUT_F32
    if pipelined:
        code |= FA_FWD_PIPELINED
    _check(q.dim() == 4 and k.shape == q.shape and v.shape == q.shape, "q, k, v shapes differ")
    _check(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v dtypes differ")
    _check(out.shape == q.shape and out.dtype == odt, "bad output tensor")
    _check(lse.shape == (B, H, N) and lse.dtype == torch.float32, "bad lse tensor")
    _check_device(q, k, v, out, lse)
    st = fwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, causal,
                 softmax_scale, code, _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd")
    return out, lse


def bwd(q, k, v, o, lse, dout, causal=False, softmax_scale=None, out_f32=False, grads=None,
        delta=None):
    """Gradients (dq, dk, dv) of the forward on 16-bit [B,H,N,d] device tensors.

    o and lse are the forward's outputs; dout is dL/do. The gradients have
    q's dtype (float32 with out_f32=True). delta is the float32 [2,B,H,N]
    scratch of per-row constants the call overwrites (allocated when not
    given).
    """
    B, H, N, d = q.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    code = _dtype_code(q)
    gdt = torch.float32 if out_f32 else q.dtype
    if grads is None:
        grads = tuple(torch.empty((B, H, N, d), dtype=gdt, device=q.device) for _ in range(3))
    dq, dk, dv = grads
    if delta is None:
        delta = torch.empty((2, B, H, N), dtype=torch.float32, device=q.device)
    if out_f32:
        code |= FA_OUT_F32
    _check(q.dim() == 4 and all(t.shape == q.shape for t in (k, v, o, dout)), "shapes differ")
    _check(all(t.dtype == q.dtype for t in (k, v, o, dout)), "dtypes differ")
    _check(all(t.shape == q.shape and t.dtype == gdt for t in grads), "bad gradient tensors")
    _check(lse.shape == (B, H, N) and lse.dtype == torch.float32, "bad lse tensor")
    _check(delta.shape == (2, B, H, N) and delta.dtype == torch.float32, "bad delta tensor")
    _check_device(q, k, v, o, lse, dout, dq, dk, dv, delta)
    st = bwd_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                 _ptr(dv), _ptr(delta), B, H, N, d, causal, softmax_scale, code, _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_bwd")
    return dq, dk, dv


def fwd_decode(q, k, v, causal=False, softmax_scale=None, seqlens_k=None, num_splits=0,
               out=None, lse=None, out_f32=False, workspace=None):
    """Decode-shaped forward: q [B,H,Nq,d] against k, v [B,H_kv,Nk,d] (16-bit
    device tensors, H a multiple of H_kv).

    seqlens_k: optional int32 [B] device tensor of keys per sequence.
    num_splits: 0 picks the library's suggestion. workspace: optional uint8
    device tensor of at least decode_workspace_bytes(...) bytes (allocated
    when needed and not given). Returns (o, lse): o [B,H,Nq,d] in q's dtype
    (float32 with out_f32=True), lse float32 [B,H,Nq].
    """
    B, H, Nq, d = q.shape
    _check(k.dim() == 4 and k.shape == v.shape, "k, v shapes differ")
    Bk, H_kv, Nk, dk = k.shape
    _check(Bk == B and dk == d, "k, v must be [B, H_kv, Nk, d]")
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    if num_splits == 0:
        num_splits = decode_splits(B, H, H_kv, Nq, Nk, d)
    code = _dtype_code(q)
    odt = torch.float32 if out_f32 else q.dtype
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=odt, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if out_f32:
        code |= FA_OUT_F32
    need = decode_workspace_bytes(B, H, Nq, d, num_splits)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _check(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v dtypes differ")
    _check(out.shape == (B, H, Nq, d) and out.dtype == odt, "bad output tensor")
    _check(lse.shape == (B, H, Nq) and lse.dtype == torch.float32, "bad lse tensor")
    extra = []
    if seqlens_k is not None:
        _check(seqlens_k.dtype == torch.int32 and tuple(seqlens_k.shape) == (B,), "seqlens_k must be int32 [B]")
        extra.append(seqlens_k)
    if workspace is not None:
        _check(workspace.dtype == torch.uint8, "workspace must be uint8")
        extra.append(workspace)
    _check_device(q, k, v, out, lse, *extra)
    wbytes = 0 if workspace is None else workspace.numel()
    st = decode_raw(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(seqlens_k), _ptr(workspace),
                    wbytes, B, H, H_kv, Nq, Nk, d, causal, softmax_scale, num_splits, code,
                    _stream(q.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd_decode")
    return out, lse


def fp8_alloc_packed(B, H, N, d, device):
    return torch.empty(fp8_packed_bytes(B, H, N, d), dtype=torch.uint8, device=device)


def fp8_codes_view(packed, B, H, N, d):
    """The e4m3 codes of a packed fp8 tensor, uint8 [B,H,N,d]."""
    return packed[: B * H * N * d].view(B, H, N, d)


def fp8_scales_view(packed, B, H, N, d):
    """The float32 block scales of a packed fp8 tensor, [B,H,ceil(N/128)]."""
    off = int(lib().fa_fp8_scales_offset(B, H, N, d))
    nb = (N + 127) // 128
    return packed[off: off + 4 * B * H * nb].view(torch.float32).view(B, H, nb)


def _prep_qkv(raw, packed_bytes, name, q, k, v, signs, q_prescale, out):
    B, H, N, d = q.shape
    _check(q.dim() == 4 and k.shape == q.shape and v.shape == q.shape, "q, k, v shapes differ")
    _check(k.dtype == q.dtype and v.dtype == q.dtype, "q, k, v dtypes differ")
    nbytes = packed_bytes(B, H, N, d)
    if out is None:
        out = tuple(torch.empty(nbytes, dtype=torch.uint8, device=q.device) for _ in range(3))
    _check(len(out) == 3, "out must hold three packed tensors")
    for o in out:
        _check(o.dtype == torch.uint8 and o.numel() >= nbytes, "packed output too small")
    if signs is not None:
        _check(signs.dtype == torch.int8 and tuple(signs.shape) == (H, d), "signs must be int8 [H, d]")
        _check_device(q, k, v, *out, signs)
    else:
        _check_device(q, k, v, *out)
    st = raw(_ptr(q), _ptr(k), _ptr(v), _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), _ptr(signs),
             B, H, N, d, _dtype_code(q), q_prescale, _stream(q.device))
    if st != FA_OK:
        raise FaError(st, name)
    return tuple(out)


def fp8_prep_qkv(q, k, v, signs=None, q_prescale=1.0, out=None):
    """The three fp8 preps of one attention call in a single launch: q and k
    rotated by signs (when given), q times q_prescale, v plain, all with
    128-row blocks and power-of-two scales. Returns (q8, k8, v8), packed
    uint8 tensors equal to those of fp8_prep(q, signs, prescale=q_prescale),
    fp8_prep(k, signs, pow2_scale=True) and fp8_prep(v, pow2_scale=True); out
    may hold three such tensors to write into. With q_prescale =
    qk_prescale(softmax_scale) they feed fwd_fp8(..., qscaled=True)."""
    return _prep_qkv(fp8_prep_qkv_raw, fp8_packed_bytes, "fa_fp8_prep_qkv", q, k, v, signs,
                     q_prescale, out)


def mx_prep_qkv(q, k, v, signs=None, q_prescale=1.0, out=None):
    """The three microscaled preps of one attention call in a single launch:
    q and k along d, rotated by signs (when given), q times q_prescale; v
    along the sequence. Returns (q8, k8, v8) equal to mx_prep(q, signs, "d",
    prescale=q_prescale), mx_prep(k, signs, "d") and mx_prep(v, None, "n");
    with q_prescale = qk_prescale(softmax_scale) they feed fwd_fp8(...,
    mx=True, qscaled=True)."""
    return _prep_qkv(mx_prep_qkv_raw, mx_packed_bytes, "fa_mx_prep_qkv", q, k, v, signs,
                     q_prescale, out)


def fp8_prep(x, signs=None, block_rows=128, out=None, rope=None, pow2_scale=False, prescale=None):
    """Random-sign Hadamard (when signs is given) + fp8 e4m3 block quantisation.

    x: 16-bit [B,H,N,d] device tensor; signs: int8 [H,d] device tensor of +-1
    or None; block_rows: 128, or 0 for one scale per tensor; rope: None, or
    (style, base, pos0) with style "interleaved" or "half" to apply the
    rotary embedding first, in the same pass; pow2_scale: round the scales up
    to powers of two (the form fwd_fp8 applies exactly for V); prescale:
    None, or a factor the values are multiplied by before quantisation (then
    the scales are always powers of two; q for fwd_fp8(..., qscaled=True)
    takes qk_prescale(softmax_scale)). Returns the packed uint8 tensor
    (codes then float32 scales) that fwd_fp8 consumes.
    """
    B, H, N, d = x.shape
    if out is None:
        out = fp8_alloc_packed(B, H, N, d, x.device)
    _check(out.dtype == torch.uint8 and out.numel() >= fp8_packed_bytes(B, H, N, d),
           "packed output too small")
    if signs is not None:
        _check(signs.dtype == torch.int8 and tuple(signs.shape) == (H, d), "signs must be int8 [H, d]")
        _check_device(x, out, signs)
    else:
        _check_device(x, out)
    code = _dtype_code(x) | (FA_SCALE_POW2 if pow2_scale else 0)
    if prescale is not None:
        style, base, pos0 = rope if rope is not None else (None, 1.0, 0)
        _check(style is None or style in ROPE_STYLES, f"rope style must be one of {sorted(ROPE_STYLES)}")
        st = fp8_prep_scaled_raw(_ptr(x), _ptr(out), _ptr(signs), B, H, N, d, block_rows, code,
                                 ROPE_STYLES[style] if style else 0, base, pos0, prescale,
                                 _stream(x.device))
    elif rope is None:
        st = fp8_prep_raw(_ptr(x), _ptr(out), _ptr(signs), B, H, N, d, block_rows,
                          code, _stream(x.device))
    else:
        style, base, pos0 = rope
        _check(style in ROPE_STYLES, f"rope style must be one of {sorted(ROPE_STYLES)}")
        st = fp8_prep_rope_raw(_ptr(x), _ptr(out), _ptr(signs), B, H, N, d, block_rows,
                               code, ROPE_STYLES[style], base, pos0, _stream(x.device))
    if st != FA_OK:
        raise FaError(st, "fa_fp8_prep")
    return out


def mx_prep(x, signs=None, axis="d", out=None, prescale=None):
    """fp8 e4m3 quantisation with a power-of-two scale per 32 elements,
    along d (axis "d": Q and K, optionally after the random-sign Hadamard)
    or along the sequence (axis "n": V). prescale (axis "d" only): None, or
    a factor the values are multiplied by first (q for fwd_fp8(...,
    mx=True, qscaled=True) takes qk_prescale(softmax_scale)). Returns the
    packed uint8 tensor (codes, then E8M0 scale bytes) that
    fwd_fp8(..., mx=True) consumes."""
    B, H, N, d = x.shape
    _check(axis in ("d", "n"), "axis must be 'd' or 'n'")
    if out is None:
        out = torch.empty(mx_packed_bytes(B, H, N, d), dtype=torch.uint8, device=x.device)
    _check(out.dtype == torch.uint8 and out.numel() >= mx_packed_bytes(B, H, N, d),
           "packed output too small")
    if signs is not None:
        _check(signs.dtype == torch.int8 and tuple(signs.shape) == (H, d), "signs must be int8 [H, d]")
        _check_device(x, out, signs)
    else:
        _check_device(x, out)
    ax = FA_MX_ALONG_D if axis == "d" else FA_MX_ALONG_N
    if prescale is not None:
        st = mx_prep_scaled_raw(_ptr(x), _ptr(out), _ptr(signs), B, H, N, d, ax, _dtype_code(x),
                                prescale, _stream(x.device))
    else:
        st = mx_prep_raw(_ptr(x), _ptr(out), _ptr(signs), B, H, N, d, ax, _dtype_code(x),
                         _stream(x.device))
    if st != FA_OK:
        raise FaError(st, "fa_mx_prep")
    return out


def mx_scales_view(packed, B, H, N, d, axis):
    """E8M0 scale bytes of a packed microscaled tensor: [B,H,N,d/32] for
    axis "d"; [B,H,ceil(N/32),32,d/32] for axis "n" (column c of a 32-row
    block at [c % 32, c // 32])."""
    off = int(lib().fa_fp8_scales_offset(B, H, N, d))
    if axis == "d":
        n = B * H * N * (d // 32)
        return packed[off: off + n].view(B, H, N, d // 32)
    nb = (N + 31) // 32
    return packed[off: off + B * H * nb * d].view(B, H, nb, 32, d // 32)


def fwd_fp8(q8, k8, v8, B, H, N, d, causal=False, softmax_scale=None, out_f32=False,
            out=None, lse=None, mx=False, qscaled=False):
    """Attention forward on packed fp8 tensors made by fp8_prep (mx=False)
    or by mx_prep (mx=True: q and k along d, v along n). qscaled: q was
    prepared with prescale=qk_prescale(softmax_scale) (block-scaled inputs:
    k and v with power-of-two scales too), so the logits need no multiply.

    Returns (o, lse) with o bf16 (float32 with out_f32=True).
    """
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(d)
    odt = torch.float32 if out_f32 else torch.bfloat16
    if out is None:
        out = torch.empty((B, H, N, d), dtype=odt, device=q8.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q8.device)
    code = ((FA_FP8_MX if mx else FA_FP8_E4M3) | (FA_OUT_F32 if out_f32 else 0)
            | (FA_FP8_QSCALED if qscaled else 0))
    need = mx_packed_bytes(B, H, N, d) if mx else fp8_packed_bytes(B, H, N, d)
    for t in (q8, k8, v8):
        _check(t.dtype == torch.uint8 and t.numel() >= need, "packed fp8 input too small")
    _check(out.shape == (B, H, N, d) and out.dtype == odt, "bad output tensor")
    _check(lse.shape == (B, H, N) and lse.dtype == torch.float32, "bad lse tensor")
    _check_device(q8, k8, v8, out, lse)
    st = fwd_raw(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(out), _ptr(lse), B, H, N, d, causal,
                 softmax_scale, code, _stream(q8.device))
    if st != FA_OK:
        raise FaError(st, "fa_fwd(fp8)")
    return out, lse
