"""MI355X (gfx950) fused exact attention: forward pass, its gradients, and a
decode-shaped (split-key) forward.

The compute lives in ``libfa.so`` (hand-written HIP for gfx950 behind a C ABI
declared in ``include/fa.h``). This package is a thin ctypes binding: it passes
torch device pointers and the current HIP stream to the library and does no
arithmetic of its own.

    from exact_attention_55_amd import fwd, bwd, fwd_decode, fp8_prep
"""

from ._lib import (  # noqa: F401
    FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED, FA_ERR_HIP, FA_ERR_TOO_LARGE,
    FA_NOALLOC_SCRATCH_BYTES, decode_noalloc_raw,
    FA_F16, FA_BF16, FA_FP8_E4M3, FA_OUT_F32, FA_SCALE_POW2, FA_FWD_PIPELINED,
    FaError, lib, lib_path, fwd, fwd_raw, bwd, bwd_raw, fwd_fp8, fp8_prep, fp8_prep_raw, fp8_packed_bytes,
    fp8_alloc_packed, fp8_scales_view, fp8_codes_view, status_string,
    fwd_decode, decode_raw, decode_splits, decode_workspace_bytes,
    fp8_prep_rope_raw, FA_ROPE_NONE, FA_ROPE_INTERLEAVED, FA_ROPE_HALF,
    FA_FP8_MX, FA_MX_ALONG_D, FA_MX_ALONG_N, mx_prep, mx_prep_raw, mx_packed_bytes, mx_scales_view,
    FA_FP8_QSCALED, fp8_prep_scaled_raw, mx_prep_scaled_raw, qk_prescale,
    fp8_prep_qkv, fp8_prep_qkv_raw, mx_prep_qkv, mx_prep_qkv_raw,
)
