"""The allocation-free decode entry point (fa_fwd_decode_noalloc, C ABI)
against the ordinary one (fa_fwd_decode with a caller workspace): both run
the same kernels with the same split count, so the outputs must be bitwise
equal. Two calls in a row, the second on a smaller problem, so the second
reads the fixed scratch after the first left its partials there; plus one
call with a single split (no scratch) and the host-side rejection of a
request that does not fit the scratch."""

import sys

import numpy as np
import pytest
import torch

import exact_attention_55_amd as fa
from exact_attention_55_amd.inputs import make_decode

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def both(B, H, Hkv, Nq, Nk, d, causal, lens, splits, seed):
    q, k, v, _ = make_decode(B, H, Hkv, Nq, Nk, d, seed, "bf16")
    qd, kd, vd = (t.to(DEV) for t in (q, k, v))
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device=DEV)
    code = fa.FA_BF16 | fa.FA_OUT_F32
    scale = 1.0 / np.sqrt(d)
    ws_bytes = fa.decode_workspace_bytes(B, H, Nq, d, splits)
    assert ws_bytes <= fa.FA_NOALLOC_SCRATCH_BYTES
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=DEV)
    o_ref = torch.empty((B, H, Nq, d), dtype=torch.float32, device=DEV)
    l_ref = torch.empty((B, H, Nq), dtype=torch.float32, device=DEV)
    o_na = torch.full((B, H, Nq, d), float("nan"), dtype=torch.float32, device=DEV)
    l_na = torch.full((B, H, Nq), float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream().cuda_stream
    slp = 0 if sl is None else sl.data_ptr()
    r = fa.decode_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_ref.data_ptr(), l_ref.data_ptr(),
                      slp or None, ws.data_ptr() if ws_bytes else None, ws_bytes, B, H, Hkv, Nq, Nk,
                      d, causal, scale, splits, code, st)
    assert r == fa.FA_OK, fa.status_string(r)
    r = fa.decode_noalloc_raw(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_na.data_ptr(),
                              l_na.data_ptr(), slp or None, B, H, Hkv, Nq, Nk, d, causal, scale,
                              splits, code, st)
    assert r == fa.FA_OK, fa.status_string(r)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ref), "O differs from fa_fwd_decode"
    assert torch.equal(l_na, l_ref), "LSE differs from fa_fwd_decode"


def test_noalloc_matches_workspace_entry_point():
    say("noalloc decode: large call (B=16 H=64 Hkv=8 Nk=4096, 8 splits)")
    both(16, 64, 8, 1, 4096, 128, True, [4096, 3000, 17, 0] * 4, 8, seed=31)
    say("noalloc decode: smaller call after it (B=2 H=8 Hkv=2 Nq=3 Nk=700, 3 splits)")
    both(2, 8, 2, 3, 700, 64, True, [700, 5], 3, seed=32)
    say("noalloc decode: one split (no scratch)")
    both(2, 4, 4, 1, 300, 256, False, None, 1, seed=33)


def test_noalloc_rejects_oversize():
    # partials of 4096 rows x 256 splits x (128 + 1) floats > 16 MiB: refused
    # on the host before any HIP call
    B, H, Nq, d, s = 64, 64, 1, 128, 256
    assert fa.decode_workspace_bytes(B, H, Nq, d, s) > fa.FA_NOALLOC_SCRATCH_BYTES
    F = 0x10000
    r = fa.decode_noalloc_raw(F, F, F, F, F, None, B, H, H, Nq, 8192, d, False, 0.1, s, fa.FA_BF16)
    assert r == fa.FA_ERR_TOO_LARGE
