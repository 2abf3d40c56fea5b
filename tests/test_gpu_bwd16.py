"""GPU parity of the 16-bit backward (fa_bwd through the C ABI) against the
float64 gradient oracle on the same seeded, 16-bit-rounded inputs.

Tolerance (no bound is printed for gradients; derived from the arithmetic,
see the design notes): each gradient is one GEMM whose left factor the kernel
rounds to the 16-bit type (P for dV, dS for dQ and dK) while the right factor
(dO, K, Q) is an exact input. So elementwise
    |G - G_ref| <= u * (|X| |Y|) + (O-rounding term) + floor
with |X| |Y| the same product over absolute values (|P|^T |dO|,
scale |dS| |K|, scale |dS|^T |Q|), u = 2^-7 for bf16 and 2^-9 for fp16
(twice the unit roundoff of the rounded factor); the forward's O, stored in
16 bits, perturbs D = rowsum(dO * O) by at most u * rowsum(|dO| |O|), which
moves dQ and dK by that times P |K| and P^T |Q|; the floor
2e-5 * max |G_ref| covers fp32 accumulation, the hardware exp2 and fp16
subnormals. With 16-bit gradients half a unit in the last place of the
stored value is added. The RMSE, normalised by the gradient's RMS, is also
bounded (<= 4u).
"""

import math
import sys

import numpy as np
import pytest
import torch

import oracle
import exact_attention_55_amd as fa
from exact_attention_55_amd.inputs import make_dout, make_qkv, to_f64

from helpers import half_ulp

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
U = {"bf16": 2.0 ** -7, "fp16": 2.0 ** -9}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bounds(q, k, v, do, causal, scale, dtype):
    """Elementwise error bounds of the three gradient GEMMs (float64): u times
    the product over absolute values, plus the effect of the forward's O
    being stored in 16 bits (it enters through D = rowsum(dO * O))."""
    B, H, N, d = q.shape
    u = U[dtype]
    mq, mk, mv = (np.empty((B, H, N, d)) for _ in range(3))
    for b in range(B):
        for h in range(H):
            p = oracle.softmax_probs(q[b, h], k[b, h], causal, scale)
            o = p @ v[b, h]
            dp = do[b, h] @ v[b, h].T
            ds = np.abs(p * (dp - np.sum(p * dp, axis=1, keepdims=True)))
            dD = u * np.sum(np.abs(do[b, h]) * np.abs(o), axis=1)        # error of D per row
            mv[b, h] = u * (p.T @ np.abs(do[b, h]))
            mq[b, h] = scale * (u * (ds @ np.abs(k[b, h])) + dD[:, None] * (p @ np.abs(k[b, h])))
            mk[b, h] = scale * (u * (ds.T @ np.abs(q[b, h])) + p.T @ (dD[:, None] * np.abs(q[b, h])))
    return mq, mk, mv


def check_grad(g, g_ref, m, dtype, out_dtype, name):
    g = np.asarray(g, dtype=np.float64)
    assert np.all(np.isfinite(g)), f"non-finite {name}"
    err = np.abs(g - g_ref)
    bound = m + 2e-5 * np.max(np.abs(g_ref))
    if out_dtype != "f32":
        bound = bound + half_ulp(g_ref, out_dtype)
    worst = float(np.max(err / bound))
    assert worst <= 1.0, f"{name}: error reaches {worst:.2f} x the bound"
    # normalised by the RMS of the gradient, or of the magnitudes the bound is
    # built from when the gradient itself vanishes (e.g. dQ, dK for N = 1)
    scale = max(np.sqrt(np.mean(g_ref ** 2)), np.sqrt(np.mean(m ** 2)) / U[dtype], 1e-30)
    nrmse = float(np.sqrt(np.mean((g - g_ref) ** 2)) / scale)
    limit = 4 * U[dtype] + (2.0 ** -8 if out_dtype != "f32" else 0.0)
    assert nrmse <= limit, f"{name}: normalised RMSE {nrmse:.2e} > {limit:.2e}"
    return worst, nrmse


def run_case(B, H, N, d, causal, dtype, out_f32, seed=11, scale=None):
    q, k, v = make_qkv(B, H, N, d, seed=seed, dtype=dtype)
    do = make_dout(B, H, N, d, seed + 500, dtype)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=causal, softmax_scale=scale)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, softmax_scale=scale, out_f32=out_f32)
    torch.cuda.synchronize()
    # the reference is the exact gradient; the bound accounts for the
    # forward's O being rounded to 16 bits before it reaches D
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    dq_r, dk_r, dv_r = oracle.attention_backward(q64, k64, v64, do64, causal, scale)
    mq, mk, mv = bounds(q64, k64, v64, do64, causal, scale, dtype)
    od = "f32" if out_f32 else dtype
    res = {}
    for name, g, gr, m in (("dq", dq, dq_r, mq), ("dk", dk, dk_r, mk), ("dv", dv, dv_r, mv)):
        res[name] = check_grad(g.float().cpu().numpy(), gr, m, dtype, od,
                               f"{name} B{B} H{H} N{N} d{d} causal={causal} {dtype}")
    return res


SMALL = [
    # B, H, N, d, causal, dtype
    (1, 1, 1, 64, False, "bf16"),
    (1, 1, 1, 128, True, "fp16"),
    (1, 2, 33, 64, True, "bf16"),
    (2, 1, 64, 128, False, "bf16"),
    (1, 1, 65, 128, True, "bf16"),
    (1, 2, 200, 64, False, "fp16"),
    (1, 2, 200, 64, True, "bf16"),
    (2, 2, 257, 128, False, "bf16"),
    (1, 2, 300, 128, True, "fp16"),
    (1, 1, 513, 128, True, "bf16"),
    (1, 1, 640, 64, False, "bf16"),
    # d = 256: one wave per SIMD, gradients in the accumulation registers;
    # key tiles of 32 in the query-parallel kernel
    (1, 1, 1, 256, False, "bf16"),
    (1, 2, 65, 256, True, "bf16"),
    (1, 1, 200, 256, False, "fp16"),
    (2, 1, 257, 256, True, "bf16"),
    (1, 1, 513, 256, True, "fp16"),
    (1, 2, 300, 256, False, "bf16"),
]


@pytest.mark.parametrize("B,H,N,d,causal,dtype", SMALL)
@pytest.mark.parametrize("out_f32", [True, False])
def test_small_full_compare(B, H, N, d, causal, dtype, out_f32):
    say(f"bwd case B={B} H={H} N={N} d={d} causal={causal} {dtype} out_f32={out_f32}")
    res = run_case(B, H, N, d, causal, dtype, out_f32)
    say(f"  worst/bound, nRMSE: {res}")


def test_non_default_scale():
    say("bwd scale 0.3, N=300 d=128 causal")
    run_case(1, 2, 300, 128, True, "bf16", True, scale=0.3)


def test_constant_v_gives_zero_dq_dk():
    """All V rows equal: O does not depend on Q or K, so dQ = dK = 0 up to
    rounding of D against dP."""
    B, H, N, d = 1, 1, 200, 64
    say("bwd constant V")
    q, k, _ = make_qkv(B, H, N, d, seed=3, dtype="bf16")
    v = make_qkv(1, 1, 1, d, seed=4, dtype="bf16")[0].expand(B, H, N, d).contiguous()
    do = make_dout(B, H, N, d, 5, "bf16")
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    o, lse = fa.fwd(qd, kd, vd, causal=True)
    dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=True, out_f32=True)
    torch.cuda.synchronize()
    scale_dq = float(np.max(np.abs(to_f64(do)))) * float(np.max(np.abs(to_f64(k))))
    assert float(dq.abs().max()) < 1e-3 * scale_dq
    assert float(dk.abs().max()) < 1e-3 * scale_dq


def test_full_workload_sampled_heads():
    """B=8 H=16 N=2048 d=128 (the forward benchmark shape), causal and not,
    in the launch configuration of the full call; two heads checked."""
    B, H, N, d = 8, 16, 2048, 128
    q, k, v = make_qkv(B, H, N, d, seed=1, dtype="bf16")
    do = make_dout(B, H, N, d, 77, "bf16")
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    for causal in (False, True):
        say(f"bwd full B=8 H=16 N=2048 d=128 causal={causal}")
        o, lse = fa.fwd(qd, kd, vd, causal=causal)
        dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, out_f32=True)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (7, 15)):
            sl = (slice(b, b + 1), slice(h, h + 1))
            q64, k64, v64, do64 = (to_f64(t[sl]) for t in (q, k, v, do))
            ref = oracle.attention_backward(q64, k64, v64, do64, causal)
            m = bounds(q64, k64, v64, do64, causal, 1.0 / math.sqrt(d), "bf16")
            for name, g, gr, mm in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, m):
                check_grad(g[sl].cpu().numpy(), gr, mm, "bf16", "f32", f"{name} head ({b},{h})")


def test_d256_sampled_heads():
    """d = 256 at B=2 H=8 N=4096 (the head shape of the long-sequence d = 256
    forward workload, a quarter of its length), causal and not, in the
    launch configuration of the full call; two heads checked element by
    element."""
    B, H, N, d = 2, 8, 4096, 256
    q, k, v = make_qkv(B, H, N, d, seed=2, dtype="bf16")
    do = make_dout(B, H, N, d, 78, "bf16")
    qd, kd, vd, dod = (t.to(DEV) for t in (q, k, v, do))
    for causal in (False, True):
        say(f"bwd B=2 H=8 N=4096 d=256 causal={causal}")
        o, lse = fa.fwd(qd, kd, vd, causal=causal)
        dq, dk, dv = fa.bwd(qd, kd, vd, o, lse, dod, causal=causal, out_f32=True)
        torch.cuda.synchronize()
        for b, h in ((0, 0), (1, 7)):
            sl = (slice(b, b + 1), slice(h, h + 1))
            q64, k64, v64, do64 = (to_f64(t[sl]) for t in (q, k, v, do))
            ref = oracle.attention_backward(q64, k64, v64, do64, causal)
            m = bounds(q64, k64, v64, do64, causal, 1.0 / math.sqrt(d), "bf16")
            for name, g, gr, mm in zip(("dq", "dk", "dv"), (dq, dk, dv), ref, m):
                w, r = check_grad(g[sl].cpu().numpy(), gr, mm, "bf16", "f32", f"{name} head ({b},{h})")
                say(f"  {name} head ({b},{h}): worst/bound {w:.2f} nRMSE {r:.2e}")
