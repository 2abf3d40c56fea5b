"""Shared helpers for the GPU parity tests: tolerances, row sampling, metrics.

Tolerances (fwd outputs vs the float64 oracle on the same rounded inputs):
  16-bit inputs:  max-abs <= 4e-3 and RMSE <= 5e-4 on O; |LSE error| <= 1e-3.
  With O stored in 16 bits both bounds apply to the error beyond half a unit
  in the last place of the stored format at |O_ref|, i.e. beyond what storing
  the exact result already costs (max(|O - O_ref| - ulp/2, 0)).
  FP8 inputs: RMSE <= 1.5e-2 vs the exact oracle; random-sign Hadamard with
  block scales must beat plain per-tensor scaling; LSE within 1e-3 of the
  oracle run on the oracle's own quantised inputs.
"""

import numpy as np
import torch

MAX_ABS = 4e-3
RMSE = 5e-4
LSE_TOL = 1e-3
FP8_RMSE = 1.5e-2


def half_ulp(x, dtype):
    """Half a unit in the last place of `dtype` at |x| (float64 array)."""
    mant = {"bf16": 7, "fp16": 10, torch.bfloat16: 7, torch.float16: 10}[dtype]
    a = np.maximum(np.abs(x), 2.0 ** -14)
    e = np.floor(np.log2(a))
    return 2.0 ** (e - mant - 1)


def sample_rows(N, seed, extra=24):
    """Tile-boundary rows plus random ones."""
    base = [0, 1, 2, 3, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257, 511, 512,
            N // 2, N - 65, N - 64, N - 33, N - 2, N - 1]
    rng = np.random.default_rng(seed)
    rows = set(r for r in base if 0 <= r < N)
    rows.update(rng.integers(0, N, size=min(extra, N)).tolist())
    return np.array(sorted(rows))


def errors(o, o_ref):
    d = np.asarray(o, dtype=np.float64) - o_ref
    return float(np.max(np.abs(d))), float(np.sqrt(np.mean(d * d)))


def check_o(o, o_ref, out_dtype, where=""):
    """Assert the 16-bit-input tolerances; out_dtype 'f32', 'bf16' or 'fp16'."""
    o = np.asarray(o, dtype=np.float64)
    assert np.all(np.isfinite(o)), f"non-finite output {where}"
    mx, rmse = errors(o, o_ref)
    if out_dtype == "f32":
        assert mx <= MAX_ABS, f"max-abs {mx:.3e} > {MAX_ABS} {where}"
        assert rmse <= RMSE, f"RMSE {rmse:.3e} > {RMSE} {where}"
    else:
        # error beyond what storing the exact result in 16 bits already costs
        excess = np.maximum(np.abs(o - o_ref) - half_ulp(o_ref, out_dtype), 0.0)
        worst = float(np.max(excess))
        ermse = float(np.sqrt(np.mean(excess * excess)))
        assert worst <= MAX_ABS, f"max-abs beyond storage rounding {worst:.3e} {where}"
        assert ermse <= RMSE, f"RMSE beyond storage rounding {ermse:.3e} {where}"
    return mx, rmse


def check_lse(lse, lse_ref, where=""):
    lse = np.asarray(lse, dtype=np.float64)
    err = float(np.max(np.abs(lse - lse_ref)))
    assert err <= LSE_TOL, f"LSE error {err:.3e} > {LSE_TOL} {where}"
    return err


def fp8_p_factor(vs, N, block_rows=128):
    """Per-key factor f_j in [1, 2) by which the block-scaled fp8 forward
    multiplies 8 p_j before rounding P' to e4m3: the significand part of
    w_j = sv_j / sv_max (vs: one head's V block scales), w_j = 2^(e_j - 1) f_j,
    whose power of two the PV product applies exactly. [N] float64."""
    w = np.maximum(np.asarray(vs, dtype=np.float64) / np.max(vs), 2.0 ** -126)
    m, _ = np.frexp(w)
    return np.repeat(2.0 * m, block_rows)[:N]


# The fp8 kernels take exponentials against a reference maximum set this
# many log2 units above an exact tile maximum (never more above the row's
# maximum than that), so their p are at least 2^-FP8_REF_MARGIN of p
# against the row maximum.
FP8_REF_MARGIN = 2


def fp8_p_rounding_bound(q, k, v, b, h, rows, causal, w=None, scale=None):
    """Elementwise bound on |O_gpu - O_dq| for query rows `rows` of head
    (b, h), where O_dq is exact attention of the dequantised inputs q, k, v
    (float64 [B,H,N,d]) and the GPU differs from it only by rounding the
    weights P' = 8 p'_j w_j to e4m3 before the PV product (p'_j relative to
    the kernel's reference maximum, the row sum taken from the unrounded p',
    the factor w_j undone exactly afterwards). An e4m3 rounding moves x by
    at most max(2^-4 x, 2^-10) (half a step of a normal, half the subnormal
    spacing 2^-9); with p_j against the row maximum and p'_j >= 2^-M p_j
    (M = FP8_REF_MARGIN),
        |dO_ic| <= sum_j max(2^-4 p_j, 2^(M-13) / w_j) |V_jc| / sum_j p_j.
    w: per-key factor of P' (the block-scaled path: fp8_p_factor; None: 1,
    the microscaled path). Returns [len(rows), d]."""
    qh = np.asarray(q[b, h], dtype=np.float64)[rows]
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.abs(np.asarray(v[b, h], dtype=np.float64))
    N, d = kh.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    s = scale * (qh @ kh.T)
    if causal:
        s = np.where(np.arange(N)[None, :] <= np.asarray(rows)[:, None], s, -np.inf)
    p = np.exp(s - s.max(axis=1, keepdims=True))
    wj = np.ones(N) if w is None else np.asarray(w, dtype=np.float64)
    err = np.maximum(2.0 ** -4 * p, np.where(p > 0, 2.0 ** (FP8_REF_MARGIN - 13) / wj[None, :], 0.0))
    return (err @ vh) / p.sum(axis=1, keepdims=True)


def p16_rounding_bound(q, k, v, b, h, causal, scale, dtype="bf16"):
    """Elementwise bound on |O_gpu - O_ref| for every row of head (b, h) when
    the GPU rounds each weight p_j to a 16-bit float (relative error <= u,
    the unit roundoff: 2^-8 for bf16, 8 significant bits; 2^-11 for fp16) and normalises by the sum of the rounded
    weights. With w_j = p_j / sum p and r_j = p_j (1 + e_j),
        O - O_ref = sum_j w_j e_j (v_j - O_ref) / (1 + sum_j w_j e_j),
    so |dO_c| <= u / (1 - u) * sum_j w_j |v_jc - O_ref_c|. Returns [N, d]
    (float64), plus 1e-5 * max|v| for the fp32 accumulation."""
    u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[dtype]
    qh = np.asarray(q[b, h], dtype=np.float64)
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    N = qh.shape[0]
    s = scale * (qh @ kh.T)
    if causal:
        s = np.where(np.arange(N)[None, :] <= np.arange(N)[:, None], s, -np.inf)
    w = np.exp(s - s.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    o = w @ vh
    dev = np.einsum("ij,ijc->ic", w, np.abs(vh[None, :, :] - o[:, None, :]))
    return u / (1.0 - u) * dev + 1e-5 * np.max(np.abs(vh))
