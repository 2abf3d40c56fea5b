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
