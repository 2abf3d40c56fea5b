"""OCP FP8 E4M3 ("fn" variant) rounding and encoding (test infrastructure only).

The pages name FP8 without fixing the format ("FlashAttention-3: Fast &
Accurate Attention with Asynchrony & Low-Precision", section "New GPU Features
on Hopper: WGMMA, TMA, FP8"). Reading: the OCP 8-bit floating point
specification's E4M3 encoding, the one gfx950 MFMA consumes:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals m/8 * 2^-6 (smallest 2^-9);
* no infinities; S.1111.111 is NaN, so the largest finite value is
  S.1111.110 = 1.75 * 2^8 = 448.

Rounding reading: round to nearest, ties to even, and saturate to +-448 (the
quantiser scales blocks to fit, so saturation only absorbs the rounding of the
scale itself). NaN inputs are outside the contract.

Written from the format definition above, with no tables: every value is
built from its exponent and mantissa.
"""

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6       # smallest normal binade 2^-6
_MANT_BITS = 3


def _binade(a):
    """floor(log2 a) for a > 0, exactly (via frexp, no log rounding)."""
    _, e = np.frexp(a)            # a = f * 2^e, f in [0.5, 1)
    return e - 1


def e4m3_round(x):
    """Nearest e4m3 value (ties to even, saturating), as float64."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    safe = np.where(a > 0, a, 1.0)
    e = np.maximum(_binade(safe), _MIN_NORMAL_EXP)
    quantum = np.ldexp(1.0, e - _MANT_BITS)     # spacing of values in binade e
    # a / quantum is exact in float64 (power-of-two scaling); np.rint rounds
    # half to even.
    r = np.rint(a / quantum) * quantum
    r = np.minimum(r, E4M3_MAX)                  # cannot trigger: 448 is a grid point
    r = np.where(a > 0, r, 0.0)
    return np.copysign(r, x)


def e4m3_encode(x):
    """Round (as e4m3_round) and return the uint8 bit patterns."""
    x = np.asarray(x, dtype=np.float64)
    r = e4m3_round(x)
    a = np.abs(r)
    sign = np.signbit(x).astype(np.uint8) << 7
    safe = np.where(a > 0, a, 1.0)
    e = _binade(safe)
    normal = a >= np.ldexp(1.0, _MIN_NORMAL_EXP)
    # normal: field = e + 7, mantissa = (a / 2^e - 1) * 8
    n_field = (e + 7).astype(np.int64)
    n_mant = np.rint((a / np.ldexp(1.0, e) - 1.0) * 8).astype(np.int64)
    # subnormal: field = 0, mantissa = a / 2^-9
    s_mant = np.rint(a / np.ldexp(1.0, _MIN_NORMAL_EXP - _MANT_BITS)).astype(np.int64)
    field = np.where(normal, n_field, 0)
    mant = np.where(normal, n_mant, s_mant)
    code = (field << 3) | mant
    code = np.where(a > 0, code, 0)
    return (sign | code.astype(np.uint8)).astype(np.uint8)


def e4m3_decode(codes):
    """Value of each uint8 e4m3 bit pattern (NaN for S.1111.111)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    field = (c >> 3) & 0xF
    mant = c & 0x7
    normal = np.ldexp(1.0 + mant / 8.0, field - 7)
    sub = np.ldexp(mant / 8.0, _MIN_NORMAL_EXP)
    val = np.where(field > 0, normal, sub)
    val = np.where((field == 0xF) & (mant == 0x7), np.nan, val)
    return sign * val
