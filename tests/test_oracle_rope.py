"""Pins for the rotary-embedding oracle (oracle/rope.py) and its fusion into
the fp8 quantiser.

Independent of the oracle's own formulas: a complex-number formulation
(each pair as a + ib multiplied by e^{i angle}), the permutation that turns
one pairing into the other, a hand-written d = 2 rotation, per-pair norm
preservation, the relative-position property of the rotated dot product,
position 0 as the identity, the position offset, and the float32 angle
rule checked against numpy's float32 arithmetic.
"""

import numpy as np
import pytest

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_complex_formulation_interleaved():
    x = rand((2, 3, 17, 16), 1)
    y = oracle.rope(x, "interleaved", 10000.0, 5)
    c, s = oracle.rope_cos_sin(17, 16, 10000.0, 5)
    z = (x[..., 0::2] + 1j * x[..., 1::2]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    assert np.allclose(y[..., 0::2], z.real, atol=1e-13)
    assert np.allclose(y[..., 1::2], z.imag, atol=1e-13)


def test_complex_formulation_half():
    x = rand((1, 2, 9, 32), 2)
    y = oracle.rope(x, "half", 500.0, 0)
    c, s = oracle.rope_cos_sin(9, 32, 500.0, 0)
    z = (x[..., :16] + 1j * x[..., 16:]) * (c.astype(np.float64) + 1j * s.astype(np.float64))
    assert np.allclose(y[..., :16], z.real, atol=1e-13)
    assert np.allclose(y[..., 16:], z.imag, atol=1e-13)


def test_pairings_are_a_permutation_of_each_other():
    d = 64
    perm = np.empty(d, dtype=int)              # interleaved index -> half index
    perm[0::2] = np.arange(d // 2)
    perm[1::2] = np.arange(d // 2) + d // 2
    x = rand((3, 40, d), 3)
    yi = oracle.rope(x[..., perm], "interleaved", 10000.0, 7)
    yh = oracle.rope(x, "half", 10000.0, 7)
    assert np.array_equal(yi, yh[..., perm])


def test_two_dimensional_rotation_by_position():
    # d = 2: one pair, frequency 1, angle = position
    x = np.array([[1.0, 0.0], [0.0, 1.0], [3.0, -2.0]])
    y = oracle.rope(x, "interleaved", 10000.0, 0)
    for p in range(3):
        a = float(np.float32(p))
        c, s = float(np.float32(np.cos(a))), float(np.float32(np.sin(a)))
        rot = np.array([[c, -s], [s, c]])
        assert np.allclose(y[p], rot @ x[p], atol=1e-15)


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_norms_preserved_and_position_zero_identity(style):
    x = rand((4, 33, 128), 4)
    y = oracle.rope(x, style)
    h = 64
    if style == "interleaved":
        nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
        ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    else:
        nx = x[..., :h] ** 2 + x[..., h:] ** 2
        ny = y[..., :h] ** 2 + y[..., h:] ** 2
    # cos/sin are float32-rounded: |c + is| = 1 within 2^-23
    assert np.allclose(nx, ny, rtol=3e-7, atol=1e-12)
    assert np.array_equal(y[:, 0], x[:, 0])                     # position 0


@pytest.mark.parametrize("style", ["interleaved", "half"])
def test_relative_position(style):
    """<R(p) q, R(p') k> depends on p - p' only (up to the float32 angles)."""
    d = 64
    q, k = rand((1, d), 5), rand((1, d), 6)
    vals = []
    for shift in (0, 11, 250):
        rq = oracle.rope(q, style, 10000.0, 30 + shift)
        rk = oracle.rope(k, style, 10000.0, 10 + shift)
        vals.append(float(rq[0] @ rk[0]))
    assert np.allclose(vals, vals[0], atol=2e-4)
    assert not np.isclose(float(oracle.rope(q, style, 10000.0, 30)[0] @ k[0]), vals[0])


def test_position_offset_is_a_row_shift():
    x = rand((2, 50, 32), 7)
    long = oracle.rope(np.concatenate([np.zeros((2, 13, 32)), x], axis=1), "half", 10000.0, 0)
    assert np.array_equal(oracle.rope(x, "half", 10000.0, 13), long[:, 13:])


def test_float32_angle_rule():
    w = oracle.rope_frequencies(128, 10000.0)
    assert w.dtype == np.float32 and w[0] == 1.0
    assert abs(float(w[1]) - 10000.0 ** (-2 / 128)) <= 2.0 ** -24
    ang = oracle.rope_angles(4000, 128, 10000.0, 100)
    p = np.float32(100 + 3999)
    assert ang[3999, 5] == np.float32(p * w[5])                 # one float32 product


def test_fused_quantiser_equals_rope_then_quantise():
    x = rand((1, 2, 200, 64), 8).astype(np.float32)
    signs = np.where(rand((2, 64), 9) > 0, 1, -1).astype(np.int8)
    rope = ("interleaved", 10000.0, 3)
    c1, s1 = oracle.fp8_quantize(x, signs, 128, rope)
    c2, s2 = oracle.fp8_quantize(oracle.rope(x, *rope), signs, 128)
    assert np.array_equal(c1, c2) and np.array_equal(s1, s2)
    # the rotary step changes the codes
    c3, _ = oracle.fp8_quantize(x, signs, 128)
    assert not np.array_equal(c1, c3)


def test_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.rope(rand((3, 4), 0), "neox")
    with pytest.raises(ValueError):
        oracle.rope(rand((3, 5), 0))
