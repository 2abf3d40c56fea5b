"""Pins for the MX quantiser oracle (oracle/mx.py).

Hand-worked blocks, the power-of-two scale rule checked against frexp,
saturation of the top of the range, all-zero and ragged blocks, lossless
round trips of values on the scaled e4m3 grid, the per-element error bound,
block independence, and the fake-quant attention against the plain
attention of the dequantised tensors.
"""

import math

import numpy as np
import pytest

import oracle
from oracle.mx import fake_quant_attention_mx, mx_dequantize, mx_quantize


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_hand_worked_block():
    x = np.zeros((1, 1, 1, 32))
    x[0, 0, 0, :4] = [1.0, 0.5, -3.0, 0.0078125]
    codes, e = mx_quantize(x, "d")
    # amax 3: floor(log2 3) = 1, e = 1 - 8 = -7, X = 2^-7
    assert e[0, 0, 0, 0] == -7
    vals = oracle.e4m3_decode(codes[0, 0, 0, :4])
    # 1 / 2^-7 = 128, 0.5 -> 64, -3 -> -384, 2^-7 -> 1: all exact e4m3 values
    assert list(vals) == [128.0, 64.0, -384.0, 1.0]
    assert np.array_equal(mx_dequantize(codes, e, "d")[0, 0, 0, :4], x[0, 0, 0, :4])


def test_exponent_rule_against_frexp():
    x = rand((2, 3, 5, 64), 1) * np.exp2(rand((2, 3, 5, 64), 2) * 6)
    _, e = mx_quantize(x, "d")
    blocks = np.abs(x.astype(np.float32).astype(np.float64)).reshape(2, 3, 5, 2, 32).max(-1)
    for a, ee in zip(blocks.ravel(), e.ravel()):
        _, ex = math.frexp(a)             # a = f * 2^ex, f in [0.5, 1)
        assert ee == (ex - 1) - 8
        assert 256.0 <= a / 2.0 ** ee < 512.0


def test_top_of_range_saturates():
    x = np.zeros((1, 1, 1, 32))
    x[0, 0, 0, 0] = 1.99                    # e = -8, 1.99 * 256 = 509.4 -> 448
    x[0, 0, 0, 1] = 1.70                    # 435.2 -> 448 (nearest e4m3 above 416)
    codes, e = mx_quantize(x, "d")
    assert e[0, 0, 0, 0] == -8
    assert oracle.e4m3_decode(codes[0, 0, 0, 0]) == 448.0
    assert oracle.e4m3_decode(codes[0, 0, 0, 1]) == 448.0


def test_zero_and_ragged_blocks_along_n():
    x = rand((1, 2, 70, 64), 3)
    x[0, 1, 32:64] = 0.0                    # one all-zero block
    codes, e = mx_quantize(x, "n")
    assert e.shape == (1, 2, 3, 64)         # ceil(70 / 32) blocks
    assert np.all(e[0, 1, 1] == -127) and np.all(codes[0, 1, 32:64] == 0)
    # the ragged block (rows 64..69) takes its own maximum
    blk = np.abs(x[0, 0, 64:70].astype(np.float32))
    assert np.array_equal(e[0, 0, 2], np.floor(np.log2(blk.max(0))).astype(int) - 8)


def test_lossless_on_scaled_grid():
    rng = np.random.default_rng(4)
    grid = oracle.e4m3_decode(np.arange(0, 127, dtype=np.uint8))      # non-negative finite codes
    vals = rng.choice(grid[grid > 0], size=(1, 1, 3, 64)) * rng.choice([-1.0, 1.0], size=(1, 1, 3, 64))
    vals[..., ::32] = 448.0                  # every block tops out at 448 * 2^k
    x = vals * 2.0 ** -10
    codes, e = mx_quantize(x, "d")
    assert np.all(e == -10)
    assert np.array_equal(mx_dequantize(codes, e, "d"), x)


@pytest.mark.parametrize("axis", ["d", "n"])
def test_error_bound_and_block_independence(axis):
    x = rand((1, 2, 96, 128), 5)
    codes, e = mx_quantize(x, axis)
    y = mx_dequantize(codes, e, axis)
    xf = x.astype(np.float32).astype(np.float64)
    scale = np.exp2(e.astype(float))
    if axis == "d":
        s = np.repeat(scale, 32, axis=-1)
    else:
        s = np.repeat(scale, 32, axis=2)[:, :, :96]
    q = np.abs(xf) / s                       # in [0, 512)
    # half an e4m3 step (2^-4 relative) below 448, plus the clamp above it
    step = np.exp2(np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 3)
    bound = np.where(q <= 448, step / 2, q - 448) * s + 1e-300
    assert np.all(np.abs(y - xf) <= bound * (1 + 1e-12))
    # changing one block does not move another block's scale or codes
    x2 = x.copy()
    if axis == "d":
        x2[0, 0, 0, :32] *= 1000.0
    else:
        x2[0, 0, :32, 0] *= 1000.0
    c2, e2 = mx_quantize(x2, axis)
    if axis == "d":
        assert np.array_equal(e2[0, 0, 0, 1:], e[0, 0, 0, 1:]) and np.array_equal(c2[0, 0, 0, 32:], codes[0, 0, 0, 32:])
    else:
        assert np.array_equal(e2[0, 0, 1:], e[0, 0, 1:]) and np.array_equal(c2[0, 0, :32, 1:], codes[0, 0, :32, 1:])


def test_hadamard_before_quantisation():
    x = rand((1, 2, 40, 64), 6)
    signs = np.where(rand((2, 64), 7) > 0, 1, -1).astype(np.int8)
    c1, e1 = mx_quantize(x, "d", signs)
    c2, e2 = mx_quantize(oracle.random_sign_hadamard(x, signs), "d")
    assert np.array_equal(c1, c2) and np.array_equal(e1, e2)


def test_fake_quant_attention_is_attention_of_dequantised():
    q, k, v = rand((1, 2, 50, 64), 8), rand((1, 2, 50, 64), 9), rand((1, 2, 50, 64), 10)
    signs = np.where(rand((2, 64), 11) > 0, 1, -1).astype(np.int8)
    o, lse = fake_quant_attention_mx(q, k, v, signs, True)
    qd = mx_dequantize(*mx_quantize(q, "d", signs), "d")
    kd = mx_dequantize(*mx_quantize(k, "d", signs), "d")
    vd = mx_dequantize(*mx_quantize(v, "n"), "n")
    o2, lse2 = oracle.attention(qd, kd, vd, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)
    # and it is close to the exact attention (the rotation cancels in Q K^T)
    oe, _ = oracle.attention(q, k, v, True)
    assert np.sqrt(np.mean((o - oe) ** 2)) < 3e-2
