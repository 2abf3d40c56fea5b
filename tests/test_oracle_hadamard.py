"""Pins for the random-sign Hadamard transform (oracle/hadamard.py).

"FlashAttention-3: Fast & Accurate Attention with Asynchrony & Low-Precision",
section "Incoherent Processing for FP8 Accuracy": Q and K are multiplied by a
random orthogonal matrix per head (Hadamard with random signs); because it is
orthogonal, QK^T and therefore attention are unchanged.
"""

import numpy as np
import pytest
import scipy.linalg

import oracle


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_fwht_matches_scipy_hadamard(d):
    rng = np.random.default_rng(d)
    x = rng.standard_normal((3, 5, d))
    np.testing.assert_allclose(oracle.fwht(x), x @ scipy.linalg.hadamard(d), atol=1e-11)


def test_fwht_involution():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((4, 128))
    np.testing.assert_allclose(oracle.fwht(oracle.fwht(x)), 128 * x, atol=1e-10)


@pytest.mark.parametrize("d", [64, 128, 256])
def test_rotation_is_orthogonal(d):
    rng = np.random.default_rng(d + 1)
    signs = (rng.integers(0, 2, (1, d)) * 2 - 1).astype(np.int8)
    m = oracle.random_sign_hadamard(np.eye(d)[None], signs)[0]   # rows e_i M
    np.testing.assert_allclose(m @ m.T, np.eye(d), atol=1e-12)
    # every entry has magnitude 1/sqrt(d): a one-hot outlier is spread evenly
    np.testing.assert_allclose(np.abs(m), 1 / np.sqrt(d), atol=1e-15)
    # explicit matrix form diag(s) H / sqrt(d)
    np.testing.assert_allclose(m, np.diag(signs[0].astype(float)) @ scipy.linalg.hadamard(d)
                               / np.sqrt(d), atol=1e-15)


def test_scores_and_attention_unchanged():
    rng = np.random.default_rng(2)
    H, N, d = 3, 48, 64
    q, k, v = (rng.standard_normal((2, H, N, d)) for _ in range(3))
    signs = (rng.integers(0, 2, (H, d)) * 2 - 1).astype(np.int8)
    qr = oracle.random_sign_hadamard(q, signs)
    kr = oracle.random_sign_hadamard(k, signs)
    np.testing.assert_allclose(qr @ np.swapaxes(kr, -1, -2), q @ np.swapaxes(k, -1, -2),
                               atol=1e-10)
    for causal in (False, True):
        o1, l1 = oracle.attention(q, k, v, causal)
        o2, l2 = oracle.attention(qr, kr, v, causal)
        np.testing.assert_allclose(o1, o2, atol=1e-10)
        np.testing.assert_allclose(l1, l2, atol=1e-10)


def test_different_signs_per_head_break_cross_head_identity():
    """Signs are per head: rotating Q with one head's signs and K with another's
    does change the scores (guards against ignoring the head index)."""
    rng = np.random.default_rng(3)
    d = 64
    q, k = rng.standard_normal((2, 1, 2, 8, d))
    signs = (rng.integers(0, 2, (2, d)) * 2 - 1).astype(np.int8)
    qr = oracle.random_sign_hadamard(q, signs)
    kr = oracle.random_sign_hadamard(k, signs[::-1])
    s1 = qr[0, 0] @ kr[0, 0].T
    assert np.max(np.abs(s1 - q[0, 0] @ k[0, 0].T)) > 1e-3
