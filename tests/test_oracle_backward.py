"""Pins for the attention-gradient oracle (oracle/backward.py).

The gradients are tied to things other than the oracle's own formulas:
central finite differences of the forward oracle, torch's CPU autograd
through scaled_dot_product_attention in float64 (an independent library
implementation), closed forms (constant V, zero scale, a single key) and
invariants that follow from the softmax rows summing to one.
"""

import numpy as np
import pytest
import torch

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def loss(q, k, v, do, causal, scale):
    o, _ = oracle.attention(q, k, v, causal, scale)
    return float(np.sum(o * do))


@pytest.mark.parametrize("causal", [False, True])
def test_finite_differences(causal):
    """Central differences of sum(O * dO) in float64 on a tiny head."""
    B, H, N, d = 1, 2, 5, 4
    q, k, v, do = (rand((B, H, N, d), s) for s in (1, 2, 3, 4))
    scale = 0.7
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal, scale)
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args = {"q": q, "k": k, "v": v}
            lp = loss(*(xp if n == name else args[n] for n in "qkv"), do, causal, scale)
            lm = loss(*(xm if n == name else args[n] for n in "qkv"), do, causal, scale)
            num[idx] = (lp - lm) / (2 * eps)
        assert np.max(np.abs(num - g)) < 1e-7, name


@pytest.mark.parametrize("causal", [False, True])
def test_torch_autograd(causal):
    """torch CPU autograd through scaled_dot_product_attention, float64."""
    B, H, N, d = 2, 2, 37, 16
    q, k, v, do = (rand((B, H, N, d), s) for s in (5, 6, 7, 8))
    scale = 1.0 / np.sqrt(d)
    tq, tk, tv = (torch.tensor(x, requires_grad=True) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
    o.backward(torch.tensor(do))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal, scale)
    for g, t in ((dq, tq), (dk, tk), (dv, tv)):
        assert np.max(np.abs(g - t.grad.numpy())) < 1e-12


def test_constant_v():
    """All V rows equal: O does not depend on Q or K, so dQ = dK = 0 and
    dV_j = sum_i P_ij dO_i."""
    B, H, N, d = 1, 1, 9, 8
    q, k, do = (rand((B, H, N, d), s) for s in (9, 10, 11))
    v = np.broadcast_to(rand((1, 1, 1, d), 12), (B, H, N, d)).copy()
    for causal in (False, True):
        dq, dk, dv = oracle.attention_backward(q, k, v, do, causal)
        assert np.max(np.abs(dq)) < 1e-12 and np.max(np.abs(dk)) < 1e-12
        # rows of P sum to one, so the dV rows sum to the dO rows' sum
        assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)


def test_zero_scale():
    """scale = 0: P is uniform over the visible keys; dQ = dK = 0 and
    dV_j = sum over the queries that see key j of dO_i / (number of keys i sees)."""
    B, H, N, d = 1, 1, 6, 3
    q, k, v, do = (rand((B, H, N, d), s) for s in (13, 14, 15, 16))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, False, 0.0)
    assert np.all(dq == 0) and np.all(dk == 0)
    assert np.allclose(dv[0, 0], np.broadcast_to(do[0, 0].mean(axis=0), (N, d)), atol=1e-14)
    dq, dk, dv = oracle.attention_backward(q, k, v, do, True, 0.0)
    expect = np.zeros((N, d))
    for j in range(N):
        for i in range(j, N):
            expect[j] += do[0, 0, i] / (i + 1)
    assert np.allclose(dv[0, 0], expect, atol=1e-14)


def test_single_key():
    """N = 1: P = [1], so dV = dO and dQ = dK = 0."""
    q, k, v, do = (rand((2, 3, 1, 8), s) for s in (17, 18, 19, 20))
    dq, dk, dv = oracle.attention_backward(q, k, v, do)
    assert np.allclose(dv, do, atol=0) and np.all(np.abs(dq) < 1e-15) and np.all(np.abs(dk) < 1e-15)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    """Rows of dS sum to zero: the dK rows sum to zero, the dV rows sum to
    the dO rows, and a common shift of every key leaves all gradients."""
    B, H, N, d = 1, 2, 23, 8
    q, k, v, do = (rand((B, H, N, d), s) for s in (21, 22, 23, 24))
    dq, dk, dv = oracle.attention_backward(q, k, v, do, causal)
    assert np.max(np.abs(dk.sum(axis=2))) < 1e-12
    assert np.allclose(dv.sum(axis=2), do.sum(axis=2), atol=1e-12)
    shift = rand((1, 1, 1, d), 25)
    dq2, dk2, dv2 = oracle.attention_backward(q, k + shift, v, do, causal)
    for a, b in ((dq, dq2), (dk, dk2), (dv, dv2)):
        assert np.max(np.abs(a - b)) < 1e-11


def test_delta_matches_definition():
    """D_i = sum_j P_ij dP_ij equals sum_c dO_ic O_ic."""
    B, H, N, d = 1, 1, 11, 5
    q, k, v, do = (rand((B, H, N, d), s) for s in (26, 27, 28, 29))
    o, _ = oracle.attention(q, k, v)
    p = oracle.softmax_probs(q[0, 0], k[0, 0], False)
    dp = do[0, 0] @ v[0, 0].T
    assert np.allclose(oracle.attention_delta(o, do)[0, 0], np.sum(p * dp, axis=1), atol=1e-12)
