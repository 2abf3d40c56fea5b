"""Pins the online-softmax recurrence (oracle/online.py) to the definition.

The recurrence (running max, separate denominator, deferred normalisation) is
read from "FlashAttention - one, two, three!", sections "FlashAttention v1."
and "FlashAttention v2.", whose formulas are missing from the text. Exactness
is the property that pins the reading: any block size and visit order must
give the naive result to rounding.
"""

import numpy as np
import pytest

import oracle


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("order", ["forward", "reverse", "shuffle"])
@pytest.mark.parametrize("N,bq,bk", [(37, 8, 8), (100, 16, 7), (64, 64, 64), (50, 1, 50), (65, 32, 1)])
def test_online_equals_naive(N, bq, bk, order, causal):
    rng = np.random.default_rng(N * 31 + bk)
    q, k, v = (rng.standard_normal((1, 2, N, 8)) * 2 for _ in range(3))
    o, lse = oracle.attention(q, k, v, causal)
    oo, lo = oracle.attention_online(q, k, v, causal, block_q=bq, block_k=bk, order=order)
    assert np.max(np.abs(o - oo)) <= 1e-12
    assert np.max(np.abs(lse - lo)) <= 1e-12


def test_online_large_logits_no_overflow():
    """Logits of several hundred: the running max keeps exp finite."""
    rng = np.random.default_rng(3)
    q, k, v = (rng.standard_normal((1, 1, 40, 4)) for _ in range(3))
    q *= 60.0
    o, lse = oracle.attention(q, k, v, False, 1.0)
    oo, lo = oracle.attention_online(q, k, v, False, 1.0, block_q=8, block_k=8)
    assert np.all(np.isfinite(oo))
    assert np.max(np.abs(o - oo)) <= 1e-11
    assert np.max(np.abs(lse - lo) / np.abs(lse)) <= 1e-14 * 100
