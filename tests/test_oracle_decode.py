"""Pins for the decode-shaped attention oracle (oracle/decode.py).

Tied to things other than the oracle's own code: a pure-Python brute force
on tiny inputs, torch's CPU scaled_dot_product_attention in float64 with an
explicit mask (an independent library routine), the square forward oracle
(pinned on its own in test_oracle_attention.py) where the shapes coincide,
closed forms (scale 0 gives the mean of the visible value rows and
LSE = ln(count)), and the conventions for rows that see no key.
"""

import math

import numpy as np
import pytest
import torch

import oracle


def rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def brute(q, k, v, causal, scale, lens):
    """Direct evaluation with Python floats and math.exp (no numpy algebra)."""
    B, H, Nq, d = q.shape
    Hkv = k.shape[1]
    g = H // Hkv
    o = np.zeros(q.shape[:3] + (v.shape[-1],))
    lse = np.full(q.shape[:3], -math.inf)
    for b in range(B):
        L = lens[b]
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(L) if not causal or j <= L - Nq + i]
                if not keys:
                    continue
                logit = {j: scale * sum(q[b, h, i, c] * k[b, h // g, j, c] for c in range(d))
                         for j in keys}
                top = max(logit.values())
                w = {j: math.exp(logit[j] - top) for j in keys}
                tot = sum(w.values())
                for c in range(v.shape[-1]):
                    o[b, h, i, c] = sum(w[j] * v[b, h // g, j, c] for j in keys) / tot
                lse[b, h, i] = top + math.log(tot)
    return o, lse


@pytest.mark.parametrize("causal", [False, True])
def test_brute_force_gqa_ragged(causal):
    B, H, Hkv, Nq, Nk, d = 3, 4, 2, 3, 9, 5
    q, k, v = rand((B, H, Nq, d), 1), rand((B, Hkv, Nk, d), 2), rand((B, Hkv, Nk, d), 3)
    lens = [9, 4, 2]                       # batch 2 has fewer keys than queries
    o, lse = oracle.attention_decode(q, k, v, causal, 0.6, lens)
    ob, lb = brute(q, k, v, causal, 0.6, lens)
    assert np.allclose(o, ob, atol=1e-12)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.allclose(lse[fin], lb[fin], atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_torch_sdpa_masked(causal):
    """torch CPU SDPA (float64) with the bottom-right mask built per batch."""
    B, H, Hkv, Nq, Nk, d = 2, 6, 3, 4, 37, 16
    q, k, v = rand((B, H, Nq, d), 4), rand((B, Hkv, Nk, d), 5), rand((B, Hkv, Nk, d), 6)
    lens = [37, 20]
    o, lse = oracle.attention_decode(q, k, v, causal, None, lens)
    g = H // Hkv
    for b in range(B):
        L = lens[b]
        kt = torch.from_numpy(k[b, :, :L]).repeat_interleave(g, dim=0)
        vt = torch.from_numpy(v[b, :, :L]).repeat_interleave(g, dim=0)
        qt = torch.from_numpy(q[b])
        mask = torch.ones(Nq, L, dtype=torch.bool)
        if causal:
            mask = torch.arange(L)[None, :] <= (L - Nq + torch.arange(Nq))[:, None]
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask)
        assert np.allclose(o[b], ref.numpy(), atol=1e-12)
        logits = (qt @ kt.transpose(-1, -2)) / math.sqrt(d)
        logits = logits.masked_fill(~mask, -math.inf)
        assert np.allclose(lse[b], torch.logsumexp(logits, dim=-1).numpy(), atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_square_case_is_the_forward(causal):
    B, H, N, d = 2, 3, 23, 8
    q, k, v = rand((B, H, N, d), 7), rand((B, H, N, d), 8), rand((B, H, N, d), 9)
    o, lse = oracle.attention_decode(q, k, v, causal)
    of, lf = oracle.attention(q, k, v, causal)
    assert np.allclose(o, of, atol=1e-12) and np.allclose(lse, lf, atol=1e-12)


def test_groups_equal_repeated_heads():
    B, H, Hkv, Nq, Nk, d = 2, 8, 2, 2, 30, 4
    q, k, v = rand((B, H, Nq, d), 10), rand((B, Hkv, Nk, d), 11), rand((B, Hkv, Nk, d), 12)
    o, lse = oracle.attention_decode(q, k, v, True)
    kr, vr = (np.repeat(x, H // Hkv, axis=1) for x in (k, v))
    o2, lse2 = oracle.attention_decode(q, kr, vr, True)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


def test_last_query_sees_every_key():
    """Causal bottom-right: the last query row is the non-causal row."""
    B, H, Nq, Nk, d = 1, 2, 5, 40, 8
    q, k, v = rand((B, H, Nq, d), 13), rand((B, H, Nk, d), 14), rand((B, H, Nk, d), 15)
    oc, lc = oracle.attention_decode(q, k, v, True)
    on, ln = oracle.attention_decode(q, k, v, False)
    assert np.allclose(oc[:, :, -1], on[:, :, -1], atol=1e-14)
    assert np.allclose(lc[:, :, -1], ln[:, :, -1], atol=1e-14)
    assert not np.allclose(oc[:, :, 0], on[:, :, 0])


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_mean_of_visible_values(causal):
    B, H, Nq, Nk, d = 2, 1, 3, 11, 4
    q, k, v = rand((B, H, Nq, d), 16), rand((B, H, Nk, d), 17), rand((B, H, Nk, d), 18)
    lens = [11, 5]
    o, lse = oracle.attention_decode(q, k, v, causal, 0.0, lens)
    for b in range(B):
        for i in range(Nq):
            n = lens[b] - (Nq - 1 - i) if causal else lens[b]
            assert np.allclose(o[b, 0, i], v[b, 0, :n].mean(axis=0), atol=1e-14)
            assert abs(lse[b, 0, i] - math.log(n)) < 1e-14


def test_rows_without_keys():
    B, H, Nq, Nk, d = 2, 2, 4, 6, 4
    q, k, v = rand((B, H, Nq, d), 19), rand((B, H, Nk, d), 20), rand((B, H, Nk, d), 21)
    o, lse = oracle.attention_decode(q, k, v, True, None, [0, 2])
    assert np.all(o[0] == 0) and np.all(np.isneginf(lse[0]))
    # L = 2 < Nq = 4: rows 0 and 1 see nothing, row 2 sees key 0, row 3 keys 0-1
    assert np.all(o[1, :, :2] == 0) and np.all(np.isneginf(lse[1, :, :2]))
    assert np.allclose(o[1, :, 2], v[1, :, 0], atol=1e-15)
    assert np.all(np.isfinite(lse[1, :, 2:]))


def test_rejects_bad_shapes():
    q = rand((1, 3, 1, 4), 0)
    k = rand((1, 2, 5, 4), 1)
    with pytest.raises(ValueError):
        oracle.attention_decode(q, k, k)
    with pytest.raises(ValueError):
        oracle.attention_decode(q[:, :2], k, k, seqlens_k=[6])
