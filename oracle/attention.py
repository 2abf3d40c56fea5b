"""Naive materialised-softmax attention in float64 (test infrastructure only).

Definition followed: "FlashAttention - one, two, three!" (Medium), section
"Standard Attention": read the N x d matrices Q and K, form the N x N logits
S = QK^T, take the row softmax, and multiply by V to get the N x d output.
FlashAttention (all three versions) is an exact rewrite of this computation:
the review "FlashAttention-3: почему внимание стало быстрее", sections
"Коротко" and "FAQ", states that the formula itself is unchanged.

Readings where the pages are silent:
* layout [B, H, N, d] for q, k, v and o; [B, H, N] for the log-sum-exp;
* softmax_scale multiplies S before the row max is taken;
* causal means key j is visible to query i iff j <= i (N_q == N_k);
* LSE_i = ln sum_j exp(S_ij) with the scale included, natural log.

The row log-sum-exp is the "few constants" per row kept in global memory
(Medium page, section "FlashAttention v1.").
"""

import numpy as np


def _logits(q, k, scale, causal, rows):
    """S = scale * Q[rows] K^T with -inf above the causal diagonal."""
    s = scale * (q[rows] @ k.T)
    if causal:
        cols = np.arange(k.shape[0])
        s[cols[None, :] > np.asarray(rows)[:, None]] = -np.inf
    return s


def _head(q, k, v, causal, scale, rows):
    """One (b, h) head, the given query rows. Returns (O[rows], LSE[rows])."""
    s = _logits(q, k, scale, causal, rows)
    m = np.max(s, axis=1, keepdims=True)          # row max (finite: row has key 0)
    p = np.exp(s - m)                               # unnormalised probabilities
    l = np.sum(p, axis=1, keepdims=True)            # row denominator
    o = (p @ v) / l
    lse = m[:, 0] + np.log(l[:, 0])
    return o, lse


def attention(q, k, v, causal=False, scale=None, chunk=1024):
    """Exact attention for all rows.

    q, k, v: float arrays [B, H, N, d] (upcast to float64 here).
    Returns (O [B, H, N, d] float64, LSE [B, H, N] float64).
    Rows are processed ``chunk`` at a time so S never exceeds chunk x N.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o = np.empty((B, H, N, v.shape[-1]), dtype=np.float64)
    lse = np.empty((B, H, N), dtype=np.float64)
    for b in range(B):
        for h in range(H):
            for r0 in range(0, N, chunk):
                rows = np.arange(r0, min(N, r0 + chunk))
                o[b, h, rows], lse[b, h, rows] = _head(q[b, h], k[b, h], v[b, h],
                                                       causal, scale, rows)
    return o, lse


def attention_rows(q, k, v, b, h, rows, causal=False, scale=None):
    """Exact attention for selected query rows of head (b, h).

    Used to check full-size GPU outputs on a sample of rows the oracle can
    afford. Returns (O [len(rows), d], LSE [len(rows)]) in float64.
    """
    qh = np.asarray(q[b, h], dtype=np.float64)
    kh = np.asarray(k[b, h], dtype=np.float64)
    vh = np.asarray(v[b, h], dtype=np.float64)
    d = qh.shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    return _head(qh, kh, vh, causal, scale, np.asarray(rows))


def softmax_probs(q, k, causal=False, scale=None):
    """The materialised probability matrix P = softmax(S) of one head [N, N].

    Exposed only so tests can check invariants of the definition itself
    (rows of P sum to one, masked entries are zero).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    if scale is None:
        scale = 1.0 / np.sqrt(q.shape[-1])
    s = _logits(q, k, scale, causal, np.arange(q.shape[0]))
    m = np.max(s, axis=1, keepdims=True)
    p = np.exp(s - m)
    return p / np.sum(p, axis=1, keepdims=True)
