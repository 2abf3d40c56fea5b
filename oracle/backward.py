"""Gradients of exact attention in float64 (test infrastructure only).

The pages treat the backward pass only through recomputation: the attention
probabilities are not stored but recomputed from the per-row constants kept
in global memory ("FlashAttention - one, two, three!" (Medium), section
"FlashAttention v1."), and the FlashAttention-3 review ("FlashAttention-3:
почему внимание стало быстрее", section «Ограничения») notes that the paper
benchmarks both directions. The gradient itself is the plain chain rule
through the "Standard Attention" definition (same Medium page) of
O = softmax(scale * Q K^T) V, written out here with the probabilities
materialised:

    S  = scale * Q K^T        (causal: -inf where key j > query i)
    P  = row softmax of S
    dV = P^T dO
    dP = dO V^T
    D_i = sum_j P_ij dP_ij  (= sum_c dO_ic O_ic)
    dS = P * (dP - D)       (elementwise, D broadcast along each row)
    dQ = scale * dS K
    dK = scale * dS^T Q

Layout reading as for the forward: [B, H, N, d] tensors.
"""

import numpy as np


def _probs(q, k, scale, causal):
    """Row softmax of scale * Q K^T for one head (float64)."""
    s = scale * (q @ k.T)
    if causal:
        n = q.shape[0]
        s[np.arange(n)[None, :] > np.arange(n)[:, None]] = -np.inf
    s = s - np.max(s, axis=1, keepdims=True)
    p = np.exp(s)
    return p / np.sum(p, axis=1, keepdims=True)


def attention_delta(o, do):
    """D = rowsum(dO * O) over the last axis, float64 [B, H, N]."""
    return np.sum(np.asarray(do, np.float64) * np.asarray(o, np.float64), axis=-1)


def attention_backward(q, k, v, do, causal=False, scale=None):
    """(dQ, dK, dV) of L = sum(O * dO) for O = attention(q, k, v), float64.

    q, k, v, do: [B, H, N, d]. The whole N x N probability matrix of one head
    is materialised (keep N modest).
    """
    q, k, v, do = (np.asarray(t, dtype=np.float64) for t in (q, k, v, do))
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    dq = np.empty_like(q)
    dk = np.empty_like(k)
    dv = np.empty_like(v)
    for b in range(B):
        for h in range(H):
            p = _probs(q[b, h], k[b, h], scale, causal)
            dv[b, h] = p.T @ do[b, h]
            dp = do[b, h] @ v[b, h].T
            dsum = np.sum(p * dp, axis=1, keepdims=True)
            ds = p * (dp - dsum)
            dq[b, h] = scale * (ds @ k[b, h])
            dk[b, h] = scale * (ds.T @ q[b, h])
    return dq, dk, dv
