"""Blockwise online-softmax emulator in float64 (test infrastructure only).

Follows "FlashAttention - one, two, three!" (Medium):
* section "FlashAttention v1.": the fused kernel walks blocks of K and V,
  exponentiates logits without the softmax denominator, and keeps the
  denominator l per row separately;
* section "FlashAttention v2.": the output is accumulated unnormalised and
  rescaled once, at the end, by the per-row normalisation constants.

The formulas are missing from the page text; the recurrence used here is the
plainest reading of those two sections. For each key block (any order):
    m_new = max(m, rowmax(S_blk))
    alpha = exp(m - m_new)            (0 when m = -inf)
    P     = exp(S_blk - m_new)
    l     = alpha * l + rowsum(P)
    o     = alpha * o + P V_blk
and at the end O = o / l, LSE = m + ln l.

The emulator exists to pin that recurrence: tests require it to equal the
naive definition in attention.py to ~1e-12 for many block sizes and visit
orders (including ragged last blocks and reverse order). The GPU kernels do
not use this file.
"""

import numpy as np


def attention_online(q, k, v, causal=False, scale=None, block_q=64, block_k=64,
                     order="forward"):
    """Online-softmax attention over key blocks.

    order: "forward" visits key blocks 0, 1, ...; "reverse" visits them last
    to first; "shuffle" visits them in a fixed pseudo-random order.
    Returns (O [B, H, N, d], LSE [B, H, N]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    o_all = np.zeros((B, H, N, v.shape[-1]))
    lse_all = np.zeros((B, H, N))
    nkb = (N + block_k - 1) // block_k
    if order == "forward":
        visit = list(range(nkb))
    elif order == "reverse":
        visit = list(range(nkb))[::-1]
    elif order == "shuffle":
        visit = list(np.random.default_rng(12345).permutation(nkb))
    else:
        raise ValueError(order)
    for b in range(B):
        for h in range(H):
            for q0 in range(0, N, block_q):
                qi = np.arange(q0, min(N, q0 + block_q))
                m = np.full(len(qi), -np.inf)
                l = np.zeros(len(qi))
                acc = np.zeros((len(qi), v.shape[-1]))
                for kb in visit:
                    kj = np.arange(kb * block_k, min(N, (kb + 1) * block_k))
                    if causal and kj[0] > qi[-1]:
                        continue                      # block wholly above the diagonal
                    s = scale * (q[b, h, qi] @ k[b, h, kj].T)
                    if causal:
                        s[kj[None, :] > qi[:, None]] = -np.inf
                    m_new = np.maximum(m, np.max(s, axis=1))
                    # rows that have seen no visible key yet keep m = -inf
                    seen = np.isfinite(m_new)
                    alpha = np.where(seen & np.isfinite(m), np.exp(m - np.where(seen, m_new, 0.0)), 0.0)
                    p = np.where(seen[:, None], np.exp(s - np.where(seen, m_new, 0.0)[:, None]), 0.0)
                    l = alpha * l + np.sum(p, axis=1)
                    acc = alpha[:, None] * acc + p @ v[b, h, kj]
                    m = m_new
                o_all[b, h, qi] = acc / l[:, None]
                lse_all[b, h, qi] = m + np.log(l)
    return o_all, lse_all
