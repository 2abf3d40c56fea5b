"""Exact attention for decode-shaped inputs, in float64 (test infrastructure
only; the GPU library never calls it).

Decode is the same function as the naive oracle, applied where a few new
query rows attend to a long key/value history: "FlashAttention-3: Fast &
Accurate Attention with Asynchrony & Low-Precision" (Embodied AI 101
transcript), section "Performance Results", names autoregressive sampling as
a use; "FlashAttention - one, two, three!" (Medium), section "Standard
Attention", gives the computation (logits, row softmax, weighted sum of value
rows). Nothing in it depends on N_q == N_k.

Readings where the pages are silent (listed in the design notes):
* layout q [B, H, Nq, d]; k, v [B, Hkv, Nk, d] with H a multiple of Hkv and
  query head h reading key/value head h // (H / Hkv) (Hkv == H is the pages'
  case; fewer key/value heads shared by groups of query heads is accepted as
  well);
* per-batch key counts L_b <= Nk (``seqlens_k``): keys L_b .. Nk-1 of batch b
  are not part of the sequence;
* causal with Nq <= L_b aligns the query rows with the last keys: query i
  sees key j iff j <= L_b - Nq + i (for Nq == Nk == L_b this is the
  forward's j <= i);
* a row with no visible key (L_b == 0, or causal with L_b - Nq + i < 0) has
  O = 0 and LSE = -inf.
"""

import numpy as np


def visible_keys(L, Nq, i, causal):
    """Number of keys query row i sees: keys 0 .. n-1 (n may be 0)."""
    if causal:
        return max(0, min(L, L - Nq + i + 1))
    return L


def attention_decode(q, k, v, causal=False, scale=None, seqlens_k=None):
    """O [B, H, Nq, d] and LSE [B, H, Nq] (float64) of decode-shaped attention."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, Nq, d = q.shape
    Hkv, Nk = k.shape[1], k.shape[2]
    if H % Hkv:
        raise ValueError("H must be a multiple of Hkv")
    group = H // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    lens = [Nk] * B if seqlens_k is None else [int(x) for x in seqlens_k]
    o = np.zeros((B, H, Nq, v.shape[-1]), dtype=np.float64)
    lse = np.full((B, H, Nq), -np.inf, dtype=np.float64)
    for b in range(B):
        L = lens[b]
        if not 0 <= L <= Nk:
            raise ValueError("seqlens_k out of range")
        for h in range(H):
            kh, vh = k[b, h // group], v[b, h // group]
            for i in range(Nq):
                n = visible_keys(L, Nq, i, causal)
                if n == 0:
                    continue
                s = scale * (kh[:n] @ q[b, h, i])         # logits of the visible keys
                m = np.max(s)
                p = np.exp(s - m)
                l = np.sum(p)
                o[b, h, i] = (p @ vh[:n]) / l
                lse[b, h, i] = m + np.log(l)
    return o, lse
