"""Rotary position embedding (RoPE) in float64 (test infrastructure only).

Source: "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
Low-Precision" (Embodied AI 101 transcript), section "Incoherent Processing
for FP8 Accuracy": rotary embeddings are a memory-bound step before attention,
and the random-sign Hadamard rotation is fused into it at no extra cost. The
pages give no formula for the rotary step itself.

Readings (listed in the design notes):
* each row of q or k at sequence position p = pos0 + n (n = row index) has
  its coordinates paired and every pair (a, b) rotated by the angle
  p * w_i: (a, b) -> (a cos - b sin, a sin + b cos), with w_i = base^(-2i/d)
  for pair i = 0 .. d/2 - 1 and base 10000 unless given;
* two pairings: "interleaved" pairs coordinates (2i, 2i+1), the original
  rotary formulation; "half" pairs (i, i + d/2), the layout many models use;
* precision: w_i is rounded once to float32, the angle is the float32
  product float32(p) * w_i (rounded to float32), its cosine and sine are
  taken exactly and rounded to float32; the rotation itself is float64. The
  GPU keeps w, the angle and cos/sin in float32, so both sides rotate by the
  same float32 angle and differ only by the last-bit rounding of cos/sin and
  of the products.
"""

import numpy as np

STYLES = ("interleaved", "half")


def rope_frequencies(d, base=10000.0):
    """w_i = base^(-2i/d) for i < d/2, rounded to float32."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * i / d).astype(np.float32)


def rope_angles(N, d, base=10000.0, pos0=0):
    """float32 angles [N, d/2]: float32(p) * w_i rounded to float32."""
    pos = (pos0 + np.arange(N)).astype(np.float32)
    return (pos[:, None] * rope_frequencies(d, base)[None, :]).astype(np.float32)


def rope_cos_sin(N, d, base=10000.0, pos0=0):
    """cos and sin of the float32 angles, each rounded to float32, [N, d/2]."""
    ang = rope_angles(N, d, base, pos0).astype(np.float64)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def rope(x, style="interleaved", base=10000.0, pos0=0):
    """Rotate rows of x [..., N, d] by their positions; returns float64."""
    if style not in STYLES:
        raise ValueError(f"unknown rotary style {style!r}")
    x = np.asarray(x, dtype=np.float64)
    N, d = x.shape[-2], x.shape[-1]
    if d % 2:
        raise ValueError("rotary embedding needs an even head dimension")
    c, s = (t.astype(np.float64) for t in rope_cos_sin(N, d, base, pos0))
    y = np.empty_like(x)
    if style == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
        y[..., 0::2] = a * c - b * s
        y[..., 1::2] = a * s + b * c
    else:
        h = d // 2
        a, b = x[..., :h], x[..., h:]
        y[..., :h] = a * c - b * s
        y[..., h:] = a * s + b * c
    return y
