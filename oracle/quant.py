"""FP8 block quantisation with optional incoherent processing (test infra only).

Sources:
* "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
  Low-Precision" (Embodied AI 101 transcript), section "Incoherent Processing
  for FP8 Accuracy": rotate Q and K by a random-sign Hadamard matrix per head
  before quantising, which spreads outliers across the head dimension.
* review "FlashAttention-3: почему внимание стало быстрее", section "Метод",
  item 3: one scale per block instead of one per tensor (block quantisation).
* same review, section "Результаты" (Table 3 discussion): the comparator is a
  baseline FP8 attention; read here as plain per-tensor scaling, no rotation.

Readings (the pages give no block shape, scale rule or rounding):
* a block is 128 consecutive rows of one (b, h) head, all d columns; the last
  block of a head may be shorter;
* per-tensor mode (block_rows == 0) uses one scale for the whole [B,H,N,d]
  tensor;
* scale = amax / 448 in float32; an all-zero block gets scale 1;
* optionally (pow2, the form used for V) that scale is rounded up to the
  next power of two, 2^ceil(log2(amax / 448)). e4m3 is a floating-point
  grid, so a power-of-two scale loses no relative precision on normal values
  (the largest code then lies in [224, 448]); what it buys is that ratios
  of block scales are powers of two, which a matrix product applies exactly
  through an E8M0 scale byte;
* code = e4m3 round-to-nearest-even, saturating, of x / scale;
* dequantised value = decode(code) * scale.
* optionally (prescale = p, the form the fp8 forward reads without a
  multiply per score when p = softmax_scale * log2(e)) the rotated float32
  values are multiplied by p in float32 before the block maximum, so the
  codes and scales represent x * p; with p a power of two this only moves
  every scale by p.

Precision of the integer decision: the rotated value is formed in float64
(the definition) and then rounded once to float32, the precision the GPU works
in; amax, scale and x / scale are float32 operations (IEEE division, correctly
rounded), so a GPU path that reproduces the float32 steps takes the same
rounding decision. The only freedom left to the GPU is the float32 rounding of
its own Hadamard butterflies, which can move a value across an e4m3 rounding
boundary when it lies within a few float32 ulps of one.
"""

import numpy as np

from .fp8 import E4M3_MAX, e4m3_encode, e4m3_decode
from .hadamard import random_sign_hadamard
from .rope import rope as rotary


def _rotated_f32(x, signs, rope=None, prescale=None):
    """The values that get quantised: x, optionally after the rotary
    embedding (rope = (style, base, pos0)), then x M when signs are given,
    rounded once to float32; with prescale, then times prescale in float32."""
    x = np.asarray(x, dtype=np.float64)
    if rope is not None:
        x = rotary(x, *rope)
    if signs is not None:
        x = random_sign_hadamard(x, signs)
    y = x.astype(np.float32)
    if prescale is not None:
        y = (y * np.float32(prescale)).astype(np.float32)
    return y


def pow2_ceil_f32(s):
    """Smallest power of two >= s for float32 s > 0 (exact, subnormals
    included), as float32."""
    s = np.asarray(s, dtype=np.float32)
    m, e = np.frexp(s)                          # s = m 2^e, m in [0.5, 1)
    up = np.ldexp(np.float32(1.0), e).astype(np.float32)
    return np.where(m == 0.5, s, up).astype(np.float32)


def fp8_quantize(x, signs=None, block_rows=128, rope=None, pow2=False, prescale=None):
    """Quantise x [B, H, N, d] to e4m3 codes with float32 scales.

    signs: [H, d] of +-1 to apply the random-sign Hadamard first (Q and K), or
    None (V, and the plain baseline).
    block_rows: rows per block (128), or 0 for one scale per tensor.
    rope: None, or (style, base, pos0) to apply the rotary embedding first
    (the fused rotary + Hadamard + quantisation step).
    pow2: round each scale up to a power of two (pow2_ceil_f32).
    prescale: None, or a float32 factor applied to the rotated values before
    the block maximum (the result then represents x * prescale).
    Returns (codes uint8 [B,H,N,d], scales float32 [B,H,ceil(N/block_rows)];
    per-tensor mode returns the same scale in every slot of a
    [B,H,ceil(N/128)] array so both modes have one layout).
    """
    y = _rotated_f32(x, signs, rope, prescale)
    B, H, N, d = y.shape
    br = block_rows if block_rows > 0 else 128
    nb = (N + br - 1) // br
    scales = np.empty((B, H, nb), dtype=np.float32)
    if block_rows == 0:
        amax = np.max(np.abs(y)) if y.size else np.float32(0)
        s = np.float32(amax) / np.float32(E4M3_MAX) if amax > 0 else np.float32(1.0)
        scales[...] = pow2_ceil_f32(s) if pow2 else s
    else:
        for j in range(nb):
            blk = np.abs(y[:, :, j * br:(j + 1) * br, :])
            amax = np.max(blk, axis=(2, 3)).astype(np.float32)
            s = amax / np.float32(E4M3_MAX)                       # float32 division
            s = np.where(amax > 0, s, np.float32(1.0))
            scales[:, :, j] = pow2_ceil_f32(s) if pow2 else s
    row_scale = np.repeat(scales, br, axis=2)[:, :, :N]           # [B,H,N]
    q = (y / row_scale[..., None]).astype(np.float32)             # float32 division
    codes = e4m3_encode(q.astype(np.float64))
    return codes, scales


def fp8_dequantize(codes, scales, block_rows=128):
    """decode(code) * scale, float64, inverse layout of fp8_quantize."""
    br = block_rows if block_rows > 0 else 128
    N = codes.shape[2]
    row_scale = np.repeat(np.asarray(scales, dtype=np.float64), br, axis=2)[:, :, :N]
    return e4m3_decode(codes) * row_scale[..., None]


def fake_quant_attention(q, k, v, signs=None, block_rows=128, causal=False,
                         scale=None, rope=None, v_pow2=True, prescaled=False):
    """Exact float64 attention on the dequantised fp8 inputs.

    Q and K are rotated by the same random-sign Hadamard (when signs is given)
    and quantised; V is quantised without rotation. Because the rotation is
    orthogonal, the attention of the rotated, unquantised inputs equals the
    plain attention; what remains is the quantisation error alone. This is the
    reference for the fp8 kernel's log-sum-exp (which never sees the rounding
    of P) and a diagnostic for its output. With rope = (style, base, pos0)
    Q and K get the rotary embedding before the rotation and quantisation.
    v_pow2: V's block scales are powers of two (the form the fp8 forward
    applies exactly).
    prescaled: Q is quantised as x * p, p = float32(scale * log2(e)), and Q
    and K with power-of-two scales, so the dequantised logits Q K^T are
    already base-2 exponents; the attention of the dequantised tensors then
    takes the softmax scale ln(2) (exp(ln2 * t) = 2^t).
    Returns (O, LSE, (qc, qs), (kc, ks), (vc, vs)).
    """
    from .attention import attention
    d = np.asarray(q).shape[-1]
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    pq = np.float32(scale * np.log2(np.e)) if prescaled else None
    qc, qs = fp8_quantize(q, signs, block_rows, rope, pow2=prescaled, prescale=pq)
    kc, ks = fp8_quantize(k, signs, block_rows, rope, pow2=prescaled)
    vc, vs = fp8_quantize(v, None, block_rows, pow2=v_pow2)
    o, lse = attention(fp8_dequantize(qc, qs, block_rows),
                       fp8_dequantize(kc, ks, block_rows),
                       fp8_dequantize(vc, vs, block_rows), causal,
                       np.log(2.0) if prescaled else scale)
    return o, lse, (qc, qs), (kc, ks), (vc, vs)
