/*
 * fa.h - C ABI of libfa.so, the MI355X (gfx950) fused exact-attention forward.
 *
 * The operation is exact softmax attention per (batch, head):
 *     S = softmax_scale * Q K^T,  P = rowsoftmax(S),  O = P V,
 *     LSE_i = ln sum_j exp(S_ij)
 * ("FlashAttention - one, two, three!" (Medium), section "Standard
 * Attention", for S, the softmax and O; section "FlashAttention v1." for
 * keeping only a few per-row constants - here the log-sum-exp - in global
 * memory). The library computes it the fused way: tiles of K and V streamed
 * through on-chip memory, an online softmax with a running row maximum and a
 * separate denominator, and one normalisation at the end (same page,
 * sections "FlashAttention v1." and "FlashAttention v2."); the N x N matrix
 * never reaches device memory.
 *
 * The FP8 path follows "FlashAttention-3: Fast & Accurate Attention with
 * Asynchrony & Low-Precision" (Embodied AI 101 transcript), section
 * "Incoherent Processing for FP8 Accuracy" (random-sign Hadamard rotation of
 * Q and K before quantising) and the review "FlashAttention-3: почему внимание
 * стало быстрее", section "Метод", item 3 (block quantisation; QK^T and PV in
 * FP8, softmax in higher precision).
 *
 * Conventions for every entry point:
 *  - Tensor pointers are DEVICE pointers owned by the caller. The library
 *    allocates no memory, keeps no pointer after returning and holds no
 *    mutable global state; calls on different streams may run concurrently.
 *  - Layout: q, k, v, o are contiguous row-major [B][H][N][d]; lse is
 *    contiguous [B][H][N] float32. Q and K share N (self-attention shape).
 *  - Calls are asynchronous: work is enqueued on `stream` (a hipStream_t;
 *    NULL means the default stream) and the call returns. Faults during
 *    execution surface at the caller's next synchronisation on that stream.
 *  - Every argument is validated before any HIP call is made; a bad argument
 *    returns a status and never aborts. B, H or N equal to 0 is a valid empty
 *    problem and returns FA_OK without launching anything.
 */
#ifndef FA_H
#define FA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes returned by every entry point. */
enum fa_status {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,   /* null/misaligned pointer, bad size or scale   */
    FA_ERR_UNSUPPORTED = 2,   /* valid request the library has no kernel for */
    FA_ERR_HIP = 3,           /* the HIP runtime rejected a launch            */
    FA_ERR_TOO_LARGE = 4      /* request exceeds the fixed scratch of an
                                 allocation-free entry point                  */
};

/* Bytes of the fixed per-device scratch array of fa_fwd_decode_noalloc. */
#define FA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* Element types. FA_OUT_F32 may be OR-ed into fa_fwd's dtype: O is then
 * written as float32 instead of the default (the input type for 16-bit
 * inputs, bfloat16 for FP8 inputs). FA_FWD_PIPELINED may be OR-ed into
 * fa_fwd's dtype: 16-bit inputs at d = 128 run the 64-rows-per-wave kernel
 * that overlaps the next block's score MFMAs, this block's exponentials and
 * the previous block's PV MFMAs inside one wave (same results up to
 * rounding; ignored for other inputs). Without the flag that kernel still
 * runs 16-bit d = 128 forwards with causal = 0 and N >= 8192, where it is
 * the faster one. FA_SCALE_POW2 may be OR-ed into
 * fa_fp8_prep's in_dtype: block scales are rounded up to powers of two.
 * FA_FP8_QSCALED may be OR-ed into fa_fwd's FP8 dtypes: q was prepared with
 * prescale softmax_scale * log2(e) (fa_fp8_prep_scaled, fa_mx_prep_scaled),
 * so the product Q K^T already is the base-2 exponent of the softmax; see
 * fa_fwd. */
enum fa_dtype {
    FA_F16 = 0,
    FA_BF16 = 1,
    FA_FP8_E4M3 = 2,
    FA_FP8_MX = 3,       /* e4m3 with microscaling (fa_mx_prep): q, k along d, v along N */
    FA_OUT_F32 = 0x100,
    FA_SCALE_POW2 = 0x200,
    FA_FWD_PIPELINED = 0x400,
    FA_FP8_QSCALED = 0x800
};

/*
 * fa_fwd - fused attention forward.
 *
 *  q, k, v  16-bit inputs [B][H][N][d] (dtype FA_F16 or FA_BF16), or, with
 *           dtype FA_FP8_E4M3, packed FP8 tensors written by fa_fp8_prep
 *           (e4m3 codes plus per-block float32 scales, see below). For FP8,
 *           q and k must have been prepared with the same sign vectors (or
 *           both without); v without signs. With dtype FA_FP8_MX: q and k
 *           from fa_mx_prep along d, v from fa_mx_prep along N.
 *  o        output [B][H][N][d]: input dtype (16-bit), bfloat16 (FP8), or
 *           float32 when FA_OUT_F32 is set. 16-byte aligned.
 *  lse      output [B][H][N] float32: natural-log log-sum-exp of each row of
 *           softmax_scale * Q K^T over its visible keys. 4-byte aligned.
 *  B, H, N  batch, heads, sequence length (>= 0; B*H*N*d < 2^62).
 *  d        head dimension: 64, 128 or 256.
 *  causal   nonzero: query i sees keys j <= i only.
 *  softmax_scale  finite and > 0 (usually 1/sqrt(d)); multiplies S before the
 *           softmax.
 *  dtype    FA_F16 | FA_BF16 | FA_FP8_E4M3 | FA_FP8_MX, optionally
 *           | FA_OUT_F32, (16-bit inputs) | FA_FWD_PIPELINED and (FP8
 *           inputs) | FA_FP8_QSCALED.
 *  stream   hipStream_t or NULL.
 *
 * FA_FP8_QSCALED (the fp8 forward's fast form, "FlashAttention-3: Fast &
 * Accurate Attention with Asynchrony & Low-Precision", "New GPU Features on
 * Hopper": the exponentials, not the products, bound the FP8 softmax): q's
 * values carry softmax_scale * log2(e) (prepared with that prescale), so
 * the logits reach exp2 straight from the matrix product, which also
 * applies the block scales as E8M0 exponents. softmax_scale is then not
 * used. FA_FP8_E4M3 inputs must have power-of-two block scales (q from
 * fa_fp8_prep_scaled, which always rounds them so; k and v prepared with
 * FA_SCALE_POW2), all normal floats: at d = 128, where the product applies
 * them, the kernel checks the scales of each head and writes NaN to O and
 * lse of the rows of a workgroup whose scales are not (the call still
 * returns FA_OK); at d = 64 and 256 the logits take one multiply-add as
 * without the flag and any scales work. FA_FP8_MX inputs need q from
 * fa_mx_prep_scaled. A q prepared without the prescale gives wrong results
 * that are not detected.
 *
 * q, k, v must be 16-byte aligned (256-byte for the FP8 dtypes). Returns FA_OK, FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED (d not in {64,128,256}, or N*d*2 > 2^31 - 2^16 - 1:
 * one head's K or V must be addressable with 31-bit offsets) or FA_ERR_HIP.
 */
int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
           int B, int H, int N, int d, int causal, float softmax_scale, int dtype,
           void* stream);

/*
 * fa_bwd - gradients dQ, dK, dV of the 16-bit forward.
 *
 * Recomputes the attention probabilities from q, k and the forward's log-sum-
 * exp instead of storing them ("FlashAttention - one, two, three!",
 * "FlashAttention v1.": recomputation for the backward pass); the gradient
 * is the chain rule through softmax(softmax_scale * Q K^T) V:
 *   dV = P^T dO, dP = dO V^T, D = rowsum(dO * O), dS = P * (dP - D),
 *   dQ = softmax_scale * dS K, dK = softmax_scale * dS^T Q.
 *
 *  q, k, v  the forward's 16-bit inputs [B][H][N][d] (dtype FA_F16 or
 *           FA_BF16), 16-byte aligned.
 *  o, lse   the forward's output (same dtype) and log-sum-exp [B][H][N].
 *  dout     gradient of the loss with respect to o, [B][H][N][d], same dtype.
 *  dq, dk, dv  outputs [B][H][N][d]: the input dtype, or float32 when
 *           FA_OUT_F32 is set in dtype. 16-byte aligned.
 *  delta    caller-owned scratch, float32 [2][B][H][N], 16-byte aligned;
 *           overwritten with the per-row constants rowsum(dout * o) and
 *           -lse / softmax_scale.
 *  B, H, N, causal, softmax_scale  as for fa_fwd.
 *  d        64 or 128 (256 returns FA_ERR_UNSUPPORTED).
 *  stream   hipStream_t or NULL.
 *
 * Launches three kernels on stream (D, then dQ, then dK/dV); no atomics, so
 * the result is deterministic. Returns FA_OK, FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta,
           int B, int H, int N, int d, int causal, float softmax_scale, int dtype,
           void* stream);

/*
 * fa_fwd_decode - attention forward for a few query rows per head against a
 * long key/value history (token-by-token generation, "FlashAttention-3: Fast
 * & Accurate Attention with Asynchrony & Low-Precision", "Performance
 * Results"). Same function as fa_fwd ("FlashAttention - one, two, three!",
 * "Standard Attention"); the keys are split over num_splits parts whose
 * partial results are merged by their log-sum-exp (the block-wise softmax
 * of the same page's "FlashAttention v1.", across parts).
 *
 *  q        16-bit queries [B][H][Nq][d] (dtype FA_F16 or FA_BF16).
 *  k, v     keys and values [B][H_kv][Nk][d], same dtype. Query head h reads
 *           key/value head h / (H / H_kv); H_kv == H is plain multi-head.
 *  o        output [B][H][Nq][d]: input dtype, or float32 with FA_OUT_F32.
 *  lse      output [B][H][Nq] float32, natural log; -inf for a row that sees
 *           no key (its o row is then 0).
 *  seqlens_k  device int32 [B]: keys 0 .. seqlens_k[b]-1 of batch b are the
 *           sequence (values are clamped to [0, Nk]); NULL: all Nk keys.
 *  workspace, workspace_bytes  caller-owned device scratch of at least
 *           fa_decode_workspace_bytes(B, H, Nq, d, num_splits) bytes,
 *           16-byte aligned (partial O and LSE per split); may be NULL when
 *           num_splits == 1.
 *  B, H, H_kv, Nq, Nk  >= 0, H a multiple of H_kv (>= 1 when H > 0).
 *  d        64, 128 or 256.
 *  causal   nonzero: the Nq query rows are the last Nq positions of the
 *           sequence: query i sees keys j <= L - Nq + i (L = the sequence's
 *           key count); rows with L - Nq + i < 0 see no key.
 *  softmax_scale  finite and > 0.
 *  num_splits  1 .. 256; fa_decode_splits() suggests one for the shape.
 *  dtype    FA_F16 | FA_BF16, optionally | FA_OUT_F32.
 *  stream   hipStream_t or NULL.
 *
 * q, k, v, o 16-byte aligned, lse and seqlens_k 4-byte aligned. Launches one
 * kernel (num_splits == 1) or two (splits, then the merge). Returns FA_OK,
 * FA_ERR_INVALID_ARG (also for a workspace that is missing or too small),
 * FA_ERR_UNSUPPORTED (d, or Nk*d*2 > 2^31 - 2^16 - 1) or FA_ERR_HIP.
 */
int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* seqlens_k, void* workspace, size_t workspace_bytes,
                  int B, int H, int H_kv, int Nq, int Nk, int d, int causal,
                  float softmax_scale, int num_splits, int dtype, void* stream);

/*
 * fa_fwd_decode_noalloc - fa_fwd_decode for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). Same arguments, kernels and results as
 * fa_fwd_decode, without the workspace: the split partials go to a fixed
 * array of FA_NOALLOC_SCRATCH_BYTES (16 MiB) in device memory, one per GPU
 * the library runs on, held until the process ends. The call makes no
 * hipMalloc or hipFree and calls no allocating library routine; the first
 * call on a device looks up that device's array address once (the device of
 * `stream`, or the current device for NULL).
 *
 * A request whose partials need more than FA_NOALLOC_SCRATCH_BYTES
 * (fa_decode_workspace_bytes(B, H, Nq, d, num_splits) > the limit) returns
 * FA_ERR_TOO_LARGE before any HIP call; num_splits == 1 uses no scratch.
 * Nothing in the array needs clearing between calls: the merge reads only
 * partials the same call's split kernel wrote. Every call on one GPU shares
 * its array, so calls that overlap on one GPU (on different streams, or
 * from different threads) race and give wrong results: serialise them.
 * Returns the statuses of fa_fwd_decode and FA_ERR_TOO_LARGE.
 */
int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* seqlens_k, int B, int H, int H_kv, int Nq, int Nk, int d,
                          int causal, float softmax_scale, int num_splits, int dtype,
                          void* stream);

/* Suggested num_splits for fa_fwd_decode (enough parts to fill the GPU, each
 * at least 256 keys). Returns 1 for invalid or empty shapes. */
int fa_decode_splits(int B, int H, int H_kv, int Nq, int Nk, int d);

/* Workspace bytes fa_fwd_decode needs for num_splits (0 when num_splits <= 1
 * or the arguments are invalid). */
size_t fa_decode_workspace_bytes(int B, int H, int Nq, int d, int num_splits);

/*
 * fa_fp8_prep - incoherent processing + FP8 block quantisation of one tensor.
 *
 *  x        16-bit input [B][H][N][d] (in_dtype FA_BF16 or FA_F16), 16-byte
 *           aligned.
 *  x8       output packed FP8 tensor of fa_fp8_packed_bytes(B,H,N,d) bytes,
 *           256-byte aligned:
 *             bytes [0, B*H*N*d)            e4m3 codes, [B][H][N][d]
 *             at fa_fp8_scales_offset(...)  float32 scales [B][H][ceil(N/128)]
 *  signs    int8 [H][d] of +1/-1: rows are first rotated, x <- x diag(s) H_d
 *           / sqrt(d) (Sylvester Hadamard H_d, same signs for Q and K of a
 *           head). NULL: no rotation (V, or the plain baseline).
 *  block_rows  128: one scale per 128 consecutive rows of a head (the last
 *           block may be shorter); 0: one scale for the whole tensor (the
 *           plain per-tensor baseline; the same scale is stored in every
 *           slot).
 *  in_dtype FA_BF16 or FA_F16, optionally | FA_SCALE_POW2.
 *
 * Per block: amax = max |x|, scale = amax / 448 in float32 (1 when amax is
 * 0); with FA_SCALE_POW2 that scale is rounded up to the next power of two
 * (same relative precision on the e4m3 grid, the largest code then lies in
 * [224, 448]). code = e4m3 round-to-nearest-even of x / scale, saturated to
 * +-448. Prepare V with FA_SCALE_POW2: the fp8 forward then applies V's
 * block scales exactly in the PV product, with P rounded to e4m3 as 8 p;
 * other V scales cost it the extra rounding of 8 p f, f in [1, 2) the
 * significand of the scale's ratio to the head's largest.
 * Without signs x / scale is the IEEE float32 quotient; with them (rotated
 * rows, whose float32 butterfly rounding already differs from an exact
 * transform) it is x times the rounded 1 / scale, at most one float32 ulp
 * from the quotient. d must be 64, 128 or 256. Per-tensor mode launches four
 * kernels (clear, amax, quantise, fill the scale slots) and uses the scale
 * slots as its reduction buffer; the tensor is only valid once the stream
 * reaches the end of the call. Returns FA_OK, FA_ERR_INVALID_ARG,
 * FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_fp8_prep(const void* x, void* x8, const int8_t* signs,
                int B, int H, int N, int d, int block_rows, int in_dtype,
                void* stream);

/*
 * fa_fp8_prep_scaled - fa_fp8_prep_rope with a prescale: the values
 * quantised are (rotary, Hadamard as there) times prescale, multiplied in
 * float32 before the block maximum, so the packed tensor represents
 * x * prescale; block scales are always rounded up to powers of two (the
 * form FA_FP8_QSCALED needs; FA_SCALE_POW2 in in_dtype is accepted and
 * changes nothing). Prepare q for fa_fwd with FA_FP8_QSCALED with
 * prescale = softmax_scale * log2(e).
 *
 *  prescale finite and > 0.
 *  rope_style FA_ROPE_NONE for no rotary step (rope_base and pos0 then
 *           unused); other arguments as for fa_fp8_prep_rope.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_fp8_prep_scaled(const void* x, void* x8, const int8_t* signs,
                       int B, int H, int N, int d, int block_rows, int in_dtype,
                       int rope_style, float rope_base, int pos0, float prescale,
                       void* stream);

/*
 * fa_fp8_prep_qkv - the three preps of one FP8 attention call in a single
 * launch ("FlashAttention-3: Fast & Accurate Attention with Asynchrony &
 * Low-Precision", "Incoherent Processing for FP8 Accuracy" and block
 * quantisation): q with the rotation by signs and prescale q_prescale, k
 * with the same rotation, v without one, all with 128-row blocks and
 * power-of-two scales. The three packed outputs equal, byte for byte, those
 * of fa_fp8_prep_scaled(q, q8, signs, ..., 128, in_dtype, FA_ROPE_NONE, 1,
 * 0, q_prescale), fa_fp8_prep(k, k8, signs, ..., 128, in_dtype |
 * FA_SCALE_POW2) and fa_fp8_prep(v, v8, NULL, ..., 128, in_dtype |
 * FA_SCALE_POW2); one launch three times the size fills the GPU better than
 * three in turn. With q_prescale = qk prescale softmax_scale * log2(e) the
 * outputs are the inputs of fa_fwd with FA_FP8_E4M3 | FA_FP8_QSCALED; with
 * q_prescale = 1 those of the plain FA_FP8_E4M3 forward.
 *
 *  q, k, v     16-bit inputs [B][H][N][d] (in_dtype FA_BF16 or FA_F16,
 *              FA_SCALE_POW2 may be set and changes nothing), 16-byte
 *              aligned.
 *  q8, k8, v8  packed outputs as fa_fp8_prep's x8, each of
 *              fa_fp8_packed_bytes(B,H,N,d) bytes, 256-byte aligned, owned by
 *              the caller; the three must not overlap one another or the
 *              inputs (overlapping outputs are rejected).
 *  signs       int8 [H][d] of +1/-1, or NULL for no rotation of q and k.
 *  q_prescale  finite and > 0.
 *  d           64, 128 or 256; 3 * B * H * ceil(N/128) < 2^31.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_fp8_prep_qkv(const void* q, const void* k, const void* v,
                    void* q8, void* k8, void* v8, const int8_t* signs,
                    int B, int H, int N, int d, int in_dtype, float q_prescale,
                    void* stream);

/* Rotary pairings for fa_fp8_prep_rope. */
enum fa_rope_style {
    FA_ROPE_NONE = 0,
    FA_ROPE_INTERLEAVED = 1,   /* pairs (2i, 2i+1) */
    FA_ROPE_HALF = 2           /* pairs (i, i + d/2) */
};

/*
 * fa_fp8_prep_rope - rotary embedding fused into fa_fp8_prep: the rotary
 * step, the random-sign Hadamard and the FP8 block quantisation of Q or K in
 * one pass over the tensor ("FlashAttention-3: Fast & Accurate Attention
 * with Asynchrony & Low-Precision", "Incoherent Processing for FP8
 * Accuracy": the Hadamard is fused into the memory-bound rotary step).
 *
 * Row n of every head is at position p = pos0 + n; each coordinate pair
 * (a, b) (pairing rope_style) becomes (a cos t - b sin t, a sin t + b cos t)
 * with t = p * w_i, w_i = rope_base^(-2i/d) for pair i < d/2. w_i and t are
 * float32 (w_i rounded once from double precision, t the float32 product),
 * cos t and sin t float32. Then as fa_fp8_prep (signs may be NULL: rotary +
 * quantisation only).
 *
 *  rope_style  FA_ROPE_INTERLEAVED or FA_ROPE_HALF (FA_ROPE_NONE: same as
 *           fa_fp8_prep).
 *  rope_base   finite and > 0 (10000 in most models).
 *  pos0     position of row 0, >= 0; pos0 + N <= 2^24 (positions exact in
 *           float32).
 *  other arguments as for fa_fp8_prep.
 *
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_fp8_prep_rope(const void* x, void* x8, const int8_t* signs,
                     int B, int H, int N, int d, int block_rows, int in_dtype,
                     int rope_style, float rope_base, int pos0, void* stream);

/* Microscaling axis for fa_mx_prep. */
enum fa_mx_axis {
    FA_MX_ALONG_D = 0,   /* one scale per row and 32 columns (Q, K) */
    FA_MX_ALONG_N = 1    /* one scale per column and 32 rows (V) */
};

/*
 * fa_mx_prep - FP8 e4m3 quantisation with microscaling: a power-of-two
 * scale per 32 elements (the finer-grained variant of the block
 * quantisation of "FlashAttention-3: почему внимание стало быстрее", «Метод»
 * item 3, in the OCP MX layout the gfx950 scaled matrix instructions read),
 * after the optional random-sign Hadamard of fa_fp8_prep (Q and K only).
 *
 *  x        16-bit input [B][H][N][d], 16-byte aligned.
 *  x8       output of fa_mx_packed_bytes(B,H,N,d) bytes, 256-byte aligned:
 *             bytes [0, B*H*N*d)            e4m3 codes, [B][H][N][d]
 *             at fa_fp8_scales_offset(...)  E8M0 scale bytes (2^(byte-127)):
 *               FA_MX_ALONG_D: [B][H][N][d/32];
 *               FA_MX_ALONG_N: [B][H][ceil(N/32)][32][d/32], the scale of
 *               column c at [c % 32][c / 32] of its 32-row block.
 *  signs    int8 [H][d] (Hadamard as in fa_fp8_prep) or NULL; must be NULL
 *           for FA_MX_ALONG_N.
 *  axis     FA_MX_ALONG_D (Q, K) or FA_MX_ALONG_N (V).
 *  in_dtype FA_BF16 or FA_F16; d 64, 128 or 256.
 *
 * Per block of 32: e = floor(log2(max |x|)) - 8 clamped to [-127, 127]
 * (-127 for an all-zero block), code = e4m3 round-to-nearest-even of
 * x * 2^-e saturated to +-448, scale byte e + 127. fa_fwd with dtype
 * FA_FP8_MX takes q and k prepared along d and v along N. Returns FA_OK,
 * FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_mx_prep(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
               int axis, int in_dtype, void* stream);

/*
 * fa_mx_prep_scaled - fa_mx_prep along d (axis must be FA_MX_ALONG_D) of
 * x * prescale: the (Hadamard-rotated) float32 values are multiplied by
 * prescale before each block's maximum, so the tensor represents
 * x * prescale. Prepare q for fa_fwd with FA_FP8_MX | FA_FP8_QSCALED with
 * prescale = softmax_scale * log2(e). prescale finite and > 0; other
 * arguments and returns as for fa_mx_prep (FA_ERR_INVALID_ARG for
 * FA_MX_ALONG_N).
 */
int fa_mx_prep_scaled(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
                      int axis, int in_dtype, float prescale, void* stream);

/*
 * fa_mx_prep_qkv - the three microscaled preps of one FA_FP8_MX attention
 * call in a single launch ("FlashAttention-3: Fast & Accurate Attention with
 * Asynchrony & Low-Precision", "Incoherent Processing for FP8 Accuracy",
 * and block quantisation at 32-element blocks): q along d with the rotation
 * by signs and prescale q_prescale, k along d with the same rotation, v
 * along N without one. The three packed outputs equal, byte for byte, those
 * of fa_mx_prep_scaled(q, q8, signs, ..., FA_MX_ALONG_D, in_dtype,
 * q_prescale), fa_mx_prep(k, k8, signs, ..., FA_MX_ALONG_D, in_dtype) and
 * fa_mx_prep(v, v8, NULL, ..., FA_MX_ALONG_N, in_dtype). With q_prescale =
 * softmax_scale * log2(e) the outputs are the inputs of fa_fwd with
 * FA_FP8_MX | FA_FP8_QSCALED; with q_prescale = 1 those of plain FA_FP8_MX.
 *
 *  q, k, v     16-bit inputs [B][H][N][d] (in_dtype FA_BF16 or FA_F16),
 *              16-byte aligned.
 *  q8, k8, v8  packed outputs as fa_mx_prep's x8, each of
 *              fa_mx_packed_bytes(B,H,N,d) bytes, 256-byte aligned, owned by
 *              the caller; the three must not overlap one another or the
 *              inputs (overlapping outputs are rejected).
 *  signs       int8 [H][d] of +1/-1, or NULL for no rotation of q and k.
 *  q_prescale  finite and > 0.
 *  d           64, 128 or 256; 2 * B * H * ceil(N/128) + B * H * ceil(N/32)
 *              < 2^31.
 * Returns FA_OK, FA_ERR_INVALID_ARG, FA_ERR_UNSUPPORTED or FA_ERR_HIP.
 */
int fa_mx_prep_qkv(const void* q, const void* k, const void* v,
                   void* q8, void* k8, void* v8, const int8_t* signs,
                   int B, int H, int N, int d, int in_dtype, float q_prescale,
                   void* stream);

/* Size in bytes of a packed microscaled tensor for [B][H][N][d] (either
 * axis); 0 for invalid sizes. Pure host arithmetic. */
size_t fa_mx_packed_bytes(int B, int H, int N, int d);

/* Size in bytes of a packed FP8 tensor for [B][H][N][d]; 0 for invalid
 * sizes. Pure host arithmetic. */
size_t fa_fp8_packed_bytes(int B, int H, int N, int d);

/* Byte offset of the float32 scales inside a packed FP8 tensor (the codes
 * size rounded up to 256). Pure host arithmetic. */
size_t fa_fp8_scales_offset(int B, int H, int N, int d);

/* Static, human-readable text for a status code. */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_H */
