// fa_fp8_prep.hip - incoherent processing + FP8 e4m3 block quantisation.
//
// Sources: "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
// Low-Precision", section "Incoherent Processing for FP8 Accuracy" (multiply
// Q and K by a random orthogonal matrix per head, realised as a Hadamard
// transform with random signs in O(d log d)); review "FlashAttention-3: почему
// внимание стало быстрее", section "Метод", item 3 (block quantisation, one
// scale per block).
//
// One workgroup per (head, 128-row block); with the rotary step, per 128-row
// block of up to four consecutive heads, whose rows share their cosines and
// sines (computed once, while the first head's loads are in flight). A row
// of d elements is spread over d/8 lanes, 8 contiguous elements per lane (one
// 16-byte load). The Sylvester
// Walsh-Hadamard butterflies of span 1, 2, 4 run inside a lane, spans 8 .. d/2
// across lanes (xor-partner exchange). The block is held in registers until
// its amax is known, so the input is read once and the codes written once,
// with streaming (nontemporal) stores: the codes are not read again by this
// kernel, and keeping them out of the way in the caches measured 15 % faster
// for three [4,16,4096,128] tensors (2 % at [8,16,8192,128]).
//
// y is the row after the optional rotary step and transform, times the
// caller's prescale (1 by default; Q for the fp8 forward's multiply-free
// logits carries softmax_scale * log2(e) this way).
// Per block: amax = max |y|, scale = amax / 448 (IEEE float32 division; 1 if
// amax is 0), code = e4m3 round-to-nearest-even of y / scale after clamping to
// +-448 (the clamp only absorbs the rounding of the scale). After the
// Hadamard, y / scale is taken as y times the rounded 1 / scale (see the
// quantisation loop).
//
// Rotary embedding (ROPE 1: pairs (2i, 2i+1); ROPE 2: pairs (i, i + d/2)):
// the same section notes that the Hadamard step is fused into the rotary
// step, both being memory-bound passes over Q and K. Before the signs, each
// pair (a, b) of the row at position p = pos0 + row turns into
// (a c - b s, a s + b c), c and s the float32 cosine and sine of the float32
// product p * w_i; the frequencies w_i = base^(-2i/d) are rounded to float32
// on the host and passed by value. Interleaved pairs sit inside a lane. For
// the half pairing a lane holds columns 4j .. 4j+3 and d/2 + 4j .. +3 (two
// 8-byte loads) instead of 8j .. 8j+7, so both members of a pair are in
// the lane too. The Hadamard stages are the same code in either layout:
// the in-lane butterfly across elements e, e+4 then works on column bit
// log2(d)-1 instead of bit 2, and since the Sylvester matrix is a Kronecker
// product over the column bits, the order of the stages does not matter.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr float kE4M3Max = 448.0f;
constexpr int kPrepThreads = 256;

// Value of x held by lane (l ^ M). Distances inside a row of 16 lanes go
// through DPP moves (VALU): xor 1 and 2 are quad permutations; xor 4 is the
// half-row mirror (l ^ 7) followed by the quad reversal (^ 3); xor 8 is the
// row mirror (l ^ 15) followed by the half-row mirror (^ 7). Longer
// distances use the LDS permute.
template <int M>
__device__ __forceinline__ float lane_xor(float x) {
    const int v = __float_as_int(x);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0xB1, 0xF, 0xF, true));
    if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(v, 0x4E, 0xF, 0xF, true));
    if constexpr (M == 4) {
        const int h = __builtin_amdgcn_mov_dpp(v, 0x141, 0xF, 0xF, true);
        return __int_as_float(__builtin_amdgcn_mov_dpp(h, 0x1B, 0xF, 0xF, true));
    }
    if constexpr (M == 8) {
        const int r = __builtin_amdgcn_mov_dpp(v, 0x140, 0xF, 0xF, true);
        return __int_as_float(__builtin_amdgcn_mov_dpp(r, 0x141, 0xF, 0xF, true));
    }
    if constexpr (M >= 16) return __shfl_xor(x, M, 64);
}

// sin and cos of a float32 angle t, |t| < 2^25. Reduction t = k (pi/2) + r
// in double precision with pi/2 split into two doubles (the error of r is far
// below a float32 ulp even for k near 2^24), then the Taylor series of sin
// and cos on |r| <= pi/4 in float32 (truncation below 2e-9), and the
// quadrant k mod 4 selects and signs the pair.
__device__ __forceinline__ void sincos_f32(float t, float* sn, float* cs) {
    constexpr double kPio2Hi = 1.5707963267948966;          // nearest double to pi/2
    constexpr double kPio2Lo = 6.123233995736766e-17;       // pi/2 - kPio2Hi
    constexpr double k2OverPi = 0.63661977236758134;
    const double td = (double)t;
    const double k = __builtin_rint(td * k2OverPi);
    const double rd = __builtin_fma(-k, kPio2Lo, __builtin_fma(-k, kPio2Hi, td));
    const float r = (float)rd;
    const float r2 = r * r;
    // sin r = r (1 - r^2/3! + r^4/5! - r^6/7! + r^8/9!); the next term,
    // r^11/11!, is below 2e-9 on |r| <= pi/4
    float ps = 1.0f / 362880.0f;
    ps = fmaf(ps, r2, -1.0f / 5040.0f);
    ps = fmaf(ps, r2, 1.0f / 120.0f);
    ps = fmaf(ps, r2, -1.0f / 6.0f);
    const float s0 = fmaf(r * r2, ps, r);
    // cos r = 1 - r^2/2! + r^4/4! - ... - r^10/10!; the next term, r^12/12!,
    // is below 2e-10 on |r| <= pi/4
    float pc = -1.0f / 3628800.0f;
    pc = fmaf(pc, r2, 1.0f / 40320.0f);
    pc = fmaf(pc, r2, -1.0f / 720.0f);
    pc = fmaf(pc, r2, 1.0f / 24.0f);
    pc = fmaf(pc, r2, -0.5f);
    const float c0 = fmaf(r2, pc, 1.0f);
    const int q = (int)(long long)k & 3;
    const float a = (q & 1) ? c0 : s0;      // sin for q = 0, 2; cos for q = 1, 3
    const float b = (q & 1) ? s0 : c0;
    *sn = (q & 2) ? -a : a;
    *cs = ((q + 1) & 2) ? -b : b;           // cos negated for q = 1, 2
}

// Microscaling exponent of a block with maximum magnitude a: floor(log2 a)
// minus 8 (the exponent of 448, the largest e4m3 normal), clamped to the
// E8M0 range [-127, 127]; -127 for a = 0 or a subnormal a (the block then
// quantises to zeros). floor(log2 a) of a normal float is its biased
// exponent field minus 127.
__device__ __forceinline__ int mx_exponent(float a) {
    const int field = (__float_as_int(a) >> 23) & 0xff;
    if (field == 0) return -127;
    const int e = field - 127 - 8;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ float to_f(__bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f(_Float16 x) { return (float)x; }

// Two floats -> two e4m3 bytes (round to nearest even), in the low 16 bits.
__device__ __forceinline__ uint32_t e4m3x2(float a, float b) {
    a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
    b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xffffu;
}

// MODE 0: per-block scales, quantise and store codes + scale.
// MODE 1: only reduce amax of the whole tensor into *gamax (atomic max on the
//         float bit pattern; amax >= 0 so integer order equals float order).
// MODE 2: quantise with the tensor-wide scale from *gamax, store codes only.
// MODE 3: microscaling along d: one power-of-two scale per 32 columns of a
//         row (4 lanes), stored as the E8M0 byte e + 127 at
//         scales[row of the tensor][column block] (see mx_exponent).
// Threads per 128-row block: 512 at d = 256 (8 passes of 16 rows) and with
// the rotary step (4 passes of 32 rows at d = 128), so a thread's rows in
// flight and the sine / cosine temporaries stay within a register budget
// that leaves several waves per SIMD to hide memory latency; 256 otherwise.
#ifndef FA_PREP_POW2_MUL            // 0: always divide by a block scale without the Hadamard
#define FA_PREP_POW2_MUL 1
#endif
#ifndef FA_PREP_WIDE                // 1: 512 threads at d = 128 without the rotary step too
#define FA_PREP_WIDE 0
#endif
template <int D, int ROPE = 0> constexpr int quant_threads() {
    return (D == 256 || (D == 128 && (ROPE != 0 || FA_PREP_WIDE))) ? 512 : kPrepThreads;
}

// Scale of a block with largest magnitude amax: amax / 448 in float32 (1 for
// an all-zero block), with pow2 rounded up to the next power of two (exact:
// frexp splits s = m 2^e with m in [0.5, 1); s is already one when m = 0.5).
// Block scales that are powers of two let the fp8 forward apply V's scales
// exactly inside the PV product.
__device__ __forceinline__ float block_scale(float amax, int pow2) {
    const float s = amax > 0.f ? amax / kE4M3Max : 1.0f;
    if (!pow2 || __builtin_amdgcn_frexp_mantf(s) == 0.5f) return s;
    return __builtin_amdgcn_ldexpf(1.0f, __builtin_amdgcn_frexp_expf(s));
}

// One workgroup's share of the prep: workgroup index bid of a grid over
// (head, 128-row block). HB heads per workgroup (rotary step: the same
// 128-row block of HB consecutive heads, which share every row's cosines and
// sines).
template <typename T, int D, bool HAD, int MODE, int ROPE, int HB = 1>
__device__ __forceinline__ void
quant_rows(const T* __restrict__ X, uint8_t* __restrict__ X8, const int8_t* __restrict__ signs,
           float* __restrict__ scales, unsigned* __restrict__ gamax, int N, int H, int nblk,
           const RopeFreqs& rf, int pow2, float prescale, int bid)
{
    constexpr int NT = quant_threads<D, ROPE>();
    constexpr int LPR = D / 8;                 // lanes per row
    constexpr int RPP = NT / LPR;              // rows per pass
    constexpr int NPASS = kQuantBlockRows / RPP;
    static_assert(HB == 1 || ROPE != 0, "several heads per workgroup only share rotary terms");
    // one reduction buffer per head of the workgroup (a buffer is not
    // written again before every wave has read it)
    __shared__ float red[HB][NT / 64];

    // SPLIT: elements 0..3 of lane j are columns 4j.., elements 4..7 columns
    // d/2 + 4j.. (the half pairing); otherwise columns 8j .. 8j+7.
    constexpr bool SPLIT = ROPE == 2;
    static_assert(!(SPLIT && MODE == 3), "microscaling takes contiguous columns");
    const int tid = threadIdx.x;
    const int j = tid % LPR, rp = tid / LPR;
    const int c0 = SPLIT ? 4 * j : 8 * j, c1 = SPLIT ? D / 2 + 4 * j : 8 * j + 4;
    const int blk = bid % nblk;
    // rotary terms of the thread's rows, computed once for the HB heads
    float rsn[ROPE != 0 ? NPASS : 1][4], rcs[ROPE != 0 ? NPASS : 1][4];
    bool rope_ready = false;
#pragma unroll 1
    for (int hh = 0; hh < HB; ++hh) {
        const int bh = (bid / nblk) * HB + hh;
        const int gslot = bh * nblk + blk;            // scale slot of this (head, block)
        const int h = bh % H;
        const size_t head = (size_t)bh * N * D;

        float sg[8];
        if (HAD) {
            const uint32_t w0 = *reinterpret_cast<const uint32_t*>(signs + (size_t)h * D + c0);
            const uint32_t w1 = *reinterpret_cast<const uint32_t*>(signs + (size_t)h * D + c1);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sg[e] = (float)(int8_t)((w0 >> (8 * e)) & 0xff);
                sg[e + 4] = (float)(int8_t)((w1 >> (8 * e)) & 0xff);
            }
        }

        // All of the thread's row loads are issued before any is used, so they
        // are in flight together (one at a time leaves each waiting a full
        // memory latency).
        // Rows past the end read the head's last row (always valid, N >= 1) and
        // are zeroed, so the loads carry no branch.
        u32x4 raw[NPASS];
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int row = blk * kQuantBlockRows + p * RPP + rp;
            const T* xr = X + head + (size_t)min(row, N - 1) * D;
            if constexpr (SPLIT) {
                const u32x2 lo = *reinterpret_cast<const u32x2*>(xr + c0);
                const u32x2 hi = *reinterpret_cast<const u32x2*>(xr + c1);
                raw[p] = u32x4{lo[0], lo[1], hi[0], hi[1]};
            } else {
                raw[p] = *reinterpret_cast<const u32x4*>(xr + c0);
            }
        }
#pragma unroll
        for (int p = 0; p < NPASS; ++p)
            if (blk * kQuantBlockRows + p * RPP + rp >= N) raw[p] = u32x4{0, 0, 0, 0};
        // while the loads are in flight: the rotary terms (first head only)
        if (ROPE != 0 && !rope_ready) {
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const float pos = (float)(rf.pos0 + blk * kQuantBlockRows + p * RPP + rp);
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    sincos_f32(pos * rf.w[4 * j + k], &rsn[p][k], &rcs[p][k]);
                }
            }
            rope_ready = true;
        }
        float v[NPASS][8];
        float amax = 0.f;
#pragma unroll
        for (int p = 0; p < NPASS; ++p) {
            const int row = blk * kQuantBlockRows + p * RPP + rp;
            typedef __attribute__((ext_vector_type(8))) T T8;
            const T8 x = __builtin_bit_cast(T8, raw[p]);
#pragma unroll
            for (int e = 0; e < 8; ++e) v[p][e] = to_f(x[e]);
            if (ROPE != 0) {
                if (ROPE == 1) {
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float sn = rsn[p][k], cs = rcs[p][k];
                        const float a = v[p][2 * k], b = v[p][2 * k + 1];
                        v[p][2 * k] = a * cs - b * sn;
                        v[p][2 * k + 1] = a * sn + b * cs;
                    }
                } else {
                    // pairs (4j + k, d/2 + 4j + k) are elements k, k + 4
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        const float sn = rsn[p][k], cs = rcs[p][k];
                        const float a = v[p][k], b = v[p][k + 4];
                        v[p][k] = a * cs - b * sn;
                        v[p][k + 4] = a * sn + b * cs;
                    }
                }
            }
            if (HAD) {
#pragma unroll
                for (int e = 0; e < 8; ++e) v[p][e] *= sg[e];
                // in-lane butterflies, spans 1, 2, 4
#pragma unroll
                for (int span = 1; span < 8; span *= 2)
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        if ((e & span) == 0) {
                            const float a = v[p][e], b = v[p][e + span];
                            v[p][e] = a + b;
                            v[p][e + span] = a - b;
                        }
                // cross-lane butterflies, spans 8 .. D/2 (partner lane j ^ m)
                static_for<0, 5>([&](auto mc) {
                    constexpr int m = 1 << decltype(mc)::value;
                    if constexpr (m < LPR) {
                        const bool upper = (j & m) != 0;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            const float other = lane_xor<m>(v[p][e]);
                            v[p][e] = upper ? (other - v[p][e]) : (v[p][e] + other);
                        }
                    }
                });
                const float rs = 1.0f / __builtin_sqrtf((float)D);
#pragma unroll
                for (int e = 0; e < 8; ++e) v[p][e] *= rs;
            }
            // the prescale: its own float32 multiply of the rotated value
#pragma unroll
            for (int e = 0; e < 8; ++e) v[p][e] *= prescale;
            if (row < N) {
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[p][e]));
            }
        }

        if (MODE == 3) {
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int row = blk * kQuantBlockRows + p * RPP + rp;
                float la = 0.f;
#pragma unroll
                for (int e = 0; e < 8; ++e) la = fmaxf(la, fabsf(v[p][e]));
                la = fmaxf(la, lane_xor<1>(la));
                la = fmaxf(la, lane_xor<2>(la));
                const int ex = mx_exponent(la);
                if (row < N) {
                    uint32_t w[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const float* x = &v[p][4 * h];
                        w[h] = e4m3x2(__builtin_ldexpf(x[0], -ex), __builtin_ldexpf(x[1], -ex)) |
                               (e4m3x2(__builtin_ldexpf(x[2], -ex), __builtin_ldexpf(x[3], -ex)) << 16);
                    }
                    __builtin_nontemporal_store(u32x2{w[0], w[1]},
                                                reinterpret_cast<u32x2*>(X8 + head + (size_t)row * D + 8 * j));
                    if ((j & 3) == 0)
                        reinterpret_cast<uint8_t*>(scales)[((size_t)bh * N + row) * (D / 32) + j / 4] =
                            (uint8_t)(ex + 127);
                }
            }
            return;
        }

        if (MODE != 2) {
            // workgroup amax
#pragma unroll
            for (int m = 32; m >= 1; m /= 2) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
            if ((tid & 63) == 0) red[hh][tid >> 6] = amax;
            __syncthreads();
            amax = red[hh][0];
#pragma unroll
            for (int w = 1; w < NT / 64; ++w) amax = fmaxf(amax, red[hh][w]);
        }
        if (MODE == 1) {
            if (tid == 0) atomicMax(gamax, __float_as_uint(amax));
            continue;
        }
        if (MODE == 2) amax = __uint_as_float(*gamax);

        const float scale = block_scale(amax, pow2);
        if (MODE == 0 && tid == 0) scales[gslot] = scale;
        // x / scale. Without the Hadamard this is the IEEE division, so the codes
        // equal those of the same float32 steps exactly. With it, the values
        // already carry float32 butterfly rounding (a code next to an e4m3
        // rounding boundary may land on the neighbouring one either way), and a
        // multiply by the rounded reciprocal, at most one float32 ulp away, adds
        // only more of the same; it replaces ~10 instructions per element in a
        // kernel that is VALU-bound with the transform.
        // A normal power-of-two scale (pow2 scales, mostly) has an exact
        // reciprocal, and x * (1 / scale) is then the division itself.
        const float inv = 1.0f / scale;
        auto store_codes = [&](auto qs) {
#pragma unroll
            for (int p = 0; p < NPASS; ++p) {
                const int row = blk * kQuantBlockRows + p * RPP + rp;
                if (row < N) {
                    const uint32_t w0 = e4m3x2(qs(v[p][0]), qs(v[p][1])) |
                                        (e4m3x2(qs(v[p][2]), qs(v[p][3])) << 16);
                    const uint32_t w1 = e4m3x2(qs(v[p][4]), qs(v[p][5])) |
                                        (e4m3x2(qs(v[p][6]), qs(v[p][7])) << 16);
                    uint8_t* xr = X8 + head + (size_t)row * D;
                    if constexpr (SPLIT) {
                        __builtin_nontemporal_store(w0, reinterpret_cast<uint32_t*>(xr + c0));
                        __builtin_nontemporal_store(w1, reinterpret_cast<uint32_t*>(xr + c1));
                    } else {
                        __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(xr + c0));
                    }
                }
            }
        };
#if FA_PREP_POW2_MUL
        const bool exact_inv = __builtin_amdgcn_frexp_mantf(scale) == 0.5f && scale >= 0x1p-126f;
#else
        const bool exact_inv = false;
#endif
        if (HAD || exact_inv)
            store_codes([&](float x) { return x * inv; });
        else
            store_codes([&](float x) { return x / scale; });
    }   // heads of the workgroup
}

template <typename T, int D, bool HAD, int MODE, int ROPE, int HB = 1>
__global__ void __launch_bounds__((quant_threads<D, ROPE>()))
fp8_prep_kernel(const T* __restrict__ X, uint8_t* __restrict__ X8, const int8_t* __restrict__ signs,
                float* __restrict__ scales, unsigned* __restrict__ gamax, int N, int H, int nblk,
                RopeFreqs rf, int pow2, float prescale)
{
    quant_rows<T, D, HAD, MODE, ROPE, HB>(X, X8, signs, scales, gamax, N, H, nblk, rf, pow2, prescale,
                                          blockIdx.x);
}

// Q, K and V of one attention call in a single launch: workgroups
// [0, grid1) take Q (the transform when signs is given, times q_prescale),
// [grid1, 2 grid1) K (the same transform), the rest V (no transform); all
// with power-of-two block scales. Each workgroup runs the same steps as in
// fp8_prep_kernel, so the codes and scales are those of three separate
// preps; one launch three times the size leaves a smaller share of the time
// to the last, partly filled round of workgroups.
template <typename T, int D>
__global__ void __launch_bounds__((quant_threads<D, 0>()))
fp8_prep_qkv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                    uint8_t* __restrict__ Q8, uint8_t* __restrict__ K8, uint8_t* __restrict__ V8,
                    const int8_t* __restrict__ signs, size_t scales_off, int N, int H, int nblk,
                    int grid1, float q_prescale)
{
    const int t = blockIdx.x / grid1, bid = blockIdx.x - t * grid1;
    const T* X = t == 0 ? Q : t == 1 ? K : V;
    uint8_t* X8 = t == 0 ? Q8 : t == 1 ? K8 : V8;
    float* scales = reinterpret_cast<float*>(X8 + scales_off);
    const float prescale = t == 0 ? q_prescale : 1.0f;
    const RopeFreqs rf{};
    if (t < 2 && signs != nullptr)
        quant_rows<T, D, true, 0, 0>(X, X8, signs, scales, nullptr, N, H, nblk, rf, 1, prescale, bid);
    else
        quant_rows<T, D, false, 0, 0>(X, X8, nullptr, scales, nullptr, N, H, nblk, rf, 1, prescale, bid);
}

// Microscaling along the sequence (V): one wave per 32-row block. Lane
// (q, cg) owns 8 adjacent columns (cg) of rows q R .. q R + R - 1 of the
// block, R = 32 / (64 / (D / 8)) (8 rows at d = 128), so one load
// instruction of the wave reads 64 / (D / 8) whole rows; the column maxima
// of the block combine over the lanes that share cg (lane xor over the
// higher lane bits), then each lane writes the codes of its rows. Rows past
// the head's end are neither read nor written. The block's scale for column
// c is stored at byte (c % 32) * (D / 32) + c / 32 of the block's D scale
// bytes, the order in which a lane of the PV matrix instruction wants its
// column scales. gb: the (head, block) index of this wave.
template <typename T, int D>
__device__ __forceinline__ void mx_cols_block(const T* __restrict__ X, uint8_t* __restrict__ X8,
                                              uint8_t* __restrict__ scales, int N, int nkb, long long gb)
{
    constexpr int CG = D / 8;                      // column groups of a block
    constexpr int RQ = 64 / CG;                    // row groups (lanes per column group)
    constexpr int R = 32 / RQ;                     // rows per lane
    const int lane = threadIdx.x & 63;
    const int cg = lane % CG, rq = lane / CG;
    const long long bh = gb / nkb;
    const int r0 = (int)(gb - bh * nkb) * 32;
    const int nr = min(32, N - r0);
    const size_t base = ((size_t)bh * N + r0 + rq * R) * D + 8 * cg;
    typedef __attribute__((ext_vector_type(8))) T T8;
    u32x4 raw[R];
#pragma unroll
    for (int r = 0; r < R; ++r)
        raw[r] = rq * R + r < nr ? *reinterpret_cast<const u32x4*>(X + base + (size_t)r * D) : u32x4{0, 0, 0, 0};
    float a[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = 0.f;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const T8 x = __builtin_bit_cast(T8, raw[r]);
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] = fmaxf(a[e], fabsf(to_f(x[e])));
    }
    static_for<0, 3>([&](auto mc) {
        constexpr int m = CG << decltype(mc)::value;
        if constexpr (m < 64) {
#pragma unroll
            for (int e = 0; e < 8; ++e) a[e] = fmaxf(a[e], lane_xor<m>(a[e]));
        }
    });
    int ex[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ex[e] = mx_exponent(a[e]);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        if (rq * R + r < nr) {
            const T8 x = __builtin_bit_cast(T8, raw[r]);
            float y[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) y[e] = __builtin_ldexpf(to_f(x[e]), -ex[e]);
            const uint32_t w0 = e4m3x2(y[0], y[1]) | (e4m3x2(y[2], y[3]) << 16);
            const uint32_t w1 = e4m3x2(y[4], y[5]) | (e4m3x2(y[6], y[7]) << 16);
            __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(X8 + base + (size_t)r * D));
        }
    }
    if (rq == 0) {
        uint8_t* sc = scales + (size_t)gb * D;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int col = 8 * cg + e;
            sc[(col % 32) * (D / 32) + col / 32] = (uint8_t)(ex[e] + 127);
        }
    }
}

template <typename T, int D>
__global__ void __launch_bounds__(kPrepThreads)
mx_prep_cols_kernel(const T* __restrict__ X, uint8_t* __restrict__ X8, uint8_t* __restrict__ scales,
                    int N, int nkb, long long nblocks)
{
    const long long gb = (long long)blockIdx.x * (kPrepThreads / 64) + (threadIdx.x >> 6);
    if (gb >= nblocks) return;
    mx_cols_block<T, D>(X, X8, scales, N, nkb, gb);
}

// The microscaled Q, K and V of one attention call in a single launch:
// workgroups [0, grid1) take Q (along d: the transform when signs is given,
// times q_prescale), [grid1, 2 grid1) K (the same transform), the rest V
// (along the sequence, one wave per 32-row block). Each workgroup runs the
// steps of the single-tensor kernels, so the outputs are theirs byte for
// byte.
template <typename T, int D>
__global__ void __launch_bounds__((quant_threads<D, 0>()))
mx_prep_qkv_kernel(const T* __restrict__ Q, const T* __restrict__ K, const T* __restrict__ V,
                   uint8_t* __restrict__ Q8, uint8_t* __restrict__ K8, uint8_t* __restrict__ V8,
                   const int8_t* __restrict__ signs, size_t scales_off, int N, int H, int nblk,
                   int grid1, int nkb, long long nvblocks, float q_prescale)
{
    constexpr int NT = quant_threads<D, 0>();
    const int bid = blockIdx.x;
    if (bid >= 2 * grid1) {
        const long long gb = (long long)(bid - 2 * grid1) * (NT / 64) + (threadIdx.x >> 6);
        if (gb < nvblocks) mx_cols_block<T, D>(V, V8, V8 + scales_off, N, nkb, gb);
        return;
    }
    const int t = bid / grid1, b = bid - t * grid1;
    const T* X = t == 0 ? Q : K;
    uint8_t* X8 = t == 0 ? Q8 : K8;
    float* scales = reinterpret_cast<float*>(X8 + scales_off);
    const float prescale = t == 0 ? q_prescale : 1.0f;
    const RopeFreqs rf{};
    if (signs != nullptr)
        quant_rows<T, D, true, 3, 0>(X, X8, signs, scales, nullptr, N, H, nblk, rf, 0, prescale, b);
    else
        quant_rows<T, D, false, 3, 0>(X, X8, nullptr, scales, nullptr, N, H, nblk, rf, 0, prescale, b);
}

__global__ void zero_u32_kernel(unsigned* p) { *p = 0u; }

// One workgroup: read the tensor-wide amax first, then fill every slot.
__global__ void __launch_bounds__(1024) fill_scales_kernel(float* scales, const unsigned* gamax,
                                                           long long n, int pow2) {
    __shared__ float sc;
    if (threadIdx.x == 0) sc = block_scale(__uint_as_float(*gamax), pow2);
    __syncthreads();
    const float s = sc;
    for (long long i = threadIdx.x; i < n; i += blockDim.x) scales[i] = s;
}

template <typename T, int D, bool HAD, int ROPE>
static hipError_t prep_t(const PrepArgs& a, hipStream_t s) {
    const int nblk = (a.N + kQuantBlockRows - 1) / kQuantBlockRows;
    const long long grid = (long long)a.B * a.H * nblk;
    float* scales = reinterpret_cast<float*>(a.x8 + a.scales_off);
    const T* x = static_cast<const T*>(a.x);
    if (a.mx == kMxAlongN) {
        const int nkb = (a.N + 31) / 32;
        const long long nblocks = (long long)a.B * a.H * nkb;
        constexpr int BPW = kPrepThreads / 64;
        hipLaunchKernelGGL((mx_prep_cols_kernel<T, D>), dim3((unsigned)((nblocks + BPW - 1) / BPW)),
                           dim3(kPrepThreads), 0, s, x, a.x8, a.x8 + a.scales_off, a.N, nkb, nblocks);
        return hipGetLastError();
    }
    if (a.mx == kMxAlongD) {
        if constexpr (ROPE != 0) return hipErrorInvalidValue;     // fa_mx_prep has no rotary step
        hipLaunchKernelGGL((fp8_prep_kernel<T, D, HAD, 3, 0>), dim3((unsigned)grid),
                           dim3(quant_threads<D, 0>()), 0, s, x, a.x8, a.signs, scales, nullptr, a.N, a.H, nblk,
                           a.rope, a.pow2, a.prescale);
        return hipGetLastError();
    }
    if (a.block_rows != 0) {
        // The rotary step: four (else two) heads per workgroup share the
        // cosines and sines of its rows (heads of a workgroup are consecutive
        // in [B][H] order, so B*H must divide evenly), as long as that leaves
        // at least 512 workgroups (fewer starve the memory system: small
        // shapes keep one head each). Measured on B=4 H=16 N=4096 d=128:
        // 1.53x the plain prep's time with one head per workgroup, 1.30x
        // with two, 1.23x with four.
        const long long heads = (long long)a.B * a.H;
        if (ROPE != 0 && heads % 4 == 0 && grid / 4 >= 512)
            hipLaunchKernelGGL((fp8_prep_kernel<T, D, HAD, 0, ROPE, ROPE != 0 ? 4 : 1>), dim3((unsigned)(grid / 4)),
                               dim3(quant_threads<D, ROPE>()), 0, s, x, a.x8, a.signs, scales, nullptr, a.N,
                               a.H, nblk, a.rope, a.pow2, a.prescale);
        else if (ROPE != 0 && heads % 2 == 0 && grid / 2 >= 512)
            hipLaunchKernelGGL((fp8_prep_kernel<T, D, HAD, 0, ROPE, ROPE != 0 ? 2 : 1>), dim3((unsigned)(grid / 2)),
                               dim3(quant_threads<D, ROPE>()), 0, s, x, a.x8, a.signs, scales, nullptr, a.N,
                               a.H, nblk, a.rope, a.pow2, a.prescale);
        else
            hipLaunchKernelGGL((fp8_prep_kernel<T, D, HAD, 0, ROPE>), dim3((unsigned)grid),
                               dim3(quant_threads<D, ROPE>()), 0, s, x, a.x8, a.signs, scales, nullptr, a.N,
                               a.H, nblk, a.rope, a.pow2, a.prescale);
        return hipGetLastError();
    }
    // Per-tensor: the first scale slot serves as the amax accumulator; the
    // fill kernel reads it before overwriting every slot.
    unsigned* gamax = reinterpret_cast<unsigned*>(scales);
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(1), 0, s, gamax);
    hipLaunchKernelGGL((fp8_prep_kernel<T, D, HAD, 1, ROPE>), dim3((unsigned)grid), dim3(quant_threads<D, ROPE>()),
                       0, s, x, a.x8, a.signs, scales, gamax, a.N, a.H, nblk, a.rope, a.pow2, a.prescale);
    hipLaunchKernelGGL((fp8_prep_kernel<T, D, HAD, 2, ROPE>), dim3((unsigned)grid), dim3(quant_threads<D, ROPE>()),
                       0, s, x, a.x8, a.signs, scales, gamax, a.N, a.H, nblk, a.rope, a.pow2, a.prescale);
    hipLaunchKernelGGL(fill_scales_kernel, dim3(1), dim3(1024), 0, s, scales,
                       (const unsigned*)gamax, grid, a.pow2);
    return hipGetLastError();
}

template <typename T, int D, int ROPE>
static hipError_t prep_r(const PrepArgs& a, hipStream_t s) {
    return a.signs ? prep_t<T, D, true, ROPE>(a, s) : prep_t<T, D, false, ROPE>(a, s);
}

template <typename T, int D>
static hipError_t prep_d(const PrepArgs& a, hipStream_t s) {
    switch (a.rope_style) {
        case 1: return prep_r<T, D, 1>(a, s);
        case 2: return prep_r<T, D, 2>(a, s);
    }
    return prep_r<T, D, 0>(a, s);
}

template <typename T>
static hipError_t prep_ty(const PrepArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return prep_d<T, 64>(a, s);
        case 128: return prep_d<T, 128>(a, s);
        case 256: return prep_d<T, 256>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fp8_prep(const PrepArgs& a, hipStream_t s) {
    return a.bf16 ? prep_ty<__bf16>(a, s) : prep_ty<_Float16>(a, s);
}

template <typename T, int D>
static hipError_t prep_qkv_d(const PrepQkvArgs& a, hipStream_t s) {
    const int nblk = (a.N + kQuantBlockRows - 1) / kQuantBlockRows;
    const long long grid1 = (long long)a.B * a.H * nblk;
    hipLaunchKernelGGL((fp8_prep_qkv_kernel<T, D>), dim3((unsigned)(3 * grid1)), dim3(quant_threads<D, 0>()),
                       0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                       static_cast<const T*>(a.v), a.q8, a.k8, a.v8, a.signs, a.scales_off, a.N, a.H, nblk,
                       (int)grid1, a.q_prescale);
    return hipGetLastError();
}

template <typename T>
static hipError_t prep_qkv_ty(const PrepQkvArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return prep_qkv_d<T, 64>(a, s);
        case 128: return prep_qkv_d<T, 128>(a, s);
        case 256: return prep_qkv_d<T, 256>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fp8_prep_qkv(const PrepQkvArgs& a, hipStream_t s) {
    return a.bf16 ? prep_qkv_ty<__bf16>(a, s) : prep_qkv_ty<_Float16>(a, s);
}

template <typename T, int D>
static hipError_t mx_prep_qkv_d(const PrepQkvArgs& a, hipStream_t s) {
    constexpr int NT = quant_threads<D, 0>();
    const int nblk = (a.N + kQuantBlockRows - 1) / kQuantBlockRows;
    const long long grid1 = (long long)a.B * a.H * nblk;
    const int nkb = (a.N + 31) / 32;
    const long long nvblocks = (long long)a.B * a.H * nkb;
    const long long gridv = (nvblocks + NT / 64 - 1) / (NT / 64);
    hipLaunchKernelGGL((mx_prep_qkv_kernel<T, D>), dim3((unsigned)(2 * grid1 + gridv)), dim3(NT), 0, s,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.q8, a.k8, a.v8, a.signs, a.scales_off, a.N, a.H, nblk, (int)grid1, nkb, nvblocks,
                       a.q_prescale);
    return hipGetLastError();
}

template <typename T>
static hipError_t mx_prep_qkv_ty(const PrepQkvArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return mx_prep_qkv_d<T, 64>(a, s);
        case 128: return mx_prep_qkv_d<T, 128>(a, s);
        case 256: return mx_prep_qkv_d<T, 256>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_mx_prep_qkv(const PrepQkvArgs& a, hipStream_t s) {
    return a.bf16 ? mx_prep_qkv_ty<__bf16>(a, s) : mx_prep_qkv_ty<_Float16>(a, s);
}

}  // namespace fa
