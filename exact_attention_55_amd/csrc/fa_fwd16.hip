// fa_fwd16.hip - fused attention forward for bf16 / fp16 inputs on gfx950.
//
// Method (cited from the pages by title and section):
//  * "FlashAttention - one, two, three!" (Medium), "FlashAttention v1.": Q, K
//    and V are processed block by block in one fused kernel; exponentials are
//    taken without the softmax denominator, which is tracked per row (l)
//    together with the running row maximum.
//  * same page, "FlashAttention v2.": the output is accumulated unnormalised
//    and divided by l once, at the end; work is split over batch, heads and
//    query blocks (one workgroup per query tile of one head).
//  * "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
//    Low-Precision", "New GPU Features on Hopper": the two GEMMs run on the
//    matrix cores, the softmax in fp32.
//
// gfx950 mapping:
//  * Workgroup = NW waves, each wave owns QW = 32*QB query rows. The wave
//    keeps its Q rows in registers as MFMA B operands for the whole kernel.
//  * K and V tiles of BC keys are staged global -> registers -> LDS, double
//    buffered: tile j+1 is fetched from HBM while tile j is computed, with one
//    workgroup barrier per tile.
//  * Scores are computed transposed, S^T = K Q^T, with 32x32x16 MFMA: each
//    lane then owns one query (column) and 16 keys per 32-key block, so the
//    row max and row sum are mostly lane-local; the two half-waves that share
//    a query combine with one cross-lane exchange.
//  * The output is also accumulated transposed, O^T += V^T P^T: the B operand
//    P^T comes straight from the S^T accumulators (no shuffles) and the
//    rescale by the per-query factor is lane-local. The rows of K fed to the
//    score MFMA are permuted within each 32-key block (bits 2 and 3 of the
//    row index swapped) so that every lane's P^T slots cover 8 consecutive
//    keys; V^T fragments then come from LDS with transposing reads.
//  * Softmax in the base-2 domain: p = exp2(s*c - m), c = scale*log2(e),
//    hardware v_exp_f32. The reference maximum m is only moved when a tile's
//    row maximum exceeds it by more than TAU (p then stays <= 2^TAU), which
//    skips almost all rescales of the O accumulators; the result is the same
//    exact softmax up to rounding because l and O use the same m.
//  * Two row sums: l~ from the rounded P actually fed to the PV MFMA (dot2
//    with ones) normalises O, which makes O an exact convex combination of V
//    rows even when one key dominates; l from the fp32 p gives the
//    log-sum-exp, free of the 16-bit rounding of P.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr float kTau = 8.0f;      // lazy-rescale threshold (log2 units)

template <typename T> __device__ __forceinline__ typename Elt<T>::x2 pack2(float a, float b);
template <> __device__ __forceinline__ bf16x2 pack2<__bf16>(float a, float b) {
    bf16x2 r = {(__bf16)a, (__bf16)b};
    return r;
}
template <> __device__ __forceinline__ f16x2 pack2<_Float16>(float a, float b) {
    f16x2 r = {(_Float16)a, (_Float16)b};
    return r;
}
// x.x + x.y + acc in fp32 (v_dot2 with ones)
__device__ __forceinline__ float sum2(bf16x2 x, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(x, one, acc, false);
}
__device__ __forceinline__ float sum2(f16x2 x, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(x, one, acc, false);
}

// Tile configuration per head dimension. NW waves per workgroup, each owning
// 32*QB query rows; BC keys per K/V tile; WPE = waves per SIMD the register
// budget is sized for (2: 256 registers per wave, so two waves share a SIMD
// and one wave's softmax overlaps the other's MFMAs).
#ifndef FA16_CFG_64
#define FA16_CFG_64 8, 1, 128, 2
#endif
#ifndef FA16_CFG_128
#define FA16_CFG_128 4, 1, 64, 2
#endif
#ifndef FA16_CFG_256
#define FA16_CFG_256 4, 1, 64, 1
#endif
template <int NW_, int QB_, int BC_, int WPE_> struct CfgT {
    static constexpr int NW = NW_, QB = QB_, BC = BC_, WPE = WPE_;
};
template <int D> struct Cfg16;
template <> struct Cfg16<64> : CfgT<FA16_CFG_64> {};
template <> struct Cfg16<128> : CfgT<FA16_CFG_128> {};
template <> struct Cfg16<256> : CfgT<FA16_CFG_256> {};

// Per-wave running state of the online softmax.
template <typename T, int D, int QB>
struct RowState {
    f32x16 o[QB][D / 32];     // O^T accumulators (unnormalised)
    float m[QB];              // reference maximum, log2 units
    float l[QB];              // sum of the rounded P fed to the MFMA
    float lx[QB];             // sum of the fp32 p (for the log-sum-exp)
};

// One K/V tile for one wave: S^T = K Q^T, optional mask, online softmax
// update, O^T += V^T P^T. MASK handles the ragged last tile and the causal
// diagonal; the main loop instantiates it without.
template <typename T, int D, int QB, int BC, bool CAUSAL, bool MASK>
__device__ __forceinline__ void tile_step(RowState<T, D, QB>& st,
                                          const typename Elt<T>::x8 (&qf)[QB][D / 16],
                                          const T* kl, const T* vl, int k_off, int v_off,
                                          int k0, int q0, int N, int hi, int l32, float c)
{
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    constexpr int KS = D + 8, VS = D + 16;
    constexpr int NCH = D / 16, NDB = D / 32, NKB = BC / 32, NPV = BC / 16;

    f32x16 s[QB][NKB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const X8 a = load16<X8>(kl + k_off + 32 * kb * KS + 16 * ch);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(a, qf[qb][ch], s[qb][kb]);
        }
    }
    if (MASK) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q = q0 + 32 * qb + l32;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int key = k0 + key_of(kb, r, hi);
                    if (key >= N || (CAUSAL && key > q)) s[qb][kb][r] = -INFINITY;
                }
        }
    }
    float mt[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        float mx = s[qb][0][0];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
        mx = fmaxf(mx, xor32(mx));
        mt[qb] = mx * c;
        need |= mt[qb] > st.m[qb] + kTau;
    }
    if (wave_any(need)) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mnew = fmaxf(st.m[qb], mt[qb]);
            const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(st.m[qb] - mnew);
            st.m[qb] = mnew;
            st.l[qb] *= alpha;
            st.lx[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) st.o[qb][db] *= alpha;
        }
    }
    X8 pf[QB][NPV];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float nm = -st.m[qb];
        float ls = st.l[qb], lx = st.lx[qb];
#pragma unroll
        for (int t = 0; t < NPV; ++t) {
            const int kb = t >> 1, r0 = 8 * (t & 1);
            X2 pp[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float p0 = exp2_hw(fmaf(s[qb][kb][r0 + 2 * j], c, nm));
                const float p1 = exp2_hw(fmaf(s[qb][kb][r0 + 2 * j + 1], c, nm));
                pp[j] = pack2<T>(p0, p1);
                ls = sum2(pp[j], ls);
                lx += p0;
                lx += p1;
            }
            pf[qb][t] = X8{pp[0][0], pp[0][1], pp[1][0], pp[1][1],
                           pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
        }
        st.l[qb] = ls;
        st.lx[qb] = lx;
    }
#pragma unroll
    for (int t = 0; t < NPV; ++t) {
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            const T* vp = vl + v_off + 16 * t * VS + 32 * db;
            const u32x2 lo = lds_read_tr16(vp);
            const u32x2 hi4 = lds_read_tr16(vp + 4 * VS);
            const X8 a = __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) st.o[qb][db] = mfma32(a, pf[qb][t], st.o[qb][db]);
        }
    }
}

template <typename T, int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(Cfg16<D>::NW * 64, Cfg16<D>::WPE)
fa_fwd16_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                void* __restrict__ Og, float* __restrict__ LSEg, int N, int num_qtiles,
                int num_blocks, float c)
{
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    constexpr int NW = Cfg16<D>::NW, QB = Cfg16<D>::QB, BC = Cfg16<D>::BC;
    constexpr int QW = 32 * QB;            // query rows per wave
    constexpr int BR = NW * QW;            // query rows per workgroup
    constexpr int KS = D + 8;              // LDS row stride of K (elements)
    constexpr int VS = D + 16;             // LDS row stride of V (elements)
    constexpr int KT = BC * KS, VT = BC * VS;
    constexpr int NCH = D / 16;
    constexpr int NDB = D / 32;
    constexpr int NT = NW * 64;
    constexpr int CPR = D / 8;             // 16-byte chunks per row
    constexpr int CPT = BC * CPR / NT;     // chunks per thread per tile
    static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");
    static_assert(BC % 32 == 0, "key tile is a multiple of 32");

    __shared__ __attribute__((aligned(16))) T smem[2 * (KT + VT)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    // Workgroup -> (head, query tile). Consecutive workgroups land on
    // different XCDs; regroup so each XCD walks whole heads (K/V of a head
    // then stay in that XCD's L2). Causal: heaviest query tiles first.
    int bid = blockIdx.x;
    if ((num_blocks & 7) == 0) bid = (bid & 7) * (num_blocks >> 3) + (bid >> 3);
    const int bh = bid / num_qtiles;
    int qt = bid - bh * num_qtiles;
    if (CAUSAL) qt = num_qtiles - 1 - qt;

    const size_t head = (size_t)bh * N * D;
    const T* Q = Qg + head;
    const T* K = Kg + head;
    const T* V = Vg + head;
    const int qtile0 = qt * BR;
    const int q0 = qtile0 + wave * QW;

    // Q^T fragments (B operand): lane holds query q0+32*qb+l32, d = 16*ch + 8*hi .. +7
    X8 qf[QB][NCH];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = q0 + 32 * qb + l32;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            if (row < N)
                qf[qb][ch] = load16<X8>(Q + (size_t)row * D + 16 * ch + 8 * hi);
            else
                qf[qb][ch] = __builtin_bit_cast(X8, u32x4{0, 0, 0, 0});
        }
    }

    // Key tiles [0, nfull) need no mask for any wave of the workgroup; tiles
    // [nfull, nkt) cross the causal diagonal or the end of the sequence.
    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const int nkt = (kend + BC - 1) / BC;
    const int nfull = (CAUSAL ? min(qtile0 + 1, N) : N) / BC;

    RowState<T, D, QB> st;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        st.m[qb] = -INFINITY;
        st.l[qb] = 0.f;
        st.lx[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) st.o[qb][db] = f32x16{};
    }

    u32x4 kst[CPT], vst[CPT];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / CPR, ch = idx % CPR;
            const int key = kt * BC + r;
            if (key < N) {
                kst[i] = *reinterpret_cast<const u32x4*>(K + (size_t)key * D + ch * 8);
                vst[i] = *reinterpret_cast<const u32x4*>(V + (size_t)key * D + ch * 8);
            } else {
                kst[i] = u32x4{0, 0, 0, 0};
                vst[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto swrite = [&](int buf) {
        T* kl = smem + buf * (KT + VT);
        T* vl = kl + KT;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / CPR, ch = idx % CPR;
            *reinterpret_cast<u32x4*>(kl + r * KS + ch * 8) = kst[i];
            *reinterpret_cast<u32x4*>(vl + r * VS + ch * 8) = vst[i];
        }
    };

    // per-lane LDS offsets
    const int k_off = krow_perm(l32) * KS + 8 * hi;                        // + 32*kb*KS + 16*ch
    const int v_off = (8 * hi + (lane & 15) / 4) * VS + 16 * (l32 / 16) + 4 * (lane & 3);

    gload(0);
    swrite(0);
    __syncthreads();

    int kt = 0;
    for (; kt < nfull; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        const T* kl = smem + buf * (KT + VT);
        tile_step<T, D, QB, BC, CAUSAL, false>(st, qf, kl, kl + KT, k_off, v_off, kt * BC, q0, N,
                                               hi, l32, c);
        if (kt + 1 < nkt) swrite(buf ^ 1);
        __syncthreads();
    }
    for (; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        const T* kl = smem + buf * (KT + VT);
        const int k0 = kt * BC;
        if (!CAUSAL || k0 <= q0 + QW - 1)       // wave has a visible key in this tile
            tile_step<T, D, QB, BC, CAUSAL, true>(st, qf, kl, kl + KT, k_off, v_off, k0, q0, N,
                                                  hi, l32, c);
        if (kt + 1 < nkt) swrite(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l~, LSE = ln2 * (m + log2 l) ----
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = st.l[qb] + xor32(st.l[qb]);
        const float lx = st.lx[qb] + xor32(st.lx[qb]);
        const float inv = 1.0f / l;
        const int row = q0 + 32 * qb + l32;
        if (row < N) {
            if (hi == 0) LSEg[(size_t)bh * N + row] = (st.m[qb] + __builtin_amdgcn_logf(lx)) * kLn2;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int dcol = 32 * db + 8 * j + 4 * hi;
                    const size_t off = head + (size_t)row * D + dcol;
                    const float v0 = st.o[qb][db][4 * j] * inv, v1 = st.o[qb][db][4 * j + 1] * inv;
                    const float v2 = st.o[qb][db][4 * j + 2] * inv, v3 = st.o[qb][db][4 * j + 3] * inv;
                    if (OUT_F32) {
                        *reinterpret_cast<f32x4*>(static_cast<float*>(Og) + off) = f32x4{v0, v1, v2, v3};
                    } else {
                        const X2 a = pack2<T>(v0, v1), b = pack2<T>(v2, v3);
                        *reinterpret_cast<u32x2*>(static_cast<T*>(Og) + off) =
                            u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
                    }
                }
            }
        }
    }
}

template <typename T, int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    constexpr int BR = Cfg16<D>::NW * 32 * Cfg16<D>::QB;
    const int num_qtiles = (a.N + BR - 1) / BR;
    const long long nblk = (long long)num_qtiles * a.B * a.H;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((fa_fwd16_kernel<T, D, CAUSAL, OUT_F32>), dim3((unsigned)nblk),
                       dim3(Cfg16<D>::NW * 64), 0, s, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.o, a.lse, a.N,
                       num_qtiles, (int)nblk, c);
    return hipGetLastError();
}

template <typename T, int D>
static hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    if (a.causal)
        return a.out_f32 ? launch_t<T, D, true, true>(a, s) : launch_t<T, D, true, false>(a, s);
    return a.out_f32 ? launch_t<T, D, false, true>(a, s) : launch_t<T, D, false, false>(a, s);
}

template <typename T>
static hipError_t launch_ty(const FwdArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return launch_d<T, 64>(a, s);
        case 128: return launch_d<T, 128>(a, s);
        case 256: return launch_d<T, 256>(a, s);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t s) {
    return bf16 ? launch_ty<__bf16>(a, s) : launch_ty<_Float16>(a, s);
}

}  // namespace fa
