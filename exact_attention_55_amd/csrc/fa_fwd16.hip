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
//  * K and V tiles of BC keys go straight from global memory into LDS
//    (global_load_lds, 16 bytes per lane, no staging registers), double
//    buffered: tile j+1 is in flight while tile j is computed, with one
//    workgroup barrier per tile. Rows are stored unpadded with their 16-byte
//    chunks XOR-swizzled (see lds_chunk), which keeps both the K fragment
//    reads and the transposing V reads free of bank conflicts.
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

// Per-wave state and per-tile steps. A wave owns 32*QB query rows; a key
// tile has BC keys. Swizzled LDS tiles: see lds_swz16 and the lane offsets ka
// (K fragments) and va (transposing V reads) set up in the kernel.
template <typename T, int D, int QB, int BC>
struct Wave16 {
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    static constexpr int RB = 2 * D;       // bytes per K / V row in LDS
    static constexpr int NCH = D / 16;     // k-steps of S^T = K Q^T
    static constexpr int NDB = D / 32;     // 32-row blocks of O^T
    static constexpr int NKB = BC / 32;    // 32-key blocks of S^T
    static constexpr int NPV = BC / 16;    // k-steps of O^T += V^T P^T

    f32x16 o[QB][NDB];   // O^T accumulators (unnormalised)
    float m[QB];         // reference maximum, log2 units
    float l[QB];         // sum of the rounded P fed to the MFMA
    float lx[QB];        // sum of the fp32 p (for the log-sum-exp)

    __device__ __forceinline__ void init() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            m[qb] = -INFINITY;
            l[qb] = 0.f;
            lx[qb] = 0.f;
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[qb][db] = f32x16{};
        }
    }

    // Distinct swizzled lane offsets: K fragments repeat every NKA k-steps
    // (NKA*32 bytes), V^T fragments every NVA d-blocks (NVA*64 bytes).
    static constexpr int NKA = (D == 64) ? 4 : 8;
    static constexpr int NVA = (D == 64) ? 2 : 4;

    // K fragment (ch, kb): row perm(l32) + 32*kb, logical chunk 2*ch + hi.
    static __device__ __forceinline__ X8 kfrag(const char* kl, const int (&ka)[NKA], int ch, int kb) {
        return load16<X8>(kl + ka[ch % NKA] + NKA * 32 * (ch / NKA) + 32 * kb * RB);
    }

    // S^T for k-steps [c0, c1) with fragments already in registers.
    static __device__ __forceinline__ void qk(f32x16 (&s)[QB][NKB], const X8 (&kf)[NKB][NCH],
                                              const X8 (&qf)[QB][NCH], int c0, int c1) {
#pragma unroll
        for (int ch = c0; ch < c1; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32(kf[kb][ch], qf[qb][ch], s[qb][kb]);
    }

    // Whole score tile: all K fragments requested before the first MFMA.
    static __device__ __forceinline__ void scores(f32x16 (&s)[QB][NKB], const char* kl,
                                                  const int (&ka)[NKA], const X8 (&qf)[QB][NCH]) {
        X8 kf[NKB][NCH];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb][ch] = kfrag(kl, ka, ch, kb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{};
        qk(s, kf, qf, 0, NCH);
    }

    template <bool CAUSAL>
    static __device__ __forceinline__ void mask(f32x16 (&s)[QB][NKB], int k0, int q0, int N, int hi,
                                                int l32) {
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

    // Row maximum of the tile in log2 units: balanced tree over the lane's
    // scores, then the lane pair that shares the query.
    static __device__ __forceinline__ void tile_max(const f32x16 (&s)[QB][NKB], float c,
                                                    float (&mt)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float part[NKB * 4];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int g = 0; g < 4; ++g)
                    part[4 * kb + g] = fmaxf(fmaxf(s[qb][kb][4 * g], s[qb][kb][4 * g + 1]),
                                             fmaxf(s[qb][kb][4 * g + 2], s[qb][kb][4 * g + 3]));
#pragma unroll
            for (int w = NKB * 4; w > 1; w /= 2)
#pragma unroll
                for (int i = 0; i < w / 2; ++i) part[i] = fmaxf(part[i], part[i + w / 2]);
            mt[qb] = pair_max(part[0]) * c;
        }
    }

    // Lazy rescale: the reference maximum moves only when the tile maximum
    // exceeds it by more than kTau (then p <= 2^kTau always holds).
    __device__ __forceinline__ void rescale(const float (&mt)[QB]) {
        bool need = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) need |= mt[qb] > m[qb] + kTau;
        if (wave_any(need)) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float mnew = fmaxf(m[qb], mt[qb]);
                const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(m[qb] - mnew);
                m[qb] = mnew;
                l[qb] *= alpha;
                lx[qb] *= alpha;
#pragma unroll
                for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
            }
        }
    }

    // P for score block kb (16 keys per lane -> two PV operands), with the
    // row sums in independent partial accumulators.
    __device__ __forceinline__ void probs(const f32x16 (&s)[QB][NKB], X8 (&pf)[QB][NPV], int kb,
                                          float c, float (&ls)[QB][2], float (&lxs)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float nm = -m[qb];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                X2 pp[4];
                float xs = 0.f;
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const float p0 = exp2_hw(fmaf(s[qb][kb][8 * h + 2 * j], c, nm));
                    const float p1 = exp2_hw(fmaf(s[qb][kb][8 * h + 2 * j + 1], c, nm));
                    pp[j] = pack2<T>(p0, p1);
                    xs += p0 + p1;
                }
                ls[qb][h] = sum2(pp[3], sum2(pp[2], sum2(pp[1], sum2(pp[0], ls[qb][h]))));
                lxs[qb][h] += xs;
                pf[qb][2 * kb + h] = X8{pp[0][0], pp[0][1], pp[1][0], pp[1][1],
                                        pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
            }
        }
    }

    // V^T fragments (t, db): key rows 16*t + 8*hi + 4*u + (lane%16)/4.
    // The second read covers rows +4, whose swizzle flips chunk bit 0:
    // va[NVA] holds that step (4*RB +- 16 bytes) for this lane.
    static __device__ __forceinline__ void vfrags(X8 (&vf)[NPV][NDB], const char* vl,
                                                  const int (&va)[NVA + 1]) {
#pragma unroll
        for (int t = 0; t < NPV; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const char* vp = vl + va[db % NVA] + NVA * 64 * (db / NVA) + 16 * t * RB;
                const u32x2 lo = lds_read_tr16(vp);
                const u32x2 hi4 = lds_read_tr16(vp + va[NVA]);
                vf[t][db] = __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
            }
    }

    __device__ __forceinline__ void pv(const X8 (&vf)[NPV][NDB], const X8 (&pf)[QB][NPV]) {
#pragma unroll
        for (int t = 0; t < NPV; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf[t][db], pf[qb][t], o[qb][db]);
    }

    __device__ __forceinline__ void begin_sums(float (&ls)[QB][2], float (&lxs)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            ls[qb][0] = l[qb];
            ls[qb][1] = 0.f;
            lxs[qb][0] = lx[qb];
            lxs[qb][1] = 0.f;
        }
    }
    __device__ __forceinline__ void end_sums(const float (&ls)[QB][2], const float (&lxs)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l[qb] = ls[qb][0] + ls[qb][1];
            lx[qb] = lxs[qb][0] + lxs[qb][1];
        }
    }

    // Softmax + PV of a tile whose scores are in s (no overlap).
    __device__ __forceinline__ void finish(const f32x16 (&s)[QB][NKB], const char* vl,
                                           const int (&va)[NVA + 1], float c) {
        float mt[QB];
        tile_max(s, c, mt);
        rescale(mt);
        X8 vf[NPV][NDB];
        vfrags(vf, vl, va);
        __builtin_amdgcn_sched_barrier(0);
        X8 pf[QB][NPV];
        float ls[QB][2], lxs[QB][2];
        begin_sums(ls, lxs);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) probs(s, pf, kb, c, ls, lxs);
        end_sums(ls, lxs);
        pv(vf, pf);
    }

    // Pipelined step, all in one wave's instruction stream:
    //   score MFMAs of the next tile (K fragments at kn) interleaved with the
    //   exponentials of this tile (scores s, maximum already applied), then
    //   the PV MFMAs of this tile interleaved with the row maximum of the next
    //   tile (returned in mtn). The next tile's K fragments come in two
    //   halves so the first half's registers are free before the second
    //   lands. sched_group_barrier fixes the MFMA / VALU alternation.
    __device__ __forceinline__ void overlap(const f32x16 (&s)[QB][NKB], f32x16 (&sn)[QB][NKB],
                                            float (&mtn)[QB], const char* kn, const int (&ka)[NKA],
                                            const char* vl, const int (&va)[NVA + 1],
                                            const X8 (&qf)[QB][NCH], float c) {
        constexpr int MF_HALF = (NCH / 2) * NKB * QB;     // score MFMAs per half
        constexpr int MF_PV = NPV * NDB * QB;             // PV MFMAs
        X8 kf[NKB][NCH];
#pragma unroll
        for (int ch = 0; ch < NCH / 2; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb][ch] = kfrag(kn, ka, ch, kb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sn[qb][kb] = f32x16{};
        X8 pf[QB][NPV];
        float ls[QB][2], lxs[QB][2];
        begin_sums(ls, lxs);
        qk(sn, kf, qf, 0, NCH / 2);
#pragma unroll
        for (int kb = 0; kb < NKB / 2; ++kb) probs(s, pf, kb, c, ls, lxs);
#pragma unroll
        for (int i = 0; i < MF_HALF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // eight VALU
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ch = NCH / 2; ch < NCH; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb][ch] = kfrag(kn, ka, ch, kb);
        __builtin_amdgcn_sched_barrier(0);
        qk(sn, kf, qf, NCH / 2, NCH);
#pragma unroll
        for (int kb = NKB / 2; kb < NKB; ++kb) probs(s, pf, kb, c, ls, lxs);
        end_sums(ls, lxs);
#pragma unroll
        for (int i = 0; i < MF_HALF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        X8 vf[NPV][NDB];
        vfrags(vf, vl, va);
        __builtin_amdgcn_sched_barrier(0);
        pv(vf, pf);
        tile_max(sn, c, mtn);
#pragma unroll
        for (int i = 0; i < MF_PV; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 2, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
};

template <typename T, int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(Cfg16<D>::NW * 64, Cfg16<D>::WPE)
fa_fwd16_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                void* __restrict__ Og, float* __restrict__ LSEg, int N, int num_qtiles,
                int num_blocks, float c)
{
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    constexpr int NW = Cfg16<D>::NW, QB = Cfg16<D>::QB, BC = Cfg16<D>::BC;
    using W = Wave16<T, D, QB, BC>;
    constexpr int QW = 32 * QB;            // query rows per wave
    constexpr int BR = NW * QW;            // query rows per workgroup
    constexpr int NCH = W::NCH, NDB = W::NDB, NKB = W::NKB, RB = W::RB;
    constexpr int TB = BC * RB;            // bytes per K (or V) tile
    constexpr int NIW = TB / 1024 / NW;    // 1 KB direct loads per wave per tile
    static_assert(TB % (1024 * NW) == 0, "tile must split into 1 KB loads per wave");
    static_assert(BC % 32 == 0, "key tile is a multiple of 32");

    // LDS: K tiles in slots 0, 1 and V tiles in slots 2, 3 (tile t uses t & 1).
    __shared__ __attribute__((aligned(1024))) char smem[4 * TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wave_u = wave_uniform(wave);
    // The tiles are written only by direct global->LDS loads, which the
    // compiler does not see as stores; a store it cannot rule out keeps the
    // LDS reads from being treated as reads of uninitialised memory.
    if (num_blocks < 0) smem[tid] = 0;

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

    // Direct-load mapping: load j of this wave fills bytes
    // [(wave*NIW + j) * 1024, +1024) of a tile; lane i writes 16 bytes at
    // +16*i, i.e. physical chunk cp of row r, which holds logical chunk
    // cp ^ lds_swz16(r) of that key row.
    int grow[NIW], gcol[NIW];
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
        const int p = (wave * NIW + j) * 1024 + 16 * lane;
        grow[j] = p / RB;
        gcol[j] = ((p % RB / 16) ^ lds_swz16<D>(grow[j])) * 8;
    }
    const int nkt_total = (N + BC - 1) / BC;
    auto load_k = [&](int t) {
        if (t >= nkt_total) return;
        char* dst = smem + (t & 1) * TB + wave_u * NIW * 1024;
#pragma unroll
        for (int j = 0; j < NIW; ++j) {
            const int key = min(t * BC + grow[j], N - 1);     // rows past N: any valid row
            load_lds16(K + (size_t)key * D + gcol[j], dst + j * 1024);
        }
    };
    auto load_v = [&](int t) {
        if (t >= nkt_total) return;
        char* dst = smem + (2 + (t & 1)) * TB + wave_u * NIW * 1024;
#pragma unroll
        for (int j = 0; j < NIW; ++j) {
            const int key = min(t * BC + grow[j], N - 1);
            load_lds16(V + (size_t)key * D + gcol[j], dst + j * 1024);
        }
    };
    auto ktile = [&](int t) -> const char* { return smem + (t & 1) * TB; };
    auto vtile = [&](int t) -> const char* { return smem + (2 + (t & 1)) * TB; };

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

    // Lane byte offsets into a swizzled tile (see lds_swz16):
    //  K fragment (ch, kb): ka[ch % NKA] + NKA*32*(ch / NKA) + 32*kb*RB.
    //  V^T fragment (t, u, db): row 16*t + 8*hi + 4*u + (lane%16)/4, bytes
    //    64*db + 32*((lane%32)/16) + 8*(lane%4): va[db % NVA] + NVA*64*(db / NVA).
    int ka[W::NKA], va[W::NVA + 1];
    {
        const int kr = krow_perm(l32);
#pragma unroll
        for (int ch = 0; ch < W::NKA; ++ch)
            ka[ch] = kr * RB + (((2 * ch + hi) ^ lds_swz16<D>(kr)) * 16);
        const int vr = 8 * hi + (lane & 15) / 4;
#pragma unroll
        for (int db = 0; db < W::NVA; ++db) {
            const int chunk = 4 * db + 2 * (l32 / 16) + ((lane & 3) >> 1);
            va[db] = vr * RB + ((chunk ^ lds_swz16<D>(vr)) * 16) + 8 * (lane & 1);
        }
        // rows vr + 4: swizzle term + 1 (bit 2 of vr is 0), i.e. chunk bit 0
        // flips; the chunk's bit 0 is (lane & 3) >> 1 for every d-block.
        va[W::NVA] = 4 * RB + (((lane & 3) >> 1) ? -16 : 16);
    }

    W st;
    st.init();
    f32x16 s[QB][NKB];

    // Invariant at the top of step t: K_t, V_t and (if any) K_{t+1} are in
    // LDS. Step t fills the slots of K_{t-1}/K_t and V_{t-1} that every wave
    // finished with before the previous barrier.
    load_k(0);
    load_v(0);
    load_k(1);
    wait_vm_all();
    __syncthreads();
    float mt[QB];
    if (nfull > 0) {
        W::scores(s, ktile(0), ka, qf);
        W::tile_max(s, c, mt);
        __syncthreads();                     // all waves done reading K_0's slot
    }
    int t = 0;
    // Pipelined full tiles: the scores of tile t+1 are computed while the
    // softmax of tile t runs.
    for (; t + 1 < nfull; ++t) {
        load_k(t + 2);
        load_v(t + 1);
        st.rescale(mt);
        f32x16 sn[QB][NKB];
        st.overlap(s, sn, mt, ktile(t + 1), ka, vtile(t), va, qf, c);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = sn[qb][kb];
        wait_vm_all();
        __syncthreads();
    }
    if (nfull > 0) {                          // last full tile: no next scores
        load_v(t + 1);
        st.finish(s, vtile(t), va, c);
        wait_vm_all();
        __syncthreads();
        ++t;
    }
    // Masked tiles: ragged end of the sequence and the causal diagonal.
    for (; t < nkt; ++t) {
        load_k(t + 1);
        load_v(t + 1);
        const int k0 = t * BC;
        if (!CAUSAL || k0 <= q0 + QW - 1) {   // wave has a visible key in this tile
            W::scores(s, ktile(t), ka, qf);
            W::template mask<CAUSAL>(s, k0, q0, N, hi, l32);
            st.finish(s, vtile(t), va, c);
        }
        wait_vm_all();
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l~, LSE = ln2 * (m + log2 l) ----
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = pair_sum(st.l[qb]);
        const float lx = pair_sum(st.lx[qb]);
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

// ---------------------------------------------------------------------------
// Ping-pong kernel (head dims 64 and 128): eight waves in two groups of four
// (one wave of each group per SIMD). Per key tile a group runs four phases,
//   QK  : score MFMAs (K fragments already in registers)
//   VS  : V^T fragments LDS -> registers, then the softmax (VALU)
//   PV  : PV MFMAs
//   LK  : next tile's K fragments LDS -> registers
// and the second group runs the same sequence one phase later, so in every
// phase one wave of each SIMD issues MFMAs while the other reads LDS and runs
// the exponentials. Workgroup barriers separate the phases ("FlashAttention-3:
// Fast & Accurate Attention with Asynchrony & Low-Precision", section
// "Overlapping GEMM and Softmax (Asynchrony)": inter-warpgroup ping-pong).
// The MFMA phases run at raised wave priority (s_setprio).
//
// Both groups run the same loop body; the second group enters it one phase
// later (its first phase only reads K_0's fragments) and the first group
// ends with one empty phase, so both pass the same number of barriers.
//
// Global -> LDS: K tile t and V tile t in slots t & 1. The first group issues
// all copies: V_{t+1} and K_{t+2} in global phase 4t+1, waited for (vmcnt)
// at the end of phase 4t+4, before the barrier that starts the first phase
// reading them. Slot reuse: V_{t+1} overwrites V_{t-1} (last read in phase
// 4t-2), K_{t+2} overwrites K_t (last read in phase 4t).
// ---------------------------------------------------------------------------
#ifndef FA16_PP_BC
#define FA16_PP_BC 64
#endif
#ifndef FA16_PP_PRIO
#define FA16_PP_PRIO 1
#endif

template <typename T, int D, bool CAUSAL, bool OUT_F32>
__device__ __forceinline__ void store_rows(const Wave16<T, D, 1, FA16_PP_BC>& st, void* Og,
                                           float* LSEg, size_t head, int bh, int N, int q0,
                                           int l32, int hi)
{
    using X2 = typename Elt<T>::x2;
    constexpr int NDB = D / 32;
    const float l = pair_sum(st.l[0]);
    const float lx = pair_sum(st.lx[0]);
    const float inv = 1.0f / l;
    const int row = q0 + l32;
    if (row >= N) return;
    if (hi == 0) LSEg[(size_t)bh * N + row] = (st.m[0] + __builtin_amdgcn_logf(lx)) * kLn2;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int dcol = 32 * db + 8 * j + 4 * hi;
            const size_t off = head + (size_t)row * D + dcol;
            const float v0 = st.o[0][db][4 * j] * inv, v1 = st.o[0][db][4 * j + 1] * inv;
            const float v2 = st.o[0][db][4 * j + 2] * inv, v3 = st.o[0][db][4 * j + 3] * inv;
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

__device__ __forceinline__ void prio_hi() { if (FA16_PP_PRIO) __builtin_amdgcn_s_setprio(1); }
__device__ __forceinline__ void prio_lo() { if (FA16_PP_PRIO) __builtin_amdgcn_s_setprio(0); }

template <typename T, int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(512, 2)
fa_fwd16_pp_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                   void* __restrict__ Og, float* __restrict__ LSEg, int N, int num_qtiles,
                   int num_blocks, float c)
{
    using X8 = typename Elt<T>::x8;
    constexpr int NW = 8, QB = 1, BC = FA16_PP_BC;
    using W = Wave16<T, D, QB, BC>;
    constexpr int QW = 32, BR = NW * QW;
    constexpr int NCH = W::NCH, NDB = W::NDB, NKB = W::NKB, NPV = W::NPV, RB = W::RB;
    constexpr int TB = BC * RB;
    static_assert(TB % (1024 * 4) == 0, "tile must split into 1 KB loads per wave");

    __shared__ __attribute__((aligned(1024))) char smem[4 * TB];   // K: slots 0,1; V: 2,3

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wave_u = wave_uniform(wave);
    const int group = wave_u >> 2;
    if (num_blocks < 0) smem[tid] = 0;   // see fa_fwd16_kernel

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

    // Direct-load mapping (first group only): load j of wave w fills bytes
    // [(w*NIL + j) * 1024, +1024) of a tile; lane i writes 16 bytes at +16*i.
    constexpr int NIL = TB / 1024 / 4;
    int grow[NIL], gcol[NIL];
#pragma unroll
    for (int j = 0; j < NIL; ++j) {
        const int p = ((wave & 3) * NIL + j) * 1024 + 16 * lane;
        grow[j] = p / RB;
        gcol[j] = ((p % RB / 16) ^ lds_swz16<D>(grow[j])) * 8;
    }
    const int nkt_total = (N + BC - 1) / BC;
    auto load_k = [&](int t) {
        if (t >= nkt_total) return;
        char* dst = smem + (t & 1) * TB + (wave_u & 3) * NIL * 1024;
#pragma unroll
        for (int j = 0; j < NIL; ++j) {
            const int key = min(t * BC + grow[j], N - 1);
            load_lds16(K + (size_t)key * D + gcol[j], dst + j * 1024);
        }
    };
    auto load_v = [&](int t) {
        if (t >= nkt_total) return;
        char* dst = smem + (2 + (t & 1)) * TB + (wave_u & 3) * NIL * 1024;
#pragma unroll
        for (int j = 0; j < NIL; ++j) {
            const int key = min(t * BC + grow[j], N - 1);
            load_lds16(V + (size_t)key * D + gcol[j], dst + j * 1024);
        }
    };
    auto ktile = [&](int t) -> const char* { return smem + (t & 1) * TB; };
    auto vtile = [&](int t) -> const char* { return smem + (2 + (t & 1)) * TB; };

    X8 qf[QB][NCH];
    {
        const int row = q0 + l32;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            if (row < N)
                qf[0][ch] = load16<X8>(Q + (size_t)row * D + 16 * ch + 8 * hi);
            else
                qf[0][ch] = __builtin_bit_cast(X8, u32x4{0, 0, 0, 0});
        }
    }
    int ka[W::NKA], va[W::NVA + 1];
    {
        const int kr = krow_perm(l32);
#pragma unroll
        for (int ch = 0; ch < W::NKA; ++ch)
            ka[ch] = kr * RB + (((2 * ch + hi) ^ lds_swz16<D>(kr)) * 16);
        const int vr = 8 * hi + (lane & 15) / 4;
#pragma unroll
        for (int db = 0; db < W::NVA; ++db) {
            const int chunk = 4 * db + 2 * (l32 / 16) + ((lane & 3) >> 1);
            va[db] = vr * RB + ((chunk ^ lds_swz16<D>(vr)) * 16) + 8 * (lane & 1);
        }
        // rows vr + 4: swizzle term + 1 (bit 2 of vr is 0), i.e. chunk bit 0
        // flips; the chunk's bit 0 is (lane & 3) >> 1 for every d-block.
        va[W::NVA] = 4 * RB + (((lane & 3) >> 1) ? -16 : 16);
    }

    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const int nkt = (kend + BC - 1) / BC;

    W st;
    st.init();
    X8 kf[NKB][NCH];
    X8 vf[NPV][NDB];
    f32x16 s[QB][NKB];
    X8 pf[QB][NPV];

    auto lk = [&](int t) {
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb][ch] = W::kfrag(ktile(t), ka, ch, kb);
    };
    auto qk = [&]() {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[0][kb] = f32x16{};
        W::qk(s, kf, qf, 0, NCH);
    };
    // Softmax of tile t with the V^T fragment reads spread over it: each
    // score block's exponentials run while the next batch of V reads lands.
    auto vsm = [&](int t, bool masked) {
        if (masked) W::template mask<CAUSAL>(s, t * BC, q0, N, hi, l32);
        float mt[QB];
        W::tile_max(s, c, mt);
        st.rescale(mt);
        float ls[QB][2], lxs[QB][2];
        st.begin_sums(ls, lxs);
        const char* vl = vtile(t);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int tt = 2 * kb; tt < 2 * kb + 2; ++tt)
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const char* vp = vl + va[db % W::NVA] + W::NVA * 64 * (db / W::NVA) + 16 * tt * RB;
                    const u32x2 lo = lds_read_tr16(vp);
                    const u32x2 hi4 = lds_read_tr16(vp + va[W::NVA]);
                    vf[tt][db] = __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
                }
            __builtin_amdgcn_sched_barrier(0);
            st.probs(s, pf, kb, c, ls, lxs);
            __builtin_amdgcn_sched_barrier(0);
        }
        st.end_sums(ls, lxs);
    };
    auto pv = [&]() { st.pv(vf, pf); };

    // prologue: K_0, V_0, K_1 in LDS; the first group reads K_0's fragments,
    // then the second group does (its phase shift).
    if (group == 0) {
        load_k(0);
        load_v(0);
        load_k(1);
    }
    phase_barrier_vm();
    if (group == 0) lk(0);
    phase_barrier();
    if (group == 1) {
        lk(0);
        phase_barrier();
    }
    // Tiles [0, nact) hold a key visible to this wave; with causal masking
    // the wave then only keeps the barrier / copy schedule for the rest.
    // (Unconditional work inside the first loop keeps the compiler from
    // carrying fragment registers across iterations.)
    const int nact = CAUSAL ? min(nkt, (q0 + QW - 1) / BC + 1) : nkt;
    int t = 0;
    for (; t < nact; ++t) {
        const int k0 = t * BC;
        const bool msk = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
        // phase 0: QK (first group: global phase 4t)
        prio_hi();
        qk();
        prio_lo();
        if (group == 0) phase_barrier_vm();
        else phase_barrier();
        // phase 1: V fragments + softmax; first group streams V_{t+1}, K_{t+2}
        if (group == 0) {
            load_v(t + 1);
            load_k(t + 2);
        }
        vsm(t, msk);
        phase_barrier();
        // phase 2: PV
        prio_hi();
        pv();
        prio_lo();
        phase_barrier();
        // phase 3: next K fragments (a stale slot when t + 1 == nkt: unused)
        lk(t + 1);
        phase_barrier();
    }
    for (; t < nkt; ++t) {
        if (group == 0) phase_barrier_vm();
        else phase_barrier();
        if (group == 0) {
            load_v(t + 1);
            load_k(t + 2);
        }
        phase_barrier();
        phase_barrier();
        phase_barrier();
    }
    if (group == 0) phase_barrier();
    store_rows<T, D, CAUSAL, OUT_F32>(st, Og, LSEg, head, bh, N, q0, l32, hi);
}

#ifndef FA16_PINGPONG
#define FA16_PINGPONG 0
#endif

template <typename T, int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    if constexpr (FA16_PINGPONG && D <= 128) {
        constexpr int BR = 256;
        const int num_qtiles = (a.N + BR - 1) / BR;
        const long long nblk = (long long)num_qtiles * a.B * a.H;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((fa_fwd16_pp_kernel<T, D, CAUSAL, OUT_F32>), dim3((unsigned)nblk),
                           dim3(512), 0, s, static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), a.o, a.lse, a.N, num_qtiles, (int)nblk,
                           a.scale * kLog2e);
        return hipGetLastError();
    }
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
