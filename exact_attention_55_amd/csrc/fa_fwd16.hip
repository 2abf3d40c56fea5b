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
//    (buffer loads with an LDS destination, 16 bytes per lane, no staging
//    registers; the tile's offset is a scalar operand and rows at or past N
//    read as zeros), double buffered: tile j+1 is in flight while tile j is
//    computed, with one workgroup barrier per tile. Rows are stored unpadded
//    with their 16-byte chunks XOR-swizzled (see lds_swz16), which keeps both
//    the K fragment reads and the transposing V reads free of bank conflicts.
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
//    hardware v_exp_f32. The reference maximum m is the exact row maximum of
//    the first key tile; later tiles take their exponentials against it
//    without computing their own maximum. Only when a tile's sum of p in some
//    lane exceeds kBig is that tile redone with its exact maximum (moving m
//    and rescaling O and the sums). The result is the same exact softmax up
//    to rounding because l and O always share m.
//  * Row sums: l~ of the rounded P actually fed to the PV MFMA (dot2 with
//    ones) normalises O, which makes O an exact convex combination of V rows
//    even when one key dominates. For fp16 it also gives the log-sum-exp
//    (relative error at most fp16's rounding of P, 2^-11: within the LSE
//    tolerance). bf16's rounding (2^-8) is not, so bf16 keeps a second,
//    fp32 sum for the log-sum-exp: two more adds per pair of exponentials
//    (2.5-5.5 % of the kernel time; FA16_XSUM=1 forces it for fp16 too).
//  * Schedule ("FlashAttention-3: ...", "Overlapping GEMM and Softmax"): two
//    waves share each SIMD, and inside a wave one step overlaps the score
//    MFMAs of key tile j+1 with the exponentials of tile j, then runs the PV
//    MFMAs of tile j. The step is written as a fixed instruction order
//    (Wave16::step): every score MFMA is preceded by the LDS read of the K
//    fragment four MFMAs ahead and followed by its share of exponentials,
//    and every PV MFMA by the reads of the V^T fragment four ahead. The
//    score phase runs at raised wave priority. FA16_SCHED=0 selects the
//    earlier two-half schedule left to the compiler (Wave16::overlap), kept
//    as an ablation.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

// A tile whose exponentials sum past kBig in some lane is redone with its
// exact row maximum (see Wave16::settle); every p is then <= kBig, which
// fp16 P (max 65504) and the fp32 accumulators hold with room to spare.
constexpr float kBig = 16384.0f;

#ifndef FA16_SCHED                 // 1: hand-ordered step; 0: compiler-scheduled overlap
#define FA16_SCHED 1
#endif
#ifndef FA16_XSUM                 // 1: separate fp32 row sum for the log-sum-exp also for fp16
#define FA16_XSUM 0
#endif
#ifndef FA16_KPD
#define FA16_KPD 4
#endif
#ifndef FA16_VPD
#define FA16_VPD 4
#endif
// 1: two wave groups per workgroup in ping-pong (see the full-tile loop of
// fa_fwd16_kernel); the d = 128 configuration then has 8 waves.
#ifndef FA16_PINGPONG
#define FA16_PINGPONG 0
#endif
// 0: the score phase of a step runs at normal wave priority.
#ifndef FA16_PRIO
#define FA16_PRIO 1
#endif

// Tile configuration per head dimension. NW waves per workgroup, each owning
// 32*QB query rows; BC keys per K/V tile; WPE = waves per SIMD the register
// budget is sized for (2: 256 registers per wave, so two waves share a SIMD
// and one wave's softmax overlaps the other's MFMAs). At d = 64 a wide form
// gives each wave 64 query rows (each K and V^T fragment read from LDS feeds
// two MFMAs, halving the LDS bytes per flop) with 32-key tiles, which still
// fits two waves per SIMD; it is launched when its grid fills the GPU twice
// over (kWideMinBlocks workgroups), since 256-row workgroups leave a short
// or small problem with too few of them.
#ifndef FA16_CFG_64
#define FA16_CFG_64 4, 1, 64, 2
#endif
#ifndef FA16_CFG_64_WIDE
#define FA16_CFG_64_WIDE 4, 2, 32, 2
#endif
#ifndef FA16_CFG_128
#if FA16_PINGPONG
#define FA16_CFG_128 8, 1, 64, 2
#else
#define FA16_CFG_128 4, 1, 64, 2
#endif
#endif
#ifndef FA16_CFG_256
#define FA16_CFG_256 4, 1, 64, 1
#endif
constexpr long long kWideMinBlocks = 1024;
template <int NW_, int QB_, int BC_, int WPE_> struct CfgT {
    static constexpr int NW = NW_, QB = QB_, BC = BC_, WPE = WPE_;
};
template <int D, bool WIDE> struct Cfg16;
template <> struct Cfg16<64, false> : CfgT<FA16_CFG_64> {};
template <> struct Cfg16<64, true> : CfgT<FA16_CFG_64_WIDE> {};
template <> struct Cfg16<128, false> : CfgT<FA16_CFG_128> {};
template <> struct Cfg16<256, false> : CfgT<FA16_CFG_256> {};

// ACC: O lives in the accumulation registers (one wave per SIMD, where the
// 512-register budget puts it there); its rare rescale then runs in place.
template <typename T, int D, int QB, int BC, bool ACC>
struct Wave16 {
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    static constexpr int RB = 2 * D;       // bytes per K / V row in LDS
    static constexpr int NCH = D / 16;     // k-steps of S^T = K Q^T
    static constexpr int NDB = D / 32;     // 32-row blocks of O^T
    static constexpr int NKB = BC / 32;    // 32-key blocks of S^T
    static constexpr int NPV = BC / 16;    // k-steps of O^T += V^T P^T

    // separate fp32 row sum for the log-sum-exp (see the file header)
    static constexpr bool XS = FA16_XSUM || std::is_same<T, __bf16>::value;

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

    // Moves the reference maximum to max(m, mt), rescaling O, l and lx.
    __device__ __forceinline__ void raise_max(const float (&mt)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mnew = fmaxf(m[qb], mt[qb]);
            const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(m[qb] - mnew);
            m[qb] = mnew;
            l[qb] *= alpha;
            lx[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                if (ACC)
                    scale_acc(o[qb][db], alpha);
                else
                    o[qb][db] *= alpha;
            }
        }
    }

    // P for score block kb (16 keys per lane -> two PV operands), with the
    // tile's row sums in independent partial accumulators.
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
                    if (XS) xs += p0 + p1;
                }
                ls[qb][h] = sum2(pp[3], sum2(pp[2], sum2(pp[1], sum2(pp[0], ls[qb][h]))));
                if (XS) lxs[qb][h] += xs;
                pf[qb][2 * kb + h] = X8{pp[0][0], pp[0][1], pp[1][0], pp[1][1],
                                        pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
            }
        }
    }

    static __device__ __forceinline__ void zero_sums(float (&ls)[QB][2], float (&lxs)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) ls[qb][0] = ls[qb][1] = lxs[qb][0] = lxs[qb][1] = 0.f;
    }

    // The reference maximum is not moved per tile. Exponentials are taken
    // against it directly; a tile is redone with its exact maximum only when
    // its sum in some lane exceeds kBig (every p is then <= kBig: no
    // overflow in fp16 P or in the fp32 accumulators). The exact softmax is
    // unchanged: O, l and lx share the reference (FlashAttention v1/v2
    // rescaling, done only when needed).
    __device__ __forceinline__ void settle(const f32x16 (&s)[QB][NKB], X8 (&pf)[QB][NPV], float c,
                                           float (&ls)[QB][2], float (&lxs)[QB][2]) {
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
            big |= (XS ? lxs[qb][0] + lxs[qb][1] : ls[qb][0] + ls[qb][1]) > kBig;
        if (wave_any(big)) {
            float mt[QB];
            tile_max(s, c, mt);
            raise_max(mt);
            zero_sums(ls, lxs);
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) probs(s, pf, kb, c, ls, lxs);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l[qb] += ls[qb][0] + ls[qb][1];
            if (XS) lx[qb] += lxs[qb][0] + lxs[qb][1];
        }
    }

    // V^T fragments (t, db): key rows 16*t + 8*hi + 4*u + (lane%16)/4, read
    // without waits in (t, db) order, rows +0..3 (base b0) then +4..7 (base
    // b1, whose swizzle differs); pv_async waits for each k-step's share.
    static __device__ __forceinline__ void vfrags_async(u32x2 (&vlo)[NPV][NDB], u32x2 (&vhi)[NPV][NDB],
                                                        const uint32_t (&b0)[NVA],
                                                        const uint32_t (&b1)[NVA]) {
        static_for<0, NPV>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            static_for<0, NDB>([&](auto dc) {
                constexpr int db = decltype(dc)::value;
                constexpr int off = NVA * 64 * (db / NVA) + 16 * t * RB;
                vlo[t][db] = lds_tr16_async<off>(b0[db % NVA]);
                vhi[t][db] = lds_tr16_async<off>(b1[db % NVA]);
            });
        });
    }

    __device__ __forceinline__ void pv_async(u32x2 (&vlo)[NPV][NDB], u32x2 (&vhi)[NPV][NDB],
                                             const X8 (&pf)[QB][NPV]) {
        static_for<0, NPV>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            constexpr int later = 2 * NDB * (NPV - 1 - t);     // reads issued after step t's
            lgkm_wait<(later > 15 ? 15 : later)>();
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                lgkm_bind(vlo[t][db]);
                lgkm_bind(vhi[t][db]);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const X8 v = __builtin_bit_cast(
                    X8, u32x4{vlo[t][db][0], vlo[t][db][1], vhi[t][db][0], vhi[t][db][1]});
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(v, pf[qb][t], o[qb][db]);
            }
        });
    }

    // Softmax + PV of a tile whose scores are in s (no overlap; masked
    // tiles). P~, the exponentials rounded to the 16-bit type, or with RESID
    // the rounding residue p - P~ (exact in fp32) instead, rounded to the
    // 16-bit type; l sums it too, and the fp32 sum for the log-sum-exp is
    // left alone. The kernel runs a tile once and, for the first key tile,
    // again with RESID: P then reaches the PV product as P~ plus
    // its residue (about 16 significant bits). The first key tile is the
    // only one where a row can see few keys, and there rounding P to bf16
    // (2^-8 relative) moves O by up to ~w(1-w) 2^-8 |v_a - v_b| on a row that
    // two keys share with weights w, 1 - w: above 4e-3 for |v_a - v_b| near
    // 8. Once a row sees a few dozen keys the effect averages out.
    // RESID: 0 P~, 1 the residue, 2 chosen at run time by rm (0 or 1): one
    // copy of the tile code for both passes, which the register budget of
    // the one-wave-per-SIMD d = 256 kernel needs (two copies spill there).
    template <int RESID = 0>
    __device__ __forceinline__ void finish(const f32x16 (&s)[QB][NKB], const uint32_t (&b0)[NVA],
                                           const uint32_t (&b1)[NVA], float c, float rm = 0.f) {
        X8 pf[QB][NPV];
        float ls[QB][2], lxs[QB][2];
        zero_sums(ls, lxs);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float nm = -m[qb];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    X2 pp[4];
                    float xs = 0.f;
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float p0 = exp2_hw(fmaf(s[qb][kb][8 * h + 2 * j], c, nm));
                        float p1 = exp2_hw(fmaf(s[qb][kb][8 * h + 2 * j + 1], c, nm));
                        if (XS) xs += p0 + p1;
                        if constexpr (RESID == 1) {
                            const X2 r = pack2<T>(p0, p1);
                            p0 -= (float)r[0];
                            p1 -= (float)r[1];
                        } else if constexpr (RESID == 2) {
                            const X2 r = pack2<T>(p0, p1);
                            p0 = fmaf(-rm, (float)r[0], p0);
                            p1 = fmaf(-rm, (float)r[1], p1);
                        }
                        pp[j] = pack2<T>(p0, p1);
                    }
                    ls[qb][h] = sum2(pp[3], sum2(pp[2], sum2(pp[1], sum2(pp[0], ls[qb][h]))));
                    if (XS && RESID == 0) lxs[qb][h] += xs;
                    if (XS && RESID == 2) lxs[qb][h] += xs * (1.f - rm);
                    pf[qb][2 * kb + h] = X8{pp[0][0], pp[0][1], pp[1][0], pp[1][1],
                                            pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
                }
            }
        }
        settle(s, pf, c, ls, lxs);
        if constexpr (NPV * NDB > 16) {
            // d = 256: the whole tile's V^T fragments would take 128 registers
            pv_by_step(b0, b1, pf);
        } else {
            u32x2 vlo[NPV][NDB], vhi[NPV][NDB];
            vfrags_async(vlo, vhi, b0, b1);
            __builtin_amdgcn_sched_barrier(0);
            pv_async(vlo, vhi, pf);
        }
    }

    // O^T += V^T P^T for the tile, one k-step at a time: the step's V^T
    // fragments are read, awaited and consumed before the next step's, so
    // only NDB fragments are live (masked tiles at d = 256).
    __device__ __forceinline__ void pv_by_step(const uint32_t (&b0)[NVA], const uint32_t (&b1)[NVA],
                                               const X8 (&pf)[QB][NPV]) {
        static_for<0, NPV>([&](auto tc) {
            constexpr int t = decltype(tc)::value;
            u32x2 vlo[NDB], vhi[NDB];
            static_for<0, NDB>([&](auto dc) {
                constexpr int db = decltype(dc)::value;
                constexpr int off = NVA * 64 * (db / NVA) + 16 * t * RB;
                vlo[db] = lds_tr16_async<off>(b0[db % NVA]);
                vhi[db] = lds_tr16_async<off>(b1[db % NVA]);
            });
            lgkm_wait<0>();
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                lgkm_bind(vlo[db]);
                lgkm_bind(vhi[db]);
            }
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const X8 v = __builtin_bit_cast(X8, u32x4{vlo[db][0], vlo[db][1], vhi[db][0], vhi[db][1]});
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(v, pf[qb][t], o[qb][db]);
            }
        });
    }

    // Pipelined step, all in one wave's instruction stream: the score MFMAs
    // of the next tile (K fragments at kn) interleaved with the exponentials
    // of this tile (scores s), then the PV MFMAs of this tile. The next
    // tile's K fragments come in two halves so the first half's registers
    // are free before the second lands. sched_group_barrier fixes the
    // MFMA / VALU alternation.
    __device__ __forceinline__ void overlap(const f32x16 (&s)[QB][NKB], f32x16 (&sn)[QB][NKB],
                                            const char* kn, const int (&ka)[NKA],
                                            const uint32_t (&b0)[NVA], const uint32_t (&b1)[NVA],
                                            const X8 (&qf)[QB][NCH], float c) {
        constexpr int MF_HALF = (NCH / 2) * NKB * QB;     // score MFMAs per half
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
        zero_sums(ls, lxs);
        // The MFMA + exponential phase runs at raised wave priority: of the
        // two waves sharing a SIMD, the one in this phase issues first and the
        // other (in its PV phase) fills the matrix core around it.
        if (FA16_PRIO) __builtin_amdgcn_s_setprio(1);
        qk(sn, kf, qf, 0, NCH / 2);
#pragma unroll
        for (int kb = 0; kb < NKB / 2; ++kb) probs(s, pf, kb, c, ls, lxs);
#pragma unroll
        for (int i = 0; i < MF_HALF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // six VALU
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
#pragma unroll
        for (int i = 0; i < MF_HALF; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        if (FA16_PRIO) __builtin_amdgcn_s_setprio(0);
        settle(s, pf, c, ls, lxs);
        u32x2 vlo[NPV][NDB], vhi[NPV][NDB];
        vfrags_async(vlo, vhi, b0, b1);
        __builtin_amdgcn_sched_barrier(0);
        pv_async(vlo, vhi, pf);
        __builtin_amdgcn_sched_barrier(0);
    }

    // ---- fine-grained schedule (compiler-visible LDS reads) ----
    __device__ __forceinline__ void pv(const X8 (&vf)[NPV][NDB], const X8 (&pf)[QB][NPV]) {
#pragma unroll
        for (int t = 0; t < NPV; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db)
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf[t][db], pf[qb][t], o[qb][db]);
    }

    // V^T fragment (t, db) with two transposing reads: rows +0..3 at
    // va[db % NVA] + NVA*64*(db / NVA) + 16*t*RB, rows +4..7 vstep further.
    static __device__ __forceinline__ X8 vfrag(const char* vl, const int (&va)[NVA], int vstep,
                                               int t, int db) {
        const char* vp = vl + va[db % NVA] + NVA * 64 * (db / NVA) + 16 * t * RB;
        const u32x2 lo = lds_read_tr16(vp);
        const u32x2 hi4 = lds_read_tr16(vp + vstep);
        return __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
    }

    // One exponential pair of the tile: scores 8*h + 2*j, +1 of block kb.
    __device__ __forceinline__ void prob_pair(const f32x16 (&s)[QB][NKB], X2 (&pp)[QB][NKB][2][4],
                                              int kb, int h, int j, float c, float (&ls)[QB][2],
                                              float (&lxs)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float p0 = exp2_hw(fmaf(s[qb][kb][8 * h + 2 * j], c, -m[qb]));
            const float p1 = exp2_hw(fmaf(s[qb][kb][8 * h + 2 * j + 1], c, -m[qb]));
            pp[qb][kb][h][j] = pack2<T>(p0, p1);
            ls[qb][h] = sum2(pp[qb][kb][h][j], ls[qb][h]);
            if (XS) lxs[qb][h] += p0 + p1;
        }
    }

    // Pipelined step as one instruction stream in program order (every
    // chunk ends in a scheduling barrier):
    //   NQK chunks, each: one LDS read KPD fragments ahead (K of the next
    //   tile; in the last VPD chunks the first V^T fragments of this tile),
    //   one score MFMA of the next tile, and an even share of this tile's
    //   exponentials, which run in the MFMA's shadow;
    //   the overflow check (a branch, rarely taken);
    //   NPVM chunks, each: the reads of the V^T fragment VPD ahead and one PV
    //   MFMA.
    // The next tile's scores go to sn: the caller alternates two register
    // sets, so nothing is copied.
    __device__ __forceinline__ void step(const f32x16 (&s)[QB][NKB], f32x16 (&sn)[QB][NKB], const char* kn,
                                         const int (&ka)[NKA], const char* vl, const int (&va)[NVA],
                                         int vstep, const X8 (&qf)[QB][NCH], float c) {
        constexpr int NKF = NCH * NKB;      // K fragments = score MFMAs per tile
        constexpr int NVF = NPV * NDB;      // V^T fragments = PV MFMAs per tile
        constexpr int NPAIR = NKB * 8;      // exponential pairs per lane per tile
        // K / V^T fragments read ahead of their MFMA (at most half a tile's)
        constexpr int KPD = NKF >= 2 * FA16_KPD ? FA16_KPD : NKF / 2;
        constexpr int VPD = NVF >= 2 * FA16_VPD ? FA16_VPD : NVF / 2;
        static_assert(NKF >= KPD + VPD && NVF > VPD, "tile too small for the read-ahead");
        // The score phase reads the first KPD V^T fragments, the PV loop those
        // from VPD on: every fragment is read only if KPD >= VPD.
        static_assert(KPD >= VPD, "V^T fragments [KPD, VPD) would never be read");
        X8 kf[NKB][NCH];
        X8 vf[NPV][NDB];
        X2 pp[QB][NKB][2][4];
        float ls[QB][2], lxs[QB][2];
        zero_sums(ls, lxs);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sn[qb][kb] = f32x16{};
        if (FA16_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < KPD; ++f) kf[f % NKB][f / NKB] = kfrag(kn, ka, f / NKB, f % NKB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NKF; ++i) {
            const int f = i + KPD;                      // fragment read in this chunk
            if (f < NKF) {
                kf[f % NKB][f / NKB] = kfrag(kn, ka, f / NKB, f % NKB);
            } else {
                const int v = f - NKF;                  // V^T fragment (t, db) = (v / NDB, v % NDB)
                vf[v / NDB][v % NDB] = vfrag(vl, va, vstep, v / NDB, v % NDB);
            }
            const int ch = i / NKB, kb = i % NKB;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sn[qb][kb] = mfma32(kf[kb][ch], qf[qb][ch], sn[qb][kb]);
#pragma unroll
            for (int q = i * NPAIR / NKF; q < (i + 1) * NPAIR / NKF; ++q)
                prob_pair(s, pp, q / 8, (q / 4) % 2, q % 4, c, ls, lxs);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FA16_PRIO) __builtin_amdgcn_s_setprio(0);
        X8 pf[QB][NPV];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const X2 (&w)[4] = pp[qb][kb][h];
                    pf[qb][2 * kb + h] =
                        X8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
                }
        settle(s, pf, c, ls, lxs);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NVF; ++j) {
            const int v = j + VPD;
            if (v < NVF) vf[v / NDB][v % NDB] = vfrag(vl, va, vstep, v / NDB, v % NDB);
            const int t = j / NDB, db = j % NDB;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf[t][db], pf[qb][t], o[qb][db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // The two halves of step() for the ping-pong schedule, which puts a
    // workgroup barrier between them: phase_a runs the score MFMAs of the
    // next tile with this tile's exponentials and the overflow check (P into
    // pf, which stays live across the barrier); phase_b the PV MFMAs.
    __device__ __forceinline__ void phase_a(const f32x16 (&s)[QB][NKB], f32x16 (&sn)[QB][NKB],
                                            const char* kn, const int (&ka)[NKA],
                                            const X8 (&qf)[QB][NCH], float c, X8 (&pf)[QB][NPV]) {
        constexpr int NKF = NCH * NKB;
        constexpr int NPAIR = NKB * 8;
        constexpr int KPD = NKF >= 2 * FA16_KPD ? FA16_KPD : NKF / 2;
        X8 kf[NKB][NCH];
        X2 pp[QB][NKB][2][4];
        float ls[QB][2], lxs[QB][2];
        zero_sums(ls, lxs);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) sn[qb][kb] = f32x16{};
        if (FA16_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < KPD; ++f) kf[f % NKB][f / NKB] = kfrag(kn, ka, f / NKB, f % NKB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NKF; ++i) {
            const int f = i + KPD;
            if (f < NKF) kf[f % NKB][f / NKB] = kfrag(kn, ka, f / NKB, f % NKB);
            const int ch = i / NKB, kb = i % NKB;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sn[qb][kb] = mfma32(kf[kb][ch], qf[qb][ch], sn[qb][kb]);
#pragma unroll
            for (int q = i * NPAIR / NKF; q < (i + 1) * NPAIR / NKF; ++q)
                prob_pair(s, pp, q / 8, (q / 4) % 2, q % 4, c, ls, lxs);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FA16_PRIO) __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const X2 (&w)[4] = pp[qb][kb][h];
                    pf[qb][2 * kb + h] =
                        X8{w[0][0], w[0][1], w[1][0], w[1][1], w[2][0], w[2][1], w[3][0], w[3][1]};
                }
        settle(s, pf, c, ls, lxs);
        __builtin_amdgcn_sched_barrier(0);
    }
    __device__ __forceinline__ void phase_b(const char* vl, const int (&va)[NVA], int vstep,
                                            const X8 (&pf)[QB][NPV]) {
        constexpr int NVF = NPV * NDB;
        constexpr int VPD = NVF >= 2 * FA16_VPD ? FA16_VPD : NVF / 2;
        X8 vf[NPV][NDB];
#pragma unroll
        for (int v = 0; v < VPD; ++v) vf[v / NDB][v % NDB] = vfrag(vl, va, vstep, v / NDB, v % NDB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NVF; ++j) {
            const int v = j + VPD;
            if (v < NVF) vf[v / NDB][v % NDB] = vfrag(vl, va, vstep, v / NDB, v % NDB);
            const int t = j / NDB, db = j % NDB;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32(vf[t][db], pf[qb][t], o[qb][db]);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

template <typename T, int D, bool CAUSAL, bool OUT_F32, bool WIDE>
__global__ void __launch_bounds__((Cfg16<D, WIDE>::NW * 64), (Cfg16<D, WIDE>::WPE))
fa_fwd16_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                void* __restrict__ Og, float* __restrict__ LSEg, int N, int num_qtiles,
                int num_blocks, float c)
{
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    constexpr int NW = Cfg16<D, WIDE>::NW, QB = Cfg16<D, WIDE>::QB, BC = Cfg16<D, WIDE>::BC;
    using W = Wave16<T, D, QB, BC, Cfg16<D, WIDE>::WPE == 1>;
    constexpr int QW = 32 * QB;            // query rows per wave
    constexpr int BR = NW * QW;            // query rows per workgroup
    constexpr int NCH = W::NCH, NDB = W::NDB, NKB = W::NKB, RB = W::RB, NVA = W::NVA;
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

    // Workgroup -> (head, query tile) (see grid_tile). Causal: the heaviest
    // query tiles (last rows) of all heads go first.
    int bh, qt;
    grid_tile(num_blocks, num_qtiles, CAUSAL, bh, qt);
    if (CAUSAL) qt = num_qtiles - 1 - qt;

    const size_t head = (size_t)bh * N * D;
    const T* Q = Qg + head;
    const int qtile0 = qt * BR;
    const int q0 = qtile0 + wave * QW;

    // K / V tiles: buffer loads over this head's rows (rows at or past N
    // read as zeros) straight into LDS. Load j of this wave fills bytes
    // [(wave*NIW + j) * 1024, +1024) of a tile; lane i writes 16 bytes at
    // +16*i, i.e. physical chunk cp of row r, which holds logical chunk
    // cp ^ lds_swz16(r) of that key row. The tile's row offset is the
    // wave-uniform SGPR offset, so a load costs no vector instructions.
    const i32x4 krs = make_rsrc(Kg + head, N * RB);
    const i32x4 vrs = make_rsrc(Vg + head, N * RB);
    uint32_t voff[NIW];
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
        const int p = (wave * NIW + j) * 1024 + 16 * lane;
        const int row = p / RB;
        voff[j] = row * RB + ((p % RB / 16) ^ lds_swz16<D>(row)) * 16;
    }
    // tiles this workgroup reads: up to its last query row (causal) or N
    const int nkt_use = ((CAUSAL ? min(N, qtile0 + BR) : N) + BC - 1) / BC;
    const uint32_t sbase = lds_addr(smem);
    auto issue = [&](const i32x4& rs, int t, int slot) {
        const uint32_t dst = sbase + slot * TB + wave_u * NIW * 1024;
#pragma unroll
        for (int j = 0; j < NIW; ++j) buffer_load_lds16(rs, dst + j * 1024, voff[j], t * TB);
    };
    auto load_k = [&](int t) { if (t < nkt_use) issue(krs, t, t & 1); };
    auto load_v = [&](int t) { if (t < nkt_use) issue(vrs, t, 2 + (t & 1)); };
    auto ktile = [&](int t) -> const char* { return smem + (t & 1) * TB; };

    // The first tile copies go out before Q's loads, so the two latencies
    // overlap (the wait below covers both).
    load_k(0);
    load_v(0);
    load_k(1);
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
    // Q (and the first tile copies) have landed before the key loop. (A wait
    // the compiler can see: otherwise it keeps Q's loads pending on paths
    // that skip the first use and re-waits inside the key loop, where vmcnt
    // also counts the tile copies in flight.)
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    // Key tiles [0, nfull) need no mask for any wave of the workgroup; tiles
    // [nfull, nkt) cross the causal diagonal or the end of the sequence.
    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const int nkt = (kend + BC - 1) / BC;
    const int nfull = (CAUSAL ? min(qtile0 + 1, N) : N) / BC;

    // Lane byte offsets into a swizzled tile (see lds_swz16):
    //  K fragment (ch, kb): ka[ch % NKA] + NKA*32*(ch / NKA) + 32*kb*RB.
    //  V^T fragment (t, u, db): row 16*t + 8*hi + 4*u + (lane%16)/4, bytes
    //    64*db + 32*((lane%32)/16) + 8*(lane%4): va[db % NVA] + NVA*64*(db / NVA)
    //    for u = 0; u = 1 (rows + 4) flips the chunk's bit 0 in the swizzle,
    //    so its offset is va + 4*RB +- 16 (vstep).
    int ka[W::NKA];
    uint32_t va[NVA], vstep;
    {
        const int kr = krow_perm(l32);
#pragma unroll
        for (int ch = 0; ch < W::NKA; ++ch)
            ka[ch] = kr * RB + (((2 * ch + hi) ^ lds_swz16<D>(kr)) * 16);
        const int vr = 8 * hi + (lane & 15) / 4;
#pragma unroll
        for (int db = 0; db < NVA; ++db) {
            const int chunk = 4 * db + 2 * (l32 / 16) + ((lane & 3) >> 1);
            va[db] = vr * RB + ((chunk ^ lds_swz16<D>(vr)) * 16) + 8 * (lane & 1);
        }
        vstep = 4 * RB + (((lane & 3) >> 1) ? -16 : 16);
    }
    int vai[NVA];
#pragma unroll
    for (int i = 0; i < NVA; ++i) vai[i] = (int)va[i];
    const int vsi = (int)vstep;
    // V read bases of a tile at LDS address base.
    auto vbases = [&](uint32_t base, uint32_t (&b0)[NVA], uint32_t (&b1)[NVA]) {
#pragma unroll
        for (int i = 0; i < NVA; ++i) {
            b0[i] = base + va[i];
            b1[i] = b0[i] + vstep;
        }
    };

    W st;
    st.init();
    f32x16 s[QB][NKB];


    // Invariant at the top of step t: K_t, V_t and (if any) K_{t+1} are in
    // LDS. Step t fills the slots of K_{t-1}/K_t and V_{t-1} that every wave
    // finished with before the previous barrier.
    wait_vm_all();
    __syncthreads();
    if (nfull > 0) {
        W::scores(s, ktile(0), ka, qf);
        float mt[QB];
        W::tile_max(s, c, mt);                // first reference maximum: exact
        st.raise_max(mt);
        __syncthreads();                     // all waves done reading K_0's slot
    }
    int t = 0;
    // Pipelined full tiles: the scores of tile t+1 are computed while the
    // softmax of tile t runs; two tiles per trip, the scores alternating
    // between s and s2.
    f32x16 s2[QB][NKB];
    auto full_step = [&](const f32x16 (&sc)[QB][NKB], f32x16 (&sn)[QB][NKB]) {
        load_k(t + 2);
        load_v(t + 1);
#if FA16_SCHED
        st.step(sc, sn, ktile(t + 1), ka, smem + (2 + (t & 1)) * TB, vai, vsi, qf, c);
#else
        uint32_t b0[NVA], b1[NVA];
        vbases(sbase + (2 + (t & 1)) * TB, b0, b1);
        st.overlap(sc, sn, ktile(t + 1), ka, b0, b1, qf, c);
#endif
        wait_vm_all();
        __syncthreads();
        ++t;
    };
    auto copy_back = [&]() {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = s2[qb][kb];
    };
    // Ping-pong ("FlashAttention-3", "Overlapping GEMM and Softmax"): waves
    // 0-3 and 4-7 of an 8-wave workgroup (the two waves of each SIMD) run
    // the same step, phase_a (score MFMAs of t+1, exponentials of t) and
    // phase_b (PV MFMAs of t), each ending in a workgroup barrier, but
    // waves 4-7 start one barrier late and waves 0-3 end one barrier
    // early. So while one wave of a SIMD runs its exponentials, the other
    // runs MFMAs. Only waves 0-3 copy tiles: K t+2 at the start of their
    // phase_a(t) (into the slot of K t, last read by waves 4-7 in their
    // phase_a(t-1), one barrier earlier), V t+1 at the start of their
    // phase_b(t) (the slot of V t-1, last read by waves 4-7 in their
    // phase_b(t-1)); each copy has landed at the barrier after the next
    // half, before its first reader.
    constexpr bool PP = FA16_PINGPONG && FA16_SCHED && NW == 8 && Cfg16<D, WIDE>::WPE == 2;
    if constexpr (PP) {
        constexpr int NL = NW / 2;                    // copying waves
        constexpr int NIWL = TB / 1024 / NL;
        const bool g0 = wave_u < NL;
        uint32_t loff[NIWL];
#pragma unroll
        for (int j = 0; j < NIWL; ++j) {
            const int p = ((wave & (NL - 1)) * NIWL + j) * 1024 + 16 * lane;
            const int row = p / RB;
            loff[j] = row * RB + ((p % RB / 16) ^ lds_swz16<D>(row)) * 16;
        }
        // copy tile tt into slot, by waves 0-3; true if issued
        auto pcopy = [&](const i32x4& rs, int tt, int slot) -> bool {
            if (tt >= nkt_use) return false;
            if (g0) {
                const uint32_t dst = sbase + slot * TB + (wave_u & (NL - 1)) * NIWL * 1024;
#pragma unroll
                for (int j = 0; j < NIWL; ++j) buffer_load_lds16(rs, dst + j * 1024, loff[j], tt * TB);
            }
            return true;
        };
        auto sync_after = [&](bool issued) {
            if (issued) sync_tiles<NIWL>(); else sync_tiles<0>();
        };
        X8 pf[QB][W::NPV];
        // Slots by the parity P of t, known at compile time (steps come in
        // pairs from t = 0), so tile addresses are immediate offsets.
        auto pp_step = [&](const f32x16 (&sc)[QB][NKB], f32x16 (&sn)[QB][NKB], auto pc) {
            constexpr int P = decltype(pc)::value;
            const bool kc = pcopy(krs, t + 2, P);
            st.phase_a(sc, sn, smem + ((P + 1) & 1) * TB, ka, qf, c, pf);
            sync_after(kc);
            const bool vc = pcopy(vrs, t + 1, 2 + ((P + 1) & 1));
            st.phase_b(smem + (2 + P) * TB, vai, vsi, pf);
            sync_after(vc);
            ++t;
        };
        if (!g0) sync_tiles<0>();                     // waves 4-7 start one barrier late
        for (; t + 2 < nfull;) {
            pp_step(s, s2, std::integral_constant<int, 0>{});
            pp_step(s2, s, std::integral_constant<int, 1>{});
        }
        if (t + 1 < nfull) {
            pp_step(s, s2, std::integral_constant<int, 0>{});
            copy_back();
        }
        if (g0) sync_tiles<0>();                      // waves 0-3 end one barrier early
        sync_tiles<0>();
    } else if constexpr (Cfg16<D, WIDE>::WPE == 1) {
        // one wave per SIMD (d = 256): the accumulation registers hold O and
        // the scores, with no room for a second set; copied each tile
        for (; t + 1 < nfull;) {
            full_step(s, s2);
            copy_back();
        }
    } else {
        for (; t + 2 < nfull;) {
            full_step(s, s2);
            full_step(s2, s);
        }
        if (t + 1 < nfull) {                  // an odd number of them: the scores end in s2
            full_step(s, s2);
            copy_back();
        }
    }
    if (nfull > 0) {                          // last full tile: no next scores
        load_v(t + 1);
        uint32_t b0[NVA], b1[NVA];
        vbases(sbase + (2 + (t & 1)) * TB, b0, b1);
        st.finish(s, b0, b1, c);
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
            uint32_t b0[NVA], b1[NVA];
            vbases(sbase + (2 + (t & 1)) * TB, b0, b1);
            if (t == 0) {                      // first reference maximum: exact
                float mt[QB];
                W::tile_max(s, c, mt);
                st.raise_max(mt);
            }
            // the first key tile (rows with fewer than BC keys) is fed to the
            // PV product as P~ plus its rounding residue (see Wave16::finish)
            if constexpr (Cfg16<D, WIDE>::WPE == 1) {
                const int npass = wave_uniform(t == 0 ? 2 : 1);
                for (int pass = 0; pass < npass; ++pass) st.template finish<2>(s, b0, b1, c, (float)pass);
            } else {
                st.finish(s, b0, b1, c);
                if (t == 0) st.template finish<1>(s, b0, b1, c);
            }
        }
        wait_vm_all();
        __syncthreads();
    }

    // ---- epilogue: O = O^T / l~, LSE = ln2 * (m + log2 l) ----
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = pair_sum(st.l[qb]);
        const float lx = W::XS ? pair_sum(st.lx[qb]) : l;
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

template <typename T, int D, bool CAUSAL, bool OUT_F32, bool WIDE>
static hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    constexpr int BR = Cfg16<D, WIDE>::NW * 32 * Cfg16<D, WIDE>::QB;
    const int num_qtiles = (a.N + BR - 1) / BR;
    const long long nblk = (long long)num_qtiles * a.B * a.H;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((fa_fwd16_kernel<T, D, CAUSAL, OUT_F32, WIDE>), dim3((unsigned)nblk),
                       dim3(Cfg16<D, WIDE>::NW * 64), 0, s, static_cast<const T*>(a.q),
                       static_cast<const T*>(a.k), static_cast<const T*>(a.v), a.o, a.lse, a.N,
                       num_qtiles, (int)nblk, c);
    return hipGetLastError();
}

template <typename T, int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_w(const FwdArgs& a, hipStream_t s) {
    if constexpr (D == 64) {
        constexpr int BRW = Cfg16<64, true>::NW * 32 * Cfg16<64, true>::QB;
        if ((long long)a.B * a.H * ((a.N + BRW - 1) / BRW) >= kWideMinBlocks)
            return launch_t<T, D, CAUSAL, OUT_F32, true>(a, s);
    }
    return launch_t<T, D, CAUSAL, OUT_F32, false>(a, s);
}

template <typename T, int D>
static hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    if (a.causal)
        return a.out_f32 ? launch_w<T, D, true, true>(a, s) : launch_w<T, D, true, false>(a, s);
    return a.out_f32 ? launch_w<T, D, false, true>(a, s) : launch_w<T, D, false, false>(a, s);
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

// d = 128 goes to the 64-rows-per-wave pipelined kernel (fa_fwd16_pipe.hip,
// one wave per SIMD) with FA_FWD_PIPELINED, and by itself when the mask is
// off and N >= kPipeMinN. That kernel halves the LDS fragment reads per MFMA
// but a single wave issues the softmax alone, and with one 256-row
// workgroup per CU nothing hides a workgroup's fixed cost (Q loads, first
// tile, O stores). On MI355X it measured 1.5-2 % faster than this file's
// kernel (two waves per SIMD) on long non-causal sequences (N = 8192,
// 16384), level at N = 4096 and about 6 % slower with the causal mask,
// where the average workgroup sees half the keys.
constexpr int kPipeMinN = 8192;

hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t s) {
    if (a.d == 128 && (a.pipelined || (!a.causal && a.N >= kPipeMinN)))
        return launch_fwd16_pipe(a, bf16, s);
    return bf16 ? launch_ty<__bf16>(a, s) : launch_ty<_Float16>(a, s);
}

}  // namespace fa
