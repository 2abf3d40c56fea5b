// fa_fwd16_pipe.hip - 16-bit fused attention forward with 64 query rows per
// wave and a three-stage pipeline inside each wave (gfx950, d = 128).
//
// Method: the same exact attention and online softmax as fa_fwd16.hip
// ("FlashAttention - one, two, three!" (Medium), "FlashAttention v1." and
// "FlashAttention v2.": blocks of K and V through on-chip memory, running row
// maximum and denominator, one normalisation at the end), with the
// intra-warpgroup overlap of "FlashAttention-3: Fast & Accurate Attention with
// Asynchrony & Low-Precision", "Overlapping GEMM and Softmax (Asynchrony)",
// carried to a gfx950 wave: while the exponentials of one block of scores
// run on the vector unit, the matrix core computes the scores of the next
// block and the P V product of the previous one.
//
// Why 64 rows per wave: each 32x32x16 MFMA takes one operand from LDS (a K
// fragment for the scores, a V^T fragment for P V). With 32 query rows per
// wave every fragment feeds one MFMA, and at full matrix-core rate the LDS
// would have to deliver more than it can (the 32-row kernel measures LDS-
// bound). With 64 rows each fragment feeds two MFMAs, halving the LDS bytes
// per flop. The 64 rows need the register file of one wave per SIMD: O (64
// rows x 128 columns of fp32, 128 registers per lane) lives in the
// accumulation registers (AGPRs); Q, two blocks of scores and two blocks of
// P in the vector registers. With one wave per SIMD nothing else hides the
// softmax, so the wave overlaps it itself (the three-stage step below).
//
// Register files: the score MFMAs are compiler builtins whose results go to
// vector registers (this file is built with the VGPR form of the MFMA
// forced), so the exponentials read them directly. The P V MFMAs are
// written as inline asm with O bound to AGPRs ("+a"): O stays there for the
// whole kernel, with no copies. The compiler does not see those MFMAs as
// MFMAs, so the places that read O with vector instructions (the rare
// rescale, the epilogue) carry their own wait states, and every input of an
// asm MFMA is written well before it (P a half step earlier, V^T by LDS
// reads the compiler waits for).
//
// Key loop: K and V tiles of 64 keys go HBM -> LDS by buffer loads with an
// LDS destination into 4-deep rings (K three tiles ahead, V two), with one
// workgroup barrier per tile; a tile is consumed as two half steps of 32
// keys. Half step h (keys 32h .. 32h+31) runs, interleaved instruction by
// instruction in a fixed order: the score MFMAs of block h+1 (S^T = K Q^T),
// the exponentials of block h (P~ rounded to the 16-bit type, row sums), and
// the P V MFMAs of block h-1 (O^T += V^T P^T). The reference maximum is the
// exact maximum of block 0; a block whose sum of exponentials passes kBig in
// some lane is redone with its exact maximum (moving m, rescaling O and the
// sums), as in fa_fwd16.hip. Tiles that cross the causal diagonal or the end
// of the sequence go through the same pipelined steps with their scores
// masked, when the workgroup has at least one full tile before them;
// otherwise (rows that see at most 256 keys) they run one 32-key block at a
// time, unpipelined, and the first key tile also goes through the exact
// split of P (P~ plus its rounding residue) for rows that see few keys.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

constexpr float kBigP = 16384.0f;   // per-lane sum of p that forces the exact-maximum redo

#ifndef FA16P_NPF
#define FA16P_NPF 3                  // fragments read ahead of their first MFMA
#endif
#ifndef FA16P_MASKED_PIPE            // 0: masked tiles always one 32-key block at a time
#define FA16P_MASKED_PIPE 1
#endif
#ifndef FA16P_QB                     // 32-row query blocks per wave: 2 (one wave per SIMD,
#define FA16P_QB 2                   // 4 per workgroup) or 1 (two per SIMD, 8 per workgroup)
#endif

// O^T += V^T P^T with O held in the accumulation registers (mfma_acc, see
// the file header): the compiler does not treat these as MFMAs.

template <typename T, int D>
struct PipeWave {
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    static constexpr int QB = FA16P_QB;    // 32-row query blocks per wave
    static constexpr int RB = 2 * D;       // bytes per K / V row in LDS
    static constexpr int NCH = D / 16;     // k-steps of the score MFMA (K fragments per block)
    static constexpr int NDB = D / 32;     // 32-row blocks of O^T
    static constexpr int NVF = 2 * NDB;    // V^T fragments per 32-key block
    static constexpr int NKA = (D == 64) ? 4 : 8;
    static constexpr int NVA = (D == 64) ? 2 : 4;
    static constexpr int NPF = FA16P_NPF;
    static constexpr bool XS = std::is_same<T, __bf16>::value;   // fp32 sum for the LSE

    f32x16 o[QB][NDB];   // O^T, in AGPRs
    float m[QB];         // reference maximum, log2 units
    float l[QB];         // sum of the rounded P fed to the MFMA
    float lx[QB];        // fp32 sum of p (bf16: for the log-sum-exp)

    // lane offsets into a swizzled tile (see fa_fwd16_kernel): K fragments
    // at ka, the two transposing reads of a V^T fragment at va and vb
    int ka[NKA];
    int va[NVA];
    int vb[NVA];

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

    // K fragment ch of key block kb of the tile at kl (32 keys x 16 d).
    __device__ __forceinline__ X8 kfrag(const char* kl, int kb, int ch) const {
        return load16<X8>(kl + 32 * kb * RB + ka[ch % NKA] + NKA * 32 * (ch / NKA));
    }
    // V^T fragment f = (t, db) of key block kb of the tile at vl: keys
    // 32 kb + 16 t + .., d-rows 32 db + ..
    __device__ __forceinline__ X8 vfrag(const char* vl, int kb, int f) const {
        const int t = f / NDB, db = f % NDB;
        const int off = 32 * kb * RB + NVA * 64 * (db / NVA) + 16 * t * RB;
        const u32x2 lo = lds_read_tr16(vl + va[db % NVA] + off);
        const u32x2 hi4 = lds_read_tr16(vl + vb[db % NVA] + off);
        return __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
    }

    // ---- unpipelined pieces (first block, masked blocks) ----

    // S^T of one 32-key block for both query blocks.
    __device__ __forceinline__ void scores(f32x16 (&s)[QB], const char* kl, int kb,
                                           const X8 (&qf)[QB][NCH]) const {
        X8 kf[NCH];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) kf[ch] = kfrag(kl, kb, ch);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[qb] = mfma32(kf[ch], qf[qb][ch], s[qb]);
    }

    template <bool CAUSAL>
    static __device__ __forceinline__ void mask(f32x16 (&s)[QB], int k0, int q0, int N, int hi,
                                                int l32) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const int q = q0 + 32 * qb + l32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + key_of(0, r, hi);
                if (key >= N || (CAUSAL && key > q)) s[qb][r] = -INFINITY;
            }
        }
    }

    // Row maximum of the block in log2 units.
    static __device__ __forceinline__ void block_max(const f32x16 (&s)[QB], float c, float (&mt)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            float part[4];
#pragma unroll
            for (int g = 0; g < 4; ++g)
                part[g] = fmaxf(fmaxf(s[qb][4 * g], s[qb][4 * g + 1]), fmaxf(s[qb][4 * g + 2], s[qb][4 * g + 3]));
            mt[qb] = pair_max(fmaxf(fmaxf(part[0], part[1]), fmaxf(part[2], part[3]))) * c;
        }
    }

    // The first reference maximum: O, l and lx are still zero, so nothing
    // is rescaled (touching the zero O here would split its AGPR live range).
    __device__ __forceinline__ void first_max(const float (&mt)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) m[qb] = mt[qb];
    }

    // Moves the reference maximum to max(m, mt), rescaling O (in place in
    // the AGPRs, with its own wait states), l and lx.
    __device__ __forceinline__ void raise_max(const float (&mt)[QB]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            const float mnew = fmaxf(m[qb], mt[qb]);
            const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(m[qb] - mnew);
            m[qb] = mnew;
            l[qb] *= alpha;
            lx[qb] *= alpha;
#pragma unroll
            for (int db = 0; db < NDB; ++db) scale_acc(o[qb][db], alpha);
        }
    }

    // One pair of exponentials of the block: values 8t + 2j, +1 of query
    // block qb, into elements 2j, 2j+1 of the P operand p[qb][t]. RESID: the
    // rounding residue p - P~ instead (exact split).
    template <bool RESID = false>
    __device__ __forceinline__ void pair(const f32x16 (&s)[QB], X8 (&p)[QB][2], int qb, int t, int j,
                                         float c, float (&ls)[QB][2], float (&lxs)[QB][2]) const {
        float p0 = exp2_hw(fmaf(s[qb][8 * t + 2 * j], c, -m[qb]));
        float p1 = exp2_hw(fmaf(s[qb][8 * t + 2 * j + 1], c, -m[qb]));
        if constexpr (RESID) {
            const X2 r = pack2<T>(p0, p1);
            p0 -= (float)r[0];
            p1 -= (float)r[1];
        } else if constexpr (XS) {
            lxs[qb][t] += p0 + p1;
        }
        const X2 r = pack2<T>(p0, p1);
        p[qb][t][2 * j] = r[0];
        p[qb][t][2 * j + 1] = r[1];
        ls[qb][t] = sum2(r, ls[qb][t]);
    }

    static __device__ __forceinline__ void zero_sums(float (&ls)[QB][2], float (&lxs)[QB][2]) {
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) ls[qb][0] = ls[qb][1] = lxs[qb][0] = lxs[qb][1] = 0.f;
    }

    // All exponentials of a block, then the overflow check (see settle).
    template <bool RESID = false>
    __device__ __forceinline__ void probs(const f32x16 (&s)[QB], X8 (&p)[QB][2], float c) {
        float ls[QB][2], lxs[QB][2];
        zero_sums(ls, lxs);
#pragma unroll
        for (int e = 0; e < 8 * QB; ++e) pair<RESID>(s, p, e / 8, (e / 4) % 2, e % 4, c, ls, lxs);
        if constexpr (RESID) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) l[qb] += ls[qb][0] + ls[qb][1];
        } else {
            settle(s, p, c, ls, lxs);
        }
    }

    // A block whose exponentials sum past kBigP in some lane is redone with
    // its exact maximum (every p is then <= 1 at the row's maximum); then the
    // block's sums join l and lx.
    __device__ __forceinline__ void settle(const f32x16 (&s)[QB], X8 (&p)[QB][2], float c,
                                           float (&ls)[QB][2], float (&lxs)[QB][2]) {
        // The check reads the sum of the rounded P (the bound is loose, so the
        // rounding does not matter): that keeps the conversions and the
        // rounded sums in their MFMA slots; with a check on the fp32 sum the
        // compiler sinks them below the branch, out of the overlap.
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) big |= ls[qb][0] + ls[qb][1] > kBigP;
        if (wave_any(big)) {
            float mt[QB];
            block_max(s, c, mt);
            raise_max(mt);
            zero_sums(ls, lxs);
#pragma unroll
            for (int e = 0; e < 8 * QB; ++e) pair(s, p, e / 8, (e / 4) % 2, e % 4, c, ls, lxs);
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l[qb] += ls[qb][0] + ls[qb][1];
            if (XS) lx[qb] += lxs[qb][0] + lxs[qb][1];
        }
    }

    // O^T += V^T P^T for one 32-key block of the tile at vl, right after
    // the vector instructions that wrote p: the asm MFMAs carry no hazard
    // tracking, so two wait states separate them from those writes (the
    // empty operands order the nop after the writes and the MFMAs after it).
    __device__ __forceinline__ void pv(const char* vl, int kb, X8 (&p)[QB][2]) {
        asm volatile("s_nop 1" : "+v"(p[0][0]), "+v"(p[0][1]), "+v"(p[1][0]), "+v"(p[1][1]));
        X8 vf[NVF];
#pragma unroll
        for (int f = 0; f < NVF; ++f) vf[f] = vfrag(vl, kb, f);
#pragma unroll
        for (int f = 0; f < NVF; ++f)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) mfma_acc(o[qb][f % NDB], vf[f], p[qb][f / NDB]);
    }

    // Fragment R of a step's stream: K0 V0 K1 V1 .. (both), K0 K1 .. or V0 V1 ..
    template <int R, bool RN, bool RP>
    __device__ __forceinline__ X8 sread(const char* kl, int kbk, const char* vl, int kbv) const {
        if constexpr (RN && RP) {
            if constexpr (R % 2 == 0) return kfrag(kl, kbk, R / 2);
            else return vfrag(vl, kbv, R / 2);
        } else if constexpr (RN) {
            return kfrag(kl, kbk, R);
        } else {
            return vfrag(vl, kbv, R);
        }
    }

    // ---- the pipelined half step ----
    //
    // NEXT: score MFMAs of the next block (K at kn, block kbn) into sn.
    // PREV: P V MFMAs of the previous block (pp_ at V vp, block kbp).
    // EXP: exponentials of this block (sc) into pc, then the overflow check.
    // The step's fragment stream (each fragment feeds QB consecutive MFMAs)
    // is K0 V0 K1 V1 .. with both, K0 K1 .. or V0 V1 .. with one. Its first
    // NPF fragments come in `pre`, read by the previous step; fragment r >=
    // NPF is read 2 NPF MFMAs before its first use, and in the step's last
    // MFMAs the first NPF fragments of the following step (kind NN / NP, at
    // kn2 / vp2 blocks kbn2 / kbp2) are read into `pre`.
    //
    // The exponentials are software-pipelined over the MFMA slots: a lone
    // wave issues in order, so a dependent chain inside one slot (fma ->
    // exp -> convert -> sum) would stall it while the matrix core idles.
    // Pair e (two scores) takes four stages in consecutive slots: the
    // exponent x = s c - m (written over sc), the two exponentials, the
    // 16-bit conversion with the pair's fp32 sum, then the dot2 into the
    // rounded-P row sum and the fp32 row sum; every instruction of a slot
    // reads results of earlier slots only. Pair starts are spread so the
    // last stage lands in the last slot.
    // NCP: global->LDS copy pieces issued by this step, piece k (cp(k)) at
    // slot k NS / NCP: spread out, since a copy holds up the wave's issue.
    template <bool NEXT, bool PREV, bool EXP, bool NN, bool NP, int NCP = 0, typename CP = int>
    __device__ __forceinline__ void step(f32x16 (&sn)[QB], f32x16 (&sc)[QB], X8 (&pc)[QB][2],
                                         const X8 (&pp_)[QB][2], X8 (&pre)[NPF], const X8 (&qf)[QB][NCH],
                                         const char* kn, int kbn, const char* vp, int kbp,
                                         const char* kn2, int kbn2, const char* vp2, int kbp2, float c,
                                         const CP& cp = 0) {
        constexpr int NF = (NEXT ? NCH : 0) + (PREV ? NVF : 0);    // fragments of this step
        constexpr int NS = NF * QB;                                 // MFMAs of this step
        constexpr int NF2 = (NN ? NCH : 0) + (NP ? NVF : 0);        // fragments of the next step
        constexpr int NPF2 = NF2 < NPF ? NF2 : NPF;
        constexpr int NE = EXP ? 8 * QB : 0;                        // exponential pairs
        static_assert(NF >= NPF, "step shorter than the read-ahead");
        static_assert(!EXP || NS >= 4, "too few slots for the exponential stages");
        X8 fr[NF];
#pragma unroll
        for (int r = 0; r < NPF; ++r) fr[r] = pre[r];
        float ls[QB][2], lxs[QB][2], e0[NE > 0 ? NE : 1], e1[NE > 0 ? NE : 1], ps[NE > 0 ? NE : 1];
        X2 rp[NE > 0 ? NE : 1];
        zero_sums(ls, lxs);
        if constexpr (NEXT) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sn[qb] = f32x16{};
        }
        float nm[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) nm[qb] = -m[qb];
        static_for<0, NS>([&](auto ic) {
            constexpr int i = decltype(ic)::value;
            if constexpr (NCP > 0) {
                static_assert(NS % NCP == 0, "copies spread evenly");
                if constexpr (i % (NS / NCP) == 0) cp(std::integral_constant<int, i / (NS / NCP)>{});
            }
            // read ahead: fragment i / QB + NPF of this step, or of the next
            if constexpr (i % QB == 0) {
                constexpr int rr = i / QB + NPF;
                if constexpr (rr < NF) {
                    fr[rr] = sread<rr, NEXT, PREV>(kn, kbn, vp, kbp);
                } else if constexpr (rr - NF < NPF2) {
                    pre[rr - NF] = sread<rr - NF, NN, NP>(kn2, kbn2, vp2, kbp2);
                }
            }
            // the MFMA of slot i
            constexpr int r = i / QB, qb_ = i % QB;
            constexpr bool isk = NEXT && (!PREV || r % 2 == 0);
            constexpr int idx = (NEXT && PREV) ? r / 2 : r;
            if constexpr (isk) {
                sn[qb_] = mfma32(fr[r], qf[qb_][idx], sn[qb_]);
            } else {
                mfma_acc(o[qb_][idx % NDB], fr[r], pp_[qb_][idx / NDB]);
            }
            // this slot's exponential stages
            if constexpr (EXP) {
                static_for<0, NE>([&](auto ec) {
                    constexpr int e = decltype(ec)::value;
                    constexpr int st0 = e * (NS - 3) / NE;             // stage 0 slot of pair e
                    constexpr int qb = e / 8, t = (e / 4) % 2, j = e % 4;
                    constexpr int v0 = 8 * t + 2 * j;
                    if constexpr (i == st0) {
                        sc[qb][v0] = fmaf(sc[qb][v0], c, nm[qb]);
                        sc[qb][v0 + 1] = fmaf(sc[qb][v0 + 1], c, nm[qb]);
                    } else if constexpr (i == st0 + 1) {
                        e0[e] = exp2_hw(sc[qb][v0]);
                        e1[e] = exp2_hw(sc[qb][v0 + 1]);
                    } else if constexpr (i == st0 + 2) {
                        rp[e] = pack2<T>(e0[e], e1[e]);
                        if (XS) ps[e] = e0[e] + e1[e];
                    } else if constexpr (i == st0 + 3) {
                        pc[qb][t][2 * j] = rp[e][0];
                        pc[qb][t][2 * j + 1] = rp[e][1];
                        ls[qb][t] = sum2(rp[e], ls[qb][t]);
                        if (XS) lxs[qb][t] += ps[e];
                    }
                });
            }
            __builtin_amdgcn_sched_barrier(0);
        });
        if constexpr (EXP) {
            // the fp32 sums stay in their slots: only the code after the
            // overflow branch reads them, and the compiler would sink them there
            if constexpr (XS) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) asm volatile("" : "+v"(lxs[qb][0]), "+v"(lxs[qb][1]));
            }
            settle_x(sc, pc, ls, lxs);
        }
    }

    // settle for a block whose scores were turned into exponents x = s c - m
    // in place: on overflow the maximum moves by the block's largest x (in
    // log2 units), O and the sums are rescaled, and P is recomputed as
    // exp2(x - that).
    __device__ __forceinline__ void settle_x(const f32x16 (&x)[QB], X8 (&p)[QB][2], float (&ls)[QB][2],
                                             float (&lxs)[QB][2]) {
        // The check reads the sum of the rounded P (the bound is loose, so the
        // rounding does not matter): that keeps the conversions and the
        // rounded sums in their MFMA slots.
        bool big = false;
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) big |= ls[qb][0] + ls[qb][1] > kBigP;
        if (wave_any(big)) {
            float xm[QB], mt[QB];
            block_max(x, 1.0f, xm);
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                xm[qb] = fmaxf(xm[qb], 0.f);      // m only moves up
                mt[qb] = m[qb] + xm[qb];
            }
            raise_max(mt);
            zero_sums(ls, lxs);
#pragma unroll
            for (int e = 0; e < 8 * QB; ++e) {
                const int qb = e / 8, t = (e / 4) % 2, j = e % 4, v0 = 8 * t + 2 * j;
                const float p0 = exp2_hw(x[qb][v0] - xm[qb]);
                const float p1 = exp2_hw(x[qb][v0 + 1] - xm[qb]);
                if (XS) lxs[qb][t] += p0 + p1;
                const X2 r = pack2<T>(p0, p1);
                p[qb][t][2 * j] = r[0];
                p[qb][t][2 * j + 1] = r[1];
                ls[qb][t] = sum2(r, ls[qb][t]);
            }
        }
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) {
            l[qb] += ls[qb][0] + ls[qb][1];
            if (XS) lx[qb] += lxs[qb][0] + lxs[qb][1];
        }
    }
};


template <typename T, int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(64 * 8 / FA16P_QB, 1)
fa_fwd16_pipe_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                     void* __restrict__ Og, float* __restrict__ LSEg, int N, int num_qtiles,
                     int num_blocks, float c)
{
    using W = PipeWave<T, D>;
    using X8 = typename W::X8;
    using X2 = typename W::X2;
    constexpr int QB = W::QB, NCH = W::NCH, NDB = W::NDB, RB = W::RB, NPF = W::NPF;
    constexpr int NW = 8 / QB;             // waves per workgroup: 256 query rows
    constexpr int QW = 32 * QB;            // query rows per wave
    constexpr int BR = NW * QW;            // query rows per workgroup
    constexpr int BC = 64;                 // keys per tile: two half steps
    constexpr int TB = BC * RB;            // bytes per K (or V) tile
    constexpr int NIW = TB / 1024 / NW;    // 1 KB copies per wave per tile and tensor
    constexpr int RING = 4;                // tiles per ring (K three ahead, V two)
    static_assert(TB % (1024 * NW) == 0, "tile must split into 1 KB loads per wave");

    // LDS: K ring (4 tiles), then V ring (4 tiles).
    __shared__ __attribute__((aligned(1024))) char smem[2 * RING * TB];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wave_u = wave_uniform(wave);
    if (num_blocks < 0) smem[tid] = 0;     // see fa_fwd16_kernel: keeps LDS reads defined

    int bh, qt;
    grid_tile(num_blocks, num_qtiles, CAUSAL, bh, qt);
    if (CAUSAL) qt = num_qtiles - 1 - qt;

    const size_t head = (size_t)bh * N * D;
    const T* Q = Qg + head;
    const int qtile0 = qt * BR;
    const int q0 = qtile0 + wave * QW;

    // Keys this workgroup reads: up to its last query row (causal) or N. The
    // copy range is cut there, so copies issued for tiles past it (the ring
    // issues a fixed number per tile, keeping the vmcnt arithmetic exact)
    // write zeros into their slot and read no memory.
    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const i32x4 krs = make_rsrc(Kg + head, kend * RB);
    const i32x4 vrs = make_rsrc(Vg + head, kend * RB);
    uint32_t voff[NIW];
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
        const int p = (wave * NIW + j) * 1024 + 16 * lane;
        const int row = p / RB;
        voff[j] = row * RB + ((p % RB / 16) ^ lds_swz16<D>(row)) * 16;
    }
    const uint32_t sbase = lds_addr(smem);
    auto issue = [&](const i32x4& rs, int t, int ring) {
        const uint32_t dst = sbase + (ring * RING + (t & (RING - 1))) * TB + wave_u * NIW * 1024;
#pragma unroll
        for (int j = 0; j < NIW; ++j) buffer_load_lds16(rs, dst + j * 1024, voff[j], (uint32_t)t * TB);
    };
    auto ktile = [&](int t) -> const char* { return smem + (t & (RING - 1)) * TB; };
    // V tile t (the ring's base is in the V lane offsets)
    auto vtile = [&](int t) -> const char* { return smem + (t & (RING - 1)) * TB; };

    // First copies (K 0..2, V 0..1) before Q's loads, so the latencies overlap.
    issue(krs, 0, 0);
    issue(krs, 1, 0);
    issue(krs, 2, 0);
    issue(vrs, 0, 1);
    issue(vrs, 1, 1);
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
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    W st;
    st.init();
    {
        const int kr = krow_perm(l32);
#pragma unroll
        for (int ch = 0; ch < W::NKA; ++ch)
            st.ka[ch] = kr * RB + (((2 * ch + hi) ^ lds_swz16<D>(kr)) * 16);
        const int vr = 8 * hi + (lane & 15) / 4;
#pragma unroll
        for (int db = 0; db < W::NVA; ++db) {
            const int chunk = 4 * db + 2 * (l32 / 16) + ((lane & 3) >> 1);
            st.va[db] = vr * RB + ((chunk ^ lds_swz16<D>(vr)) * 16) + 8 * (lane & 1);
        }
        // the V ring's base is folded into the V lane offsets, so that a V^T
        // read's slot, block and d offsets fit the 16-bit LDS immediate
        const int vstep = 4 * RB + (((lane & 3) >> 1) ? -16 : 16);
#pragma unroll
        for (int db = 0; db < W::NVA; ++db) {
            st.va[db] += RING * TB;
            st.vb[db] = st.va[db] + vstep;
        }
    }

    // Tiles [0, nfull) need no mask for any wave of the workgroup. When there
    // is at least one, the masked tiles after them (the causal diagonal, the
    // ragged end) also run through the pipelined steps, their scores masked
    // between the step that computes them and the one that takes their
    // exponentials; a workgroup with none (its rows see at most 256 keys)
    // takes the one-block-at-a-time path below, with the exact split of P.
    const int nkt = (kend + BC - 1) / BC;
    const int nfull = (CAUSAL ? min(qtile0 + 1, N) : N) / BC;
#if FA16P_MASKED_PIPE
    const int nloop = nfull > 0 ? nkt : 0;
#else
    const int nloop = nfull;
#endif
    // scores of 32-key block kb of tile t, before their exponentials
    auto mask_if = [&](f32x16 (&s)[QB], int t, int kb) {
        if (t >= nfull) W::template mask<CAUSAL>(s, t * BC + 32 * kb, q0, N, hi, l32);
    };

    // the copies of iteration j (K j+3 and V j+2: NIW pieces each, one
    // piece per call) into their ring slots
    auto copies = [&](int j) {
        const uint32_t kd = sbase + ((j + 3) & (RING - 1)) * TB + wave_u * NIW * 1024;
        const uint32_t vd = sbase + (RING + ((j + 2) & (RING - 1))) * TB + wave_u * NIW * 1024;
        const uint32_t ko = (uint32_t)(j + 3) * TB, vo = (uint32_t)(j + 2) * TB;
        return [=](auto pc) {
            constexpr int pce = decltype(pc)::value;
            if constexpr (pce < NIW) buffer_load_lds16(krs, kd + pce * 1024, voff[pce], ko);
            else buffer_load_lds16(vrs, vd + (pce - NIW) * 1024, voff[pce - NIW], vo);
        };
    };

    sync_tiles<0>();                       // K 0..2, V 0..1 visible

    f32x16 sA[QB], sB[QB];
    X8 pA[QB][2], pB[QB][2];
    X8 pre[NPF];
    if (nloop > 0) {
        // block 0: scores, and the reference maximum from them (exact)
        st.scores(sA, ktile(0), 0, qf);
        float mt[QB];
        W::block_max(sA, c, mt);
        st.first_max(mt);
        // the first step's first fragments: K of block 1
#pragma unroll
        for (int r = 0; r < NPF; ++r) pre[r] = st.kfrag(ktile(0), 1, r);
        // tile 0: half step 0 (scores of block 1, exponentials of block 0),
        // half step 1 (scores of block 2, exponentials of 1, P V of 0)
        const auto cp0 = copies(0);
        if (nloop > 1) {
            st.template step<true, false, true, true, true, 2 * NIW>(
                sB, sA, pA, pB, pre, qf, ktile(0), 1, nullptr, 0, ktile(1), 0, vtile(0), 0, c, cp0);
            st.template step<true, true, true, true, true>(
                sA, sB, pB, pA, pre, qf, ktile(1), 0, vtile(0), 0, ktile(1), 1, vtile(0), 1, c);
        } else {
            st.template step<true, false, true, false, true, 2 * NIW>(
                sB, sA, pA, pB, pre, qf, ktile(0), 1, nullptr, 0, nullptr, 0, vtile(0), 0, c, cp0);
            st.template step<false, true, true, false, true>(
                sA, sB, pB, pA, pre, qf, nullptr, 0, vtile(0), 0, nullptr, 0, vtile(0), 1, c);
        }
        // tiles 1 .. nfull-2: both half steps full; the tile copies of an
        // iteration are spread over its first half step
        int j = 1;
        for (; j + 1 < nloop; ++j) {
            sync_tiles<2 * NIW>();             // K j+2, V j+1 landed; K j-1, V j-2 free
            mask_if(sA, j, 0);
            st.template step<true, true, true, true, true, 2 * NIW>(
                sB, sA, pA, pB, pre, qf, ktile(j), 1, vtile(j - 1), 1, ktile(j + 1), 0, vtile(j), 0, c,
                copies(j));
            mask_if(sB, j, 1);
            st.template step<true, true, true, true, true>(
                sA, sB, pB, pA, pre, qf, ktile(j + 1), 0, vtile(j), 0, ktile(j + 1), 1, vtile(j), 1, c);
        }
        if (j < nloop) {                     // last tile: no scores after it
            sync_tiles<2 * NIW>();
            mask_if(sA, j, 0);
            st.template step<true, true, true, false, true, 2 * NIW>(
                sB, sA, pA, pB, pre, qf, ktile(j), 1, vtile(j - 1), 1, nullptr, 0, vtile(j), 0, c, copies(j));
            mask_if(sB, j, 1);
            st.template step<false, true, true, false, true>(
                sA, sB, pB, pA, pre, qf, nullptr, 0, vtile(j), 0, nullptr, 0, vtile(j), 1, c);
            ++j;
        }
        // drain: P V of the last block
        st.template step<false, true, false, false, false>(sA, sB, pA, pB, pre, qf, nullptr, 0,
                                                          vtile(nloop - 1), 1, nullptr, 0, nullptr, 0, c);
    }

    // Masked tiles (causal diagonal, ragged end) of a workgroup without a
    // full tile: one 32-key block at a time.
    for (int t = nloop; t < nkt; ++t) {
        sync_tiles<0>();                       // every copy issued so far has landed
        issue(krs, t + 3, 0);                  // K t-1, V t-2 are free
        issue(vrs, t + 2, 1);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
            const int k0 = t * BC + 32 * kb;
            if (k0 >= N || (CAUSAL && k0 > q0 + QW - 1)) continue;   // no visible key for this wave
            st.scores(sA, ktile(t), kb, qf);
            W::template mask<CAUSAL>(sA, k0, q0, N, hi, l32);
            if (t == 0 && kb == 0) {           // first reference maximum: exact
                float mt[QB];
                W::block_max(sA, c, mt);
                st.first_max(mt);
            }
            st.probs(sA, pA, c);
            st.pv(vtile(t), kb, pA);
            if (t == 0) {                      // rows that see few keys: the exact split of P
                st.template probs<true>(sA, pB, c);
                st.pv(vtile(t), kb, pB);
            }
        }
    }

    // ---- epilogue: O = O^T / l~, LSE = ln2 * (m + log2 l) ----
    // O was written by asm MFMAs: wait for the last of them before reading.
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) acc_settle(st.o[qb][0], st.o[qb][1], st.o[qb][2], st.o[qb][3]);
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

template <typename T, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    constexpr int D = 128, BR = 256;
    const int num_qtiles = (a.N + BR - 1) / BR;
    const long long nblk = (long long)num_qtiles * a.B * a.H;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const float c = a.scale * kLog2e;
    hipLaunchKernelGGL((fa_fwd16_pipe_kernel<T, D, CAUSAL, OUT_F32>), dim3((unsigned)nblk),
                       dim3(64 * 8 / FA16P_QB), 0, s,
                       static_cast<const T*>(a.q), static_cast<const T*>(a.k), static_cast<const T*>(a.v),
                       a.o, a.lse, a.N, num_qtiles, (int)nblk, c);
    return hipGetLastError();
}

template <typename T>
hipError_t launch_ty(const FwdArgs& a, hipStream_t s) {
    if (a.causal) return a.out_f32 ? launch_t<T, true, true>(a, s) : launch_t<T, true, false>(a, s);
    return a.out_f32 ? launch_t<T, false, true>(a, s) : launch_t<T, false, false>(a, s);
}

}  // namespace

hipError_t launch_fwd16_pipe(const FwdArgs& a, bool bf16, hipStream_t s) {
    if (a.d != 128) return hipErrorInvalidValue;
    return bf16 ? launch_ty<__bf16>(a, s) : launch_ty<_Float16>(a, s);
}

}  // namespace fa
