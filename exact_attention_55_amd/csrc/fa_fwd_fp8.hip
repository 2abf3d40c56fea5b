// fa_fwd_fp8.hip - fused attention forward on FP8 e4m3 inputs (gfx950).
//
// Sources: "FlashAttention-3: Fast & Accurate Attention with Asynchrony &
// Low-Precision", sections "New GPU Features on Hopper: WGMMA, TMA, FP8" (QK^T
// and PV on the FP8 matrix path, softmax and exponentials in higher
// precision) and "Incoherent Processing for FP8 Accuracy"; review
// "FlashAttention-3: почему внимание стало быстрее", section "Метод", item 3
// (block quantisation). Inputs are the packed tensors of fa_fp8_prep: e4m3
// codes plus one float32 scale per 128 rows of a head.
//
// Same structure as the 16-bit kernel (transposed score tile S^T = K Q^T,
// transposed output O^T += V^T P^T, reference maximum from the first tile
// with an overflow-checked redo, buffer loads straight into swizzled
// double-buffered LDS tiles, a hand-ordered pipeline of the next tile's
// score MFMAs with this tile's exponentials), with 32x32x64 e4m3 MFMA.
// Scale handling, per query block i and key tile j:
//  * logits: s = acc * sq_i * sk_j * softmax_scale; in the base-2 domain the
//    product c_j = sq_i * sk_j * softmax_scale * log2(e) is one scalar per
//    tile, folded into the fma that feeds exp2;
//  * P is quantised to e4m3 for the PV MFMA. The V block scale enters as
//    w_j = sv_j / sv_max (sv_max = largest V block scale of the head), split
//    as w_j = 2^e_j * f_j / 2 with f_j in [1, 2): the power of two rides in
//    the PV MFMA's scale byte for V (exact), and P' = 8 p f_j, with the
//    factor folded into the exponent, p' = exp2(s*c - m + log2(8 f_j)), so
//    the V block scale costs no extra VALU work. V prepared with
//    power-of-two block scales (fa_fp8_prep with FA_SCALE_POW2) has f_j = 1:
//    P' = 8 p, and a row dominated by the key at its exact maximum (p =
//    2^-kMaxMargin there, see below) takes that key's weight exactly. Other
//    f_j leave every P' with its e4m3 rounding of 2^-4 relative, including
//    that dominant one. (Folding all of w_j into P' would also push blocks
//    with small V scales into e4m3's subnormal range.) A tile whose P' sum
//    in some lane exceeds kBig8 = 448 (the e4m3 maximum) is redone with its
//    exact maximum, so every P' is <= 448. The reference maximum is set
//    kMaxMargin = 2 (log2 units) above an exact one, at the first tile and
//    at each redo: a row whose scores just jumped keeps two more powers of
//    two of headroom before the next redo (on the 0.1 % outlier inputs
//    5.2 -> 2.6 % of tiles redone), so at that point every P' is below 4
//    (f_j < 2), and P' >= 2 p keeps p >= 2^-7 normal;
//  * the row sum l accumulates the unquantised p (rowsum(P') / (8 f_j));
//  * epilogue: O = O_acc * sv_max / (8 l).
// Microscaled inputs (fa_mx_prep: one power-of-two E8M0 scale per 32
// elements, along d for Q and K, along the sequence for V) take the scaled
// form of the same MFMA, which applies a per-lane scale byte to each 32
// k-values of A and of B: the score MFMAs take the Q and K bytes of their
// d-block, the PV MFMAs the V bytes of their 32-key block and 2^-3 for P'
// (so P' = 8p exactly as above, without w_j), the logits only the softmax
// scale, and the epilogue is O = O_acc / l. The scale bytes of a tile travel
// into LDS with the tile.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr float kPScale = 8.0f;     // P multiplier before e4m3 rounding
constexpr int kPScaleE8M0 = 124;    // 2^-3: the microscaled PV MFMA undoes kPScale
constexpr float kBig8 = 448.0f;     // per-lane tile sum of P' that forces the exact-maximum path
#ifndef FA8_MARGIN                 // reference maximum above the exact one it is set from (log2 units)
#define FA8_MARGIN 2.0f
#endif
#ifndef FA8_QS                     // 0: prescaled q runs the kernel with a multiply per score too
#define FA8_QS 1
#endif
#ifndef FA8_PAIRSYNC               // 0: block-scaled d = 128 key loop with a barrier per tile
#define FA8_PAIRSYNC 1
#endif
constexpr float kMaxMargin = FA8_MARGIN;

#ifndef FA8_PRIO                   // 0: the score phase runs at normal wave priority
#define FA8_PRIO 1
#endif
#ifndef FA8_KEEP                   // 0: the compiler may sink the next tile's score MFMAs behind the overflow check
#define FA8_KEEP 1
#endif
#ifndef FA8_RING                   // K and V tiles in LDS per workgroup (ring depth), 2 or 4
#define FA8_RING 2
#endif
#ifndef FA8_CFG_64
#define FA8_CFG_64 4, 64, 2
#endif
#ifndef FA8_CFG_128
#define FA8_CFG_128 4, 64, 2
#endif
#ifndef FA8_CFG_256
#define FA8_CFG_256 4, 64, 1
#endif
// NW waves of 32 query rows, BC keys per tile, WPE waves per SIMD budget.
template <int NW_, int BC_, int WPE_> struct Cfg8T {
    static constexpr int NW = NW_, BC = BC_, WPE = WPE_;
};
template <int D> struct Cfg8;
template <> struct Cfg8<64> : Cfg8T<FA8_CFG_64> {};
template <> struct Cfg8<128> : Cfg8T<FA8_CFG_128> {};
template <> struct Cfg8<256> : Cfg8T<FA8_CFG_256> {};

// Four floats -> four e4m3 bytes. The first conversion writes the low half
// of a register whose high half the second overwrites, so it starts from
// any value (a's bits: no register has to be zeroed first).
__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, __float_as_int(a), false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

// Per-lane E8M0 scale bytes of one tile for the microscaled path, kept as
// the loaded words (SW = ceil(d/128) words of 4 bytes): k[kb] holds the key
// row's bytes shifted right by 8*hi, so the score MFMA of k-step ch takes
// byte 2*ch of it; v holds the V bytes of the lane's d-row, byte db for
// d-block db. Unused (and optimised away) on the block-scaled path.
template <int NKB, int SW>
struct TileScales {
    uint32_t k[NKB][SW];
    uint32_t v[SW];
    // block-scaled path: E8M0 byte of the power-of-two part of the tile's V
    // block scale relative to the head's largest (see tile_scales)
    int vblk = 127;
    // block-scaled path with base-2 logits from the product: E8M0 byte of
    // the tile's K block scale (a power of two)
    int kblk = 127;
    __device__ __forceinline__ int kbyte(int kb, int ch) const {
        return (k[kb][ch >> 1] >> (16 * (ch & 1))) & 0xff;
    }
    __device__ __forceinline__ int vbyte(int db) const { return (v[db >> 2] >> (8 * (db & 3))) & 0xff; }
};

// ACC: O lives in the accumulation registers (one wave per SIMD); its rare
// rescale then runs in place.
template <int D, int BC, bool MX, bool ACC, bool QS>
struct Wave8 {
    static constexpr int RB = D;           // bytes per K / V row in LDS
    static constexpr int NCH = D / 64;     // k-steps of S^T = K Q^T
    static constexpr int NDB = D / 32;     // 32-row blocks of O^T
    static constexpr int NKB = BC / 32;    // 32-key blocks of S^T
    static constexpr int NPV = BC / 64;    // k-steps of O^T += V^T P'^T
    static constexpr int NVA = NDB;        // V lane offsets, one per d-block
    static constexpr int NKA = NCH;        // K lane offsets, per k-step (x2 chunks)
    static_assert(NKB == 2 * NPV, "one PV MFMA per two score blocks");
    using TS = TileScales<NKB, (D + 127) / 128>;

    // Score MFMA with the tile's scales (microscaled; or block-scaled with
    // base-2 logits, QS: the K and Q block scales as E8M0 bytes) or unit
    // scales.
    __device__ __forceinline__ f32x16 mm(const i32x8& a, const i32x8& b, const f32x16& c, int sa,
                                         int sb) const {
        if constexpr (MX || QS) return mfma32_fp8s(a, b, c, sa, sb);
        else return mfma32_fp8s(a, b, c, usc, usc);
    }
    // K scale operand of the score MFMA (key block kb, k-step ch)
    static __device__ __forceinline__ int kscale(const TS& ts, int kb, int ch) {
        return MX ? ts.kbyte(kb, ch) : (QS ? ts.kblk : 127);
    }
    static constexpr bool KS_HELD = MX || QS;   // per-tile K scale operands
    // P V MFMA of d-block db: microscaled, the V bytes of the block and 2^-3
    // for P'; block-scaled, the power-of-two part of the tile's V scale
    // (exact) and unit P'.
    // Scale operands are the one MFMA input the compiler lets a later
    // instruction overwrite too early: the matrix unit reads them when the
    // MFMA starts, which for the last of a run of back-to-back MFMAs is well
    // after its issue, and an LDS load landing in such a register right after
    // the PV block was seen to corrupt O (run to run). The PV scales are
    // therefore held in registers of their own (pvs) from just before their
    // block until the next PV block begins (a whole score phase later) or,
    // after finish(), until a read of the last PV result shows the block
    // done; the microscaled score MFMAs keep theirs the same way.
    // Constant scale operands (unit 2^0; 2^-3 for the microscaled P') live in
    // registers of their own for the same reason (usc, psc).
    static constexpr int NPS = MX ? NDB : 1;
    int pvs[NPS];
    int usc, psc;
    __device__ __forceinline__ void hold_pv_scales() {
#pragma unroll
        for (int i = 0; i < NPS; ++i) asm volatile("" ::"v"(pvs[i]));
        asm volatile("" ::"v"(usc), "v"(psc));
    }
    // (Re)load pvs for the tile with scales ts, after the previous block's
    // are released.
    __device__ __forceinline__ void set_pv_scales(const TS& ts) {
        hold_pv_scales();
#pragma unroll
        for (int i = 0; i < NPS; ++i) {
            pvs[i] = MX ? ts.vbyte(i) : ts.vblk;
            asm volatile("" : "+v"(pvs[i]));
        }
    }
    // P V MFMA of d-block db: microscaled, the V bytes of the block and 2^-3
    // for P'; block-scaled, the power-of-two part of the tile's V scale
    // (exact) and unit P'. Scales from pvs (set_pv_scales).
    __device__ __forceinline__ f32x16 mm_pv(const i32x8& a, const i32x8& b, const f32x16& c, int db) {
        return mfma32_fp8s(a, b, c, pvs[MX ? db : 0], psc);
    }
    // After a PV block with nothing of the kind behind it: a read of its last
    // result waits for the block, then pvs may go.
    __device__ __forceinline__ void settle_pv_block() {
        const int r = __builtin_amdgcn_readfirstlane(__float_as_int(o[NDB - 1][0]));
        asm volatile("" ::"s"(r));
        hold_pv_scales();
    }

    f32x16 o[NDB];
    float m, l;
    // QS (d = 128 only): the first score MFMA of every pipelined tile
    // starts from nmv = log2(8) - m instead of zero, so the product is the
    // exponent itself and the exponentials take no multiply-add (nmv kept
    // current across every move of m). (At d = 64 the 16 registers cost the
    // kernel its third wave per SIMD, at d = 256 they crowd the
    // accumulation registers, and the per-tile K scale operands cost more
    // than the multiply-adds they save: measured 2-4 % slower. Prescaled
    // inputs at those d take the plain kernel with unit logit multiplier.)
    static constexpr bool BAKE = QS;
    static_assert(!QS || D == 128, "the multiply-free form is built for d = 128");
    f32x16 nmv;
    __device__ __forceinline__ void set_nmv(float x) {
#pragma unroll
        for (int i = 0; i < 16; ++i) nmv[i] = x;
    }

    __device__ __forceinline__ void init() {
        m = -INFINITY;
        l = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
#pragma unroll
        for (int i = 0; i < NPS; ++i) {
            pvs[i] = 127;
            asm volatile("" : "+v"(pvs[i]));
        }
        usc = 127;
        psc = MX ? kPScaleE8M0 : 127;
        asm volatile("" : "+v"(usc), "+v"(psc));
        if constexpr (BAKE) set_nmv(0.f);
    }

    // K fragment (ch, kb): row perm(l32) + 32*kb, 16-byte logical chunks
    // 4*ch + 2*hi + e (block-scaled path) or 4*ch + hi + 2*e (microscaled
    // path), e = 0, 1; ka[ch][e] holds the swizzled lane offset (see
    // lds_swz8). The 64 k-values of one 8-bit MFMA operand are bytes 0-15 of
    // both half-waves for k 0-31 and bytes 16-31 for k 32-63, and the scale
    // of half-wave h covers k [32h, 32h + 32): with the microscaled chunk
    // order that range is d-block 2*ch + h of the row.
    static __device__ __forceinline__ i32x8 kfrag(const char* kl, const int (&ka)[NKA][2], int ch, int kb) {
        const char* p = kl + 32 * kb * RB;
        const u32x4 a0 = *reinterpret_cast<const u32x4*>(p + ka[ch][0]);
        const u32x4 a1 = *reinterpret_cast<const u32x4*>(p + ka[ch][1]);
        return i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                     (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
    }

    // All score MFMAs of a tile back to back (first and ragged tiles); the
    // microscaled K scale operands stay held until a read of the last score
    // shows the MFMAs done (see pvs).
    __device__ __forceinline__ void qk(f32x16 (&s)[NKB], const i32x8 (&kf)[NKB][NCH],
                                       const i32x8 (&qf)[NCH], const TS& ts, const int (&qs)[NCH]) {
        int ks[NCH][NKB];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) {
                ks[ch][kb] = kscale(ts, kb, ch);
                if (KS_HELD) asm volatile("" : "+v"(ks[ch][kb]));
            }
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = mm(kf[kb][ch], qf[ch], s[kb], ks[ch][kb], qs[ch]);
        if constexpr (KS_HELD) {
            const int r = __builtin_amdgcn_readfirstlane(__float_as_int(s[NKB - 1][0]));
            asm volatile("" ::"s"(r));
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) asm volatile("" ::"v"(ks[ch][kb]));
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) asm volatile("" ::"v"(qs[ch]));
        }
    }

    __device__ __forceinline__ void scores(f32x16 (&s)[NKB], const char* kl, const int (&ka)[NKA][2],
                                           const i32x8 (&qf)[NCH], const TS& ts, const int (&qs)[NCH]) {
        i32x8 kf[NKB][NCH];
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) kf[kb][ch] = kfrag(kl, ka, ch, kb);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = f32x16{};
        qk(s, kf, qf, ts, qs);
    }

    template <bool CAUSAL>
    static __device__ __forceinline__ void mask(f32x16 (&s)[NKB], int k0, int q0, int N, int hi,
                                                int l32) {
        const int q = q0 + l32;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int key = k0 + key_of(kb, r, hi);
                if (key >= N || (CAUSAL && key > q)) s[kb][r] = -INFINITY;
            }
    }

    // Row maximum of the tile in log2 units (cj > 0 commutes with max).
    static __device__ __forceinline__ float tile_max(const f32x16 (&s)[NKB], float cj) {
        float part[NKB * 4];
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
            for (int g = 0; g < 4; ++g)
                part[4 * kb + g] = fmaxf(fmaxf(s[kb][4 * g], s[kb][4 * g + 1]),
                                         fmaxf(s[kb][4 * g + 2], s[kb][4 * g + 3]));
#pragma unroll
        for (int w = NKB * 4; w > 1; w /= 2)
#pragma unroll
            for (int i = 0; i < w / 2; ++i) part[i] = fmaxf(part[i], part[i + w / 2]);
        return pair_max(part[0]) * cj;
    }

    // Moves the reference maximum to max(m, mt + kMaxMargin) (mt: an exact
    // tile maximum), rescaling O and l.
    __device__ __forceinline__ void raise_max(float mt) {
        const float mnew = fmaxf(m, mt + kMaxMargin);
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(m - mnew);
        m = mnew;
        l *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
            if (ACC)
                scale_acc(o[db], alpha);
            else
                o[db] *= alpha;
        }
    }

    // P' for score blocks 2t, 2t+1 -> PV operand t. Dword g of the operand
    // holds the e4m3 bytes of registers 4*(g%4)..+3 of score block 2t + g/4;
    // group q = 8t + g of the tile.
    // FMA: p' = exp2(s cj + nm) (nm = log2(8 f_j) - m); otherwise the scores
    // already are that exponent (BAKE pipelined tiles) and p' = exp2(s).
    template <bool FMA = true>
    __device__ __forceinline__ void prob_group(const f32x16 (&s)[NKB], uint32_t (&w)[NPV][8], int q,
                                               float cj, float nm, float (&ls)[2]) {
        const int t = q / 8, g = q % 8;
        const int kb = 2 * t + g / 4, r = 4 * (g % 4);
        auto ex = [&](float x) { return exp2_hw(FMA ? fmaf(x, cj, nm) : x); };
        const float p0 = ex(s[kb][r]);
        const float p1 = ex(s[kb][r + 1]);
        const float p2 = ex(s[kb][r + 2]);
        const float p3 = ex(s[kb][r + 3]);
        ls[g & 1] += (p0 + p1) + (p2 + p3);
        w[t][g] = cvt4_e4m3(p0, p1, p2, p3);
    }
    static __device__ __forceinline__ void pack_p(const uint32_t (&w)[NPV][8], i32x8 (&pf)[NPV]) {
#pragma unroll
        for (int t = 0; t < NPV; ++t)
            pf[t] = i32x8{(int)w[t][0], (int)w[t][1], (int)w[t][2], (int)w[t][3],
                          (int)w[t][4], (int)w[t][5], (int)w[t][6], (int)w[t][7]};
    }

    // Exponentials against the reference maximum; a tile whose P' sum in
    // some lane exceeds kBig8 is redone with its exact maximum (moving m,
    // rescaling O and l). Then l takes the tile's unquantised row sum.
    // The redo reads this tile's scores, so they stay in registers until
    // here, next to the next tile's (step pins those MFMAs before this
    // branch). The exponents are s cj + nm (nm = bj - m, or 0 for BAKE scores
    // that carry it); a score's logit in the units of m is that plus
    // m - bj. FIX (BAKE pipelined step): the next tile's scores sn, issued
    // with the old m, and nmv move with m.
    template <bool FIX>
    __device__ __forceinline__ void settle(const f32x16 (&s)[NKB], f32x16 (&sn)[NKB],
                                           uint32_t (&w)[NPV][8], float cj, float nm, float bj,
                                           float lscale, float (&ls)[2]) {
        if (wave_any(ls[0] + ls[1] > kBig8)) {
            const float m0 = m;
            raise_max(BAKE ? tile_max(s, cj) + (nm + m0 - bj) : tile_max(s, cj));
            const float delta = m0 - m;                        // <= 0
            const float nmr = BAKE ? nm + delta : bj - m;
            ls[0] = ls[1] = 0.f;
#pragma unroll
            for (int q = 0; q < 8 * NPV; ++q) prob_group(s, w, q, cj, nmr, ls);
            if constexpr (BAKE && FIX) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) sn[kb] += delta;
                nmv += delta;
            }
        }
        l += (ls[0] + ls[1]) * lscale;
    }

    // V^T fragment (t, db): slots 8c..8c+7 = keys 64t + 16c + 8hi + 0..7 of
    // d-row 32*db + l32; one transposing read of 8 rows per c. Bytes 0-15 of
    // both half-waves are keys 64t + [0, 32), bytes 16-31 keys 64t + [32, 64):
    // the two 32-key V scale blocks of the microscaled PV MFMA.
    static __device__ __forceinline__ i32x8 vfrag(const char* vl, const int (&va)[NVA], int t, int db) {
        const char* vp = vl + va[db] + 64 * t * RB;
        const u32x2 r0 = lds_read_tr8(vp);
        const u32x2 r1 = lds_read_tr8(vp + 16 * RB);
        const u32x2 r2 = lds_read_tr8(vp + 32 * RB);
        const u32x2 r3 = lds_read_tr8(vp + 48 * RB);
        return i32x8{(int)r0[0], (int)r0[1], (int)r1[0], (int)r1[1],
                     (int)r2[0], (int)r2[1], (int)r3[0], (int)r3[1]};
    }

    // Softmax + PV of the tile in s (no overlap). baked: the scores carry
    // log2(8) - m already (BAKE, issued by a pipelined step).
    __device__ __forceinline__ void finish(f32x16 (&s)[NKB], const char* vl,
                                           const int (&va)[NVA], float cj, float bj, float lscale,
                                           const TS& ts, bool baked = false) {
        uint32_t w[NPV][8];
        float ls[2] = {0.f, 0.f};
        const float nm = baked ? 0.f : bj - m;
#pragma unroll
        for (int q = 0; q < 8 * NPV; ++q) prob_group(s, w, q, cj, nm, ls);
        settle<false>(s, s, w, cj, nm, bj, lscale, ls);
        i32x8 pf[NPV];
        pack_p(w, pf);
        i32x8 vf[NPV][NDB];
#pragma unroll
        for (int t = 0; t < NPV; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db) vf[t][db] = vfrag(vl, va, t, db);
        set_pv_scales(ts);
#pragma unroll
        for (int t = 0; t < NPV; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db) o[db] = mm_pv(vf[t][db], pf[t], o[db], db);
        settle_pv_block();
    }

    // Pipelined step as one instruction stream in program order (every chunk
    // ends in a scheduling barrier): per score MFMA of the next tile (K at
    // kn), the LDS reads of the fragment KPD ahead (in the last chunks the
    // first VPD V^T fragments of this tile) and an even share of this tile's
    // exponential groups; the overflow check; per PV MFMA of this tile, the
    // reads of the V^T fragment VPD ahead. The next tile's scores go to sn
    // (the caller alternates two register sets, so nothing is copied).
    // tsn: scales of the next tile's score MFMAs; ts: this tile's PV scales.
    __device__ __forceinline__ void step(const f32x16 (&s)[NKB], f32x16 (&sn)[NKB], const char* kn,
                                         const int (&ka)[NKA][2], const char* vl, const int (&va)[NVA],
                                         const i32x8 (&qf)[NCH], float cj, float bj, float lscale,
                                         const TS& tsn, const TS& ts, const int (&qs)[NCH]) {
        constexpr int NKF = NCH * NKB;      // K fragments = score MFMAs per tile
        constexpr int NVF = NPV * NDB;      // V^T fragments = PV MFMAs per tile
        constexpr int NG = 8 * NPV;         // exponential groups (4 each) per lane
        constexpr int KPD = NKF >= 4 ? 2 : 1;
        constexpr int VPD = (NKF - KPD) < 2 ? (NKF - KPD) : 2;
        static_assert(VPD >= 1 && VPD < NVF, "tile too small for the read-ahead");
        // The score phase reads V^T fragments [0, min(KPD, VPD)), the PV loop
        // those from VPD on: every fragment is read only if KPD >= VPD.
        static_assert(KPD >= VPD, "V^T fragments [KPD, VPD) would never be read");
        i32x8 kf[NKB][NCH];
        i32x8 vf[NPV][NDB];
        uint32_t w[NPV][8];
        float ls[2] = {0.f, 0.f};
        // microscaled score MFMAs: their K scale operands, held until the PV
        // block (see pvs)
        int ks[NKF];
#pragma unroll
        for (int i = 0; i < NKF; ++i) {
            ks[i] = kscale(tsn, i % NKB, i / NKB);
            if (KS_HELD) asm volatile("" : "+v"(ks[i]));
        }
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            if constexpr (BAKE) sn[kb] = nmv;
            else sn[kb] = f32x16{};
        }
        const float nm = bj - m;
        if (FA8_PRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int f = 0; f < KPD; ++f) kf[f % NKB][f / NKB] = kfrag(kn, ka, f / NKB, f % NKB);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < NKF; ++i) {
            const int f = i + KPD;
            if (f < NKF) {
                kf[f % NKB][f / NKB] = kfrag(kn, ka, f / NKB, f % NKB);
            } else if (f - NKF < VPD) {
                const int v = f - NKF;
                vf[v / NDB][v % NDB] = vfrag(vl, va, v / NDB, v % NDB);
            }
            const int ch = i / NKB, kb = i % NKB;
            sn[kb] = mm(kf[kb][ch], qf[ch], sn[kb], ks[i], qs[ch]);
#pragma unroll
            for (int q = i * NG / NKF; q < (i + 1) * NG / NKF; ++q) prob_group<!BAKE>(s, w, q, cj, nm, ls);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FA8_PRIO) __builtin_amdgcn_s_setprio(0);
        // An empty use of each of the next tile's score tiles before the
        // overflow branch: without it the compiler sinks their MFMAs (whose
        // results are first read in the next step) behind the branch, where
        // they run back to back with the PV MFMAs instead of among the
        // exponentials. By this point the last of them is a chunk of
        // exponentials old, so the use costs no wait states. Not at d = 64:
        // the scores held together there cost the microscaled kernel its
        // third wave per SIMD (measured 8-11 % slower), and the block-scaled
        // one gains nothing.
        if (FA8_KEEP && D > 64) {
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) asm volatile("" ::"v"(sn[kb][0]));
        }
        settle<true>(s, sn, w, cj, BAKE ? 0.f : nm, bj, lscale, ls);
        i32x8 pf[NPV];
        pack_p(w, pf);
        if (KS_HELD) {
#pragma unroll
            for (int i = 0; i < NKF; ++i) asm volatile("" ::"v"(ks[i]));
        }
        set_pv_scales(ts);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < NVF; ++j) {
            const int v = j + VPD;
            if (v < NVF) vf[v / NDB][v % NDB] = vfrag(vl, va, v / NDB, v % NDB);
            const int t = j / NDB, db = j % NDB;
            o[db] = mm_pv(vf[t][db], pf[t], o[db], db);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
};

template <int D, bool CAUSAL, bool OUT_F32, bool MX, bool QS>
__global__ void __launch_bounds__(Cfg8<D>::NW * 64, Cfg8<D>::WPE)
fa_fwd_fp8_kernel(const uint8_t* __restrict__ Qg, const uint8_t* __restrict__ Kg,
                  const uint8_t* __restrict__ Vg, void* __restrict__ Og, float* __restrict__ LSEg,
                  int N, int num_qtiles, int num_blocks, int nsb, size_t scales_off, float c)
{
    constexpr int NW = Cfg8<D>::NW, BC = Cfg8<D>::BC;
    using W = Wave8<D, BC, MX, Cfg8<D>::WPE == 1, QS>;
    using TS = typename W::TS;
    constexpr int SBY = D / 32;            // microscaling: scale bytes per row of Q or K
    static_assert(!MX || W::NPV == 1, "microscaled V scales are held for one PV k-step per tile");
    constexpr int QW = 32, BR = NW * QW;
    // QS block-scaled: the waves of a workgroup share one Q scale block, so
    // the scale checks below agree across them
    static_assert(!QS || MX || kQuantBlockRows % BR == 0, "one Q scale block per workgroup");
    constexpr int NCH = W::NCH, NDB = W::NDB, NKB = W::NKB, NVA = W::NVA, RB = W::RB;
    constexpr int TB = BC * RB;            // bytes per K (or V) tile
    constexpr int NIW = TB / 1024 / NW;    // 1 KB direct loads per wave per tile
    static_assert(TB % (1024 * NW) == 0, "tile must split into 1 KB loads per wave");
    static_assert(kQuantBlockRows % BC == 0 && kQuantBlockRows % QW == 0, "scale blocks");

    // LDS: a ring of R slots for K tiles (tile t in slot t & (R - 1)), then
    // one for V tiles; microscaled path: then the tiles' scale bytes, R slots
    // for K and R for V, of SCB bytes each. Copies run R - 1 tiles ahead of
    // use. The key loop runs R tiles per trip, so every slot is a
    // compile-time offset there.
    // (d = 256 and the multiply-free form keep 2: with 4 they run out of
    // registers)
    // PS (block-scaled, d = 128): the pipelined tiles go in pairs with one
    // barrier per pair; a pair starting at even tile t copies K t+3, t+4 and
    // V t+2, t+3 into the slots the previous pair finished with (ring of 4),
    // and its closing barrier publishes them, so each copy has two steps to
    // land and a wave that falls behind (a redo) holds the others up once
    // per two tiles. Measured +2.5 % non-causal, neutral causal; the
    // microscaled kernel spills two registers with it and loses 2-3 %
    // causal, so it keeps a barrier per tile.
    constexpr bool PS = FA8_PAIRSYNC && D == 128 && !MX;
    constexpr int R = PS ? 4 : ((D == 256 || QS) ? 2 : FA8_RING);
    static_assert(R == 2 || R == 4, "ring depth");
    auto ring = [](int t) { return t & (R - 1); };
    constexpr int KSB = BC * (D / 32);     // K scale bytes of a tile (one row per key)
    constexpr int VSB = (BC / 32) * D;     // V scale bytes of a tile (32-key blocks)
    constexpr int SCB = (KSB > 256 ? KSB : 256);
    static_assert(SBY % 4 == 0 || KSB + 4 <= SCB, "room for the dword-aligned start of 2-byte scale rows");
    static_assert(KSB == VSB, "one scale slot size for K and V");
    // Block-scaled path: the K and V block scales of a tile travel with its V
    // tile into one of R BSB-byte slots (K floats, then V floats).
    constexpr int BSB = 512;
    __shared__ __attribute__((aligned(1024))) char smem[2 * R * TB + (MX ? 2 * R * SCB : R * BSB)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    const int wave_u = wave_uniform(wave);
    // Tiles are written only by direct global->LDS loads (invisible to the
    // compiler as stores); a store it cannot rule out keeps the reads alive.
    if (num_blocks < 0) smem[tid] = 0;

    // Workgroup -> (head, query tile) (see grid_tile); causal: heaviest first.
    int bh, qt;
    grid_tile(num_blocks, num_qtiles, CAUSAL, bh, qt);
    if (CAUSAL) qt = num_qtiles - 1 - qt;

    const size_t head = (size_t)bh * N * D;
    const uint8_t* Q = Qg + head;
    const uint8_t* K = Kg + head;
    const uint8_t* V = Vg + head;
    const float* Qs = reinterpret_cast<const float*>(Qg + scales_off) + (size_t)bh * nsb;
    const float* Ks = reinterpret_cast<const float*>(Kg + scales_off) + (size_t)bh * nsb;
    const float* Vs = reinterpret_cast<const float*>(Vg + scales_off) + (size_t)bh * nsb;
    const int qtile0 = qt * BR;
    const int q0 = qtile0 + wave * QW;

    // Block-scaled path: largest V block scale of the head. Microscaled
    // path: the matrix instructions apply every scale, the logits only take
    // softmax_scale * log2(e).
    // QS (q carries softmax_scale * log2(e), power-of-two block scales): the
    // logits need no multiplier; the Q and K block scales go to the score
    // MFMAs as E8M0 bytes, which needs every Q, K and V block scale of the
    // head to be a normal power of two (checked here; rows of a workgroup
    // whose scales are not get NaN).
    float svmax = 1.f, cq = QS ? 1.f : c;
    bool qs_ok = true;
    int qblk = 127;
    if constexpr (!MX) {
        svmax = 0.f;
        for (int i = lane; i < nsb; i += 64) {
            svmax = fmaxf(svmax, Vs[i]);
            if (QS) qs_ok = qs_ok && e8m0_of_pow2(Vs[i]) >= 0 && e8m0_of_pow2(Ks[i]) >= 0;
        }
#pragma unroll
        for (int mm = 32; mm >= 1; mm /= 2) svmax = fmaxf(svmax, __shfl_xor(svmax, mm, 64));
        const float sq = Qs[min(q0, N - 1) / kQuantBlockRows];
        if constexpr (QS) {
            qblk = e8m0_of_pow2(sq);
            qs_ok = !wave_any(!qs_ok || qblk < 0);
            qblk = wave_uniform(qblk);
        } else {
            cq = sq * c;
        }
    }
    const float rsvmax = 1.0f / svmax;

    // Tile copies: buffer loads straight into LDS (see fa_fwd16_kernel),
    // chunk swizzle lds_swz8; rows at or past N read as zeros.
    const i32x4 krs = make_rsrc(K, N * RB);
    const i32x4 vrs = make_rsrc(V, N * RB);
    uint32_t voff[NIW];
#pragma unroll
    for (int j = 0; j < NIW; ++j) {
        const int p = (wave * NIW + j) * 1024 + 16 * lane;
        const int row = p / RB;
        voff[j] = row * RB + ((p % RB / 16) ^ lds_swz8<D>(row)) * 16;
    }
    // row of the K tile this lane feeds to MFMA row l32 of score block 0
    const int krow0 = krow_perm(l32);
    // Microscaled path: E8M0 scale bytes. K of key row k: bytes
    // [k*SBY, +SBY) of the head's K scales; V of 32-key block kb, d-row r:
    // bytes [kb*D + (r % 32)*SBY, +SBY) (one byte per d-block). A tile's
    // bytes are contiguous in both (KSB = VSB bytes) and are copied into LDS
    // with the tile (wave 0, 4 bytes per lane, rows past the end read as
    // zeros). A lane of the score MFMA for key block kb, k-step ch takes K
    // byte 2*ch + hi of its key row; of the PV MFMA, V byte db of block
    // 2t + hi. With d = 64 (2 bytes per row) a head's K scales may start
    // 2 bytes into a dword and end inside one: the copy starts at the dword
    // below (kdelta bytes early, read back at +kdelta) and covers whole
    // dwords (bounds are checked per dword); the extra bytes lie inside the
    // packed buffer (its scale area is at least 2 bytes longer than the Q/K
    // scales whenever their total is not a whole number of dwords).
    const size_t nkb32 = ((size_t)N + 31) / 32;
    const size_t kso = (size_t)bh * N * SBY;
    const int kdelta = (int)(kso & 3);
    const i32x4 ksrs = make_rsrc(Kg + scales_off + kso - kdelta, MX ? (kdelta + N * SBY + 3) & ~3 : 0);
    const i32x4 vsrs = make_rsrc(Vg + scales_off + (size_t)bh * nkb32 * D, MX ? (int)(nkb32 * D) : 0);
    const uint32_t scbase = lds_addr(smem) + 2 * R * TB;
    auto load_sc = [&](const i32x4& rs, int t, int slot) {
        if (wave_u != 0) return;
        // 256 bytes per instruction; with KSB < 256 the upper lanes copy the
        // next tile's bytes (or zeros) into the unused end of the slot
#pragma unroll
        for (int i = 0; i < (KSB + 255) / 256; ++i)
            buffer_load_lds4(rs, scbase + slot * SCB + 256 * i, 4 * lane, t * KSB + 256 * i);
    };
    constexpr int SW = (SBY + 3) / 4;
    // scale words of the lane for the tile in K slot ks / V slot vs
    auto read_k = [&](TS& ts, int ks) {
        const char* p = smem + 2 * R * TB + ks * SCB + kdelta;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
            const char* q = p + (32 * kb + krow0) * SBY;
            uint32_t w0, w1 = 0;
            if constexpr (SBY == 2) w0 = *reinterpret_cast<const uint16_t*>(q);
            else if constexpr (SBY == 4) w0 = *reinterpret_cast<const uint32_t*>(q);
            else { const u32x2 x = *reinterpret_cast<const u32x2*>(q); w0 = x[0]; w1 = x[1]; }
            ts.k[kb][0] = w0 >> (8 * hi);
            if constexpr (SW > 1) ts.k[kb][1] = w1 >> (8 * hi);
        }
    };
    auto read_v = [&](TS& ts, int vs) {
        const char* q = smem + 2 * R * TB + (R + vs) * SCB + hi * D + l32 * SBY;
        if constexpr (SBY == 2) ts.v[0] = *reinterpret_cast<const uint16_t*>(q);
        else if constexpr (SBY == 4) ts.v[0] = *reinterpret_cast<const uint32_t*>(q);
        else { const u32x2 x = *reinterpret_cast<const u32x2*>(q); ts.v[0] = x[0]; ts.v[SW - 1] = x[1]; }
    };
    // Block-scaled path: 64 scale floats from the tile's block on (lane i:
    // block + i, past the head's end zeros) by one dword LDS-DMA each for K
    // and V; only the first is used. A global load here would make the
    // compiler wait for all vector memory traffic, the tile copies included.
    const i32x4 bks = make_rsrc(Ks, MX ? 0 : nsb * 4);
    const i32x4 bvs = make_rsrc(Vs, MX ? 0 : nsb * 4);
    auto load_bs = [&](int t, int s) {
        if (wave_u != 0) return;
        const int soff = (t * BC) / kQuantBlockRows * 4;
        buffer_load_lds4(bks, scbase + s * BSB, 4 * lane, soff);
        buffer_load_lds4(bvs, scbase + s * BSB + 256, 4 * lane, soff);
    };
    float tks = 1.f, tvs = 1.f;            // block scales of the tile whose softmax comes next
    auto read_bs = [&](int s) {
        if constexpr (!MX) {
            tks = uniform_f(*reinterpret_cast<const float*>(smem + 2 * R * TB + s * BSB));
            tvs = uniform_f(*reinterpret_cast<const float*>(smem + 2 * R * TB + s * BSB + 256));
        }
    };
    // QS block-scaled: E8M0 byte of K block scale idx of slot s (the slot of
    // tile t holds the scales of blocks t*BC/128 + 0, 1, ...; the tile's own
    // block and the next one). Every K scale of the head was checked to be a
    // normal power of two above, so its exponent is the byte.
    auto read_kblk = [&](TS& ts, int s, int idx) {
        if constexpr (QS && !MX) {
            const float f = uniform_f(*reinterpret_cast<const float*>(smem + 2 * R * TB + s * BSB + 4 * idx));
            ts.kblk = wave_uniform(126 + __builtin_amdgcn_frexp_expf(f));
        }
    };
    auto blk_of = [](int t) { return t * BC / kQuantBlockRows; };
    const int nkt_total = (N + BC - 1) / BC;
    const uint32_t sbase = lds_addr(smem);
    // copy of K (V = false) or V tile t into its ring slot
    auto load_kv = [&](const i32x4& rs, int t, bool V) {
        if (t >= nkt_total) return;
        const int slot = (V ? R : 0) + ring(t);
        if constexpr (MX) load_sc(V ? vsrs : ksrs, t, slot);
        else if (V) load_bs(t, ring(t));
        const uint32_t dst = sbase + slot * TB + wave_u * NIW * 1024;
#pragma unroll
        for (int j = 0; j < NIW; ++j) buffer_load_lds16(rs, dst + j * 1024, voff[j], t * TB);
    };
    auto ktile = [&](int t) -> const char* { return smem + ring(t) * TB; };
    auto vtile = [&](int t) -> const char* { return smem + (R + ring(t)) * TB; };
    // per-tile scale terms: score multiplier, P exponent offset, l weight;
    // block-scaled path also the V scale byte of the PV MFMAs (into vt)
    auto tile_scales = [&](float& cj, float& bj, float& lscale, TS& vt) {
        if constexpr (MX) {
            cj = QS ? 1.0f : c;
            bj = 3.0f;                                         // log2(kPScale)
            lscale = 1.0f / kPScale;
        } else {
            // w = sv_j / sv_max in (0, 1] is split as 2^(e-1) * f with f in
            // [1, 2): the power of two goes to the PV MFMA's V scale byte
            // (exact), only f into P' = 8 p f. Folding all of w into P'
            // would push the weights of blocks with small V scales into
            // e4m3's subnormal range, where they round coarsely. P' and l
            // share f, so the normalisation stays consistent. w is held at
            // >= 2^-126 so the byte stays in range (a block that much
            // weaker than the head's strongest is weighted 2^-126 instead).
            const float wv = fmaxf(tvs * rsvmax, 0x1p-126f);
            const int ex = __builtin_amdgcn_frexp_expf(wv);                 // >= -125
            const float f = 2.0f * __builtin_amdgcn_frexp_mantf(wv);       // [1, 2)
            if constexpr (QS) {                                      // w a power of two: f = 1
                cj = 1.0f;
                bj = 3.0f;
                lscale = 1.0f / kPScale;
            } else {
                cj = uniform_f(cq * tks);
                bj = uniform_f(__builtin_amdgcn_logf(kPScale * f));      // log2(8 f)
                lscale = uniform_f(__builtin_amdgcn_rcpf(kPScale * f));
            }
            vt.vblk = wave_uniform(126 + ex);                            // 2^(ex - 1)
        }
    };
    // The first tile copies go out before Q's loads, so the two latencies
    // overlap (the wait below covers both).
    load_kv(krs, 0, false);
    load_kv(vrs, 0, true);
    // per-step loop: K 1 .. R-1 and V 1 .. R-2 ahead; pairs: K 1, 2 and V 1
#pragma unroll
    for (int i = 1; i < (PS ? 3 : R); ++i) {
        load_kv(krs, i, false);
        if (i < (PS ? 2 : R - 1)) load_kv(vrs, i, true);
    }
    // Q^T fragments: query q0 + l32, bytes [64*ch + 32*hi, +32) (microscaled:
    // [64*ch + 16*hi, +16) and [64*ch + 32 + 16*hi, +16), the chunk order of
    // the K fragments); its MX scale byte 2*ch + hi of the row
    i32x8 qf[NCH];
    int qs[NCH];
    {
        const int row = q0 + l32;
        uint32_t qw[2] = {0x7f7f7f7fu, 0x7f7f7f7fu};
        if (MX && row < N) {
            const uint8_t* sp = Qg + scales_off + ((size_t)bh * N + row) * SBY;
            if constexpr (SBY == 2) {
                qw[0] = *reinterpret_cast<const uint16_t*>(sp);
            } else if constexpr (SBY == 4) {
                qw[0] = *reinterpret_cast<const uint32_t*>(sp);
            } else {
                const u32x2 x = *reinterpret_cast<const u32x2*>(sp);
                qw[0] = x[0];
                qw[1] = x[1];
            }
        }
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
            qs[ch] = MX ? (qw[ch >> 1] >> (16 * (ch & 1) + 8 * hi)) & 0xff : qblk;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            u32x4 a = u32x4{0, 0, 0, 0}, b = u32x4{0, 0, 0, 0};
            if (row < N) {
                const uint8_t* p = Q + (size_t)row * D + 64 * ch + (MX ? 16 : 32) * hi;
                a = *reinterpret_cast<const u32x4*>(p);
                b = *reinterpret_cast<const u32x4*>(p + (MX ? 32 : 16));
            }
            qf[ch] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                           (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        }
    }
    // Q and the first tile copies have landed (a wait the compiler sees; see
    // fa_fwd16_kernel).
    __builtin_amdgcn_s_waitcnt(kVmcnt0);
    if constexpr (QS && !MX) {
        if (!qs_ok) {                      // scales unusable as E8M0 bytes: NaN rows
            const int row = q0 + l32;
            if (row < N) {
                const float nan = __builtin_nanf("");
                if (hi == 0) LSEg[(size_t)bh * N + row] = nan;
                for (int col = hi; col < D; col += 2) {
                    const size_t off = head + (size_t)row * D + col;
                    if (OUT_F32) static_cast<float*>(Og)[off] = nan;
                    else static_cast<__bf16*>(Og)[off] = (__bf16)nan;
                }
            }
            return;
        }
    }

    // Lane offsets into swizzled tiles.
    int ka[W::NKA][2], va[NVA];
    {
        const int kr = krow0;
#pragma unroll
        for (int ch = 0; ch < W::NKA; ++ch)
#pragma unroll
            for (int e = 0; e < 2; ++e)
                ka[ch][e] = kr * RB + (((MX ? 4 * ch + hi + 2 * e : 4 * ch + 2 * hi + e)) ^ lds_swz8<D>(kr)) * 16;
        const int vr = 8 * hi + (lane & 15) / 2;
#pragma unroll
        for (int db = 0; db < NVA; ++db) {
            const int chunk = 2 * db + (l32 / 16);
            va[db] = vr * RB + ((chunk ^ lds_swz8<D>(vr)) * 16) + 8 * (lane & 1);
        }
    }

    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const int nkt = (kend + BC - 1) / BC;
    const int nfull = (CAUSAL ? min(qtile0 + 1, N) : N) / BC;

    W st;
    st.init();
    f32x16 s[NKB];

    // Scale registers (microscaled path): tk holds the K scales of the tile
    // whose scores come next, tv the V scales of the tile whose PV comes
    // next; the scales of a tile are requested with its copy and read after
    // the barrier that publishes it.
    TS tk, tv;
    TS tk2, tv2;                           // pairs: the same for the pair's second step
    wait_vm_all();
    __syncthreads();
    if constexpr (MX) {
        read_k(tk, 0);
        read_v(tv, 0);
    }
    read_bs(0);
    read_kblk(tk, 0, 0);
    if (nfull > 0) {
        float cj, bj, ls;
        tile_scales(cj, bj, ls, tv);
        st.scores(s, ktile(0), ka, qf, tk, qs);
        st.raise_max(W::tile_max(s, cj));    // first reference maximum: from the exact one
        if constexpr (W::BAKE) {
            // from here on the pipelined scores carry log2(8) - m
            const float nm = bj - st.m;
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] += nm;
            st.set_nmv(nm);
        }
        if constexpr (MX) read_k(tk, 1);
        read_kblk(tk, 0, blk_of(1) - blk_of(0));
        if constexpr (PS) {                  // the second step of the first pair
            if constexpr (MX) {
                read_k(tk2, 2);
                read_v(tv2, 1);
            }
            read_kblk(tk2, 0, blk_of(2) - blk_of(0));
        }
        __syncthreads();                     // all waves done reading K_0's slot
    }
    int t = 0;
    // Pipelined full tiles, two per trip: the scores alternate between s and
    // s2, so no step copies them.
    f32x16 s2[NKB];
    // Block-scaled path: the two key tiles of a 128-row scale block share
    // their scale terms, so the even tile computes them and the odd one
    // keeps them (and its scale floats are not read). The key loop runs
    // tiles in pairs, so the parity is known at compile time there.
    constexpr bool PAIR = !MX && 2 * BC == kQuantBlockRows;
    float pcj = 0.f, pbj = 0.f, pls = 0.f;
    auto full_step = [&](const f32x16 (&sc)[NKB], f32x16 (&sn)[NKB]) {
        load_kv(krs, t + R, false);
        load_kv(vrs, t + R - 1, true);
        if (!PAIR || (t & 1) == 0) tile_scales(pcj, pbj, pls, tv);
        st.step(sc, sn, ktile(t + 1), ka, vtile(t), va, qf, pcj, pbj, pls, tk, tv, qs);
        // K of t + 2 and V of t + 1 have landed. They were copied R - 2
        // steps ago; the copies of the steps since may stay in flight
        // (2 NIW tile copies per wave and step; wave 0, which also copies
        // scales, then waits for some of its newer copies too).
        if (R == 2) wait_vm_all();
        else wait_vm<(R - 2) * 2 * NIW>();
        __syncthreads();
        if constexpr (MX) {
            read_k(tk, ring(t + 2));           // tile t + 2
            read_v(tv, ring(t + 1));           // tile t + 1
        }
        if (!PAIR || (t & 1) == 1) read_bs(ring(t + 1));
        if (blk_of(t + 2) != blk_of(t + 1)) read_kblk(tk, ring(t + 1), 1);   // tile t + 2
        ++t;
    };
    // Tile pairs (t even): steps t and t + 1 use K t+1, t+2 and V t, t+1,
    // published by the previous pair's barrier (tk, tk2, tv, tv2 hold their
    // scales); the copies of K t+3, t+4 and V t+2, t+3 go into the slots of
    // K t-1, t and V t-2, t-1, which that barrier released.
    auto pair_steps = [&]() {
        static_assert(!PS || PAIR || MX, "a pair shares one scale block");
        load_kv(krs, t + 3, false);
        load_kv(krs, t + 4, false);
        load_kv(vrs, t + 2, true);
        load_kv(vrs, t + 3, true);
        tile_scales(pcj, pbj, pls, tv);      // block-scaled: tile t's block, shared by t + 1
        st.step(s, s2, ktile(t + 1), ka, vtile(t), va, qf, pcj, pbj, pls, tk, tv, qs);
        st.step(s2, s, ktile(t + 2), ka, vtile(t + 1), va, qf, pcj, pbj, pls, tk2, MX ? tv2 : tv, qs);
        wait_vm_all();
        __syncthreads();
        if constexpr (MX) {
            read_k(tk, ring(t + 3));
            read_k(tk2, ring(t + 4));
            read_v(tv, ring(t + 2));
            read_v(tv2, ring(t + 3));
        }
        read_bs(ring(t + 2));
        read_kblk(tk, ring(t + 2), blk_of(t + 3) - blk_of(t + 2));
        read_kblk(tk2, ring(t + 2), blk_of(t + 4) - blk_of(t + 2));
        t += 2;
    };
    if constexpr (PS) {
        // a pair at t needs full tiles t .. t+2 (its steps take the scores
        // of t+1 and t+2)
        for (; t + 4 < nfull; ) {            // two pairs per trip: every slot a constant
            pair_steps();
            pair_steps();
        }
        if (t + 2 < nfull) pair_steps();
        // back to the per-step invariant (K up to t+3, V up to t+2 copied):
        // K t+3 into the slot of K t-1, V t+2 into that of V t-2, both
        // released by the last barrier
        load_kv(krs, t + 3, false);
        load_kv(vrs, t + 2, true);
    } else {
        for (; t + R < nfull; ) {
#pragma unroll
            for (int u = 0; u < R; u += 2) {
                full_step(s, s2);
                full_step(s2, s);
            }
        }
    }
    // fewer than R full steps left; after an odd number of them the scores
    // are in s2
    bool odd = false;
#pragma unroll
    for (int u = 0; u < R - 1; ++u) {
        if (t + 1 < nfull) {
            if (u % 2 == 0) full_step(s, s2);
            else full_step(s2, s);
            odd = !odd;
        }
    }
    if (odd) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) s[kb] = s2[kb];
    }
    if (nfull > 0) {                          // last full tile
        if (R == 2) load_kv(vrs, t + 1, true);     // (with R = 4 already copied)
        float cj, bj, lscale;
        tile_scales(cj, bj, lscale, tv);
        st.finish(s, vtile(t), va, cj, bj, lscale, tv, W::BAKE);
        wait_vm_all();
        __syncthreads();
        if constexpr (MX) read_v(tv, ring(t + 1));   // the K scales of t + 1 are in tk already
        read_bs(ring(t + 1));
        read_kblk(tk, ring(t + 1), 0);
        ++t;
    }
    for (; t < nkt; ++t) {                    // ragged end / causal diagonal
        // one tile ahead (with R = 4 possibly a second copy of a tile already
        // there: the same bytes into a slot no wave reads in this iteration)
        load_kv(krs, t + 1, false);
        load_kv(vrs, t + 1, true);
        const int k0 = t * BC;
        if (!CAUSAL || k0 <= q0 + QW - 1) {
            float cj, bj, lscale;
            tile_scales(cj, bj, lscale, tv);
            st.scores(s, ktile(t), ka, qf, tk, qs);
            W::template mask<CAUSAL>(s, k0, q0, N, hi, l32);
            if (t == 0) st.raise_max(W::tile_max(s, cj));   // first reference maximum: from the exact one
            st.finish(s, vtile(t), va, cj, bj, lscale, tv);
        }
        wait_vm_all();
        __syncthreads();
        if constexpr (MX) {
            read_k(tk, ring(t + 1));
            read_v(tv, ring(t + 1));
        }
        read_bs(ring(t + 1));
        read_kblk(tk, ring(t + 1), 0);
    }

    // ---- epilogue: O = O_acc * sv_max / (8 l) (microscaled: O_acc / l, the
    // PV instruction already applied 2^-3), LSE = ln2 * (m + log2 l) ----
    const float l = pair_sum(st.l);
    const float inv = MX ? 1.0f / l : svmax / (kPScale * l);
    const int row = q0 + l32;
    if (row < N) {
        if (hi == 0) LSEg[(size_t)bh * N + row] = (st.m + __builtin_amdgcn_logf(l)) * kLn2;
#pragma unroll
        for (int db = 0; db < NDB; ++db) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int dcol = 32 * db + 8 * j + 4 * hi;
                const size_t off = head + (size_t)row * D + dcol;
                const float v0 = st.o[db][4 * j] * inv, v1 = st.o[db][4 * j + 1] * inv;
                const float v2 = st.o[db][4 * j + 2] * inv, v3 = st.o[db][4 * j + 3] * inv;
                if (OUT_F32) {
                    *reinterpret_cast<f32x4*>(static_cast<float*>(Og) + off) = f32x4{v0, v1, v2, v3};
                } else {
                    const bf16x2 a = {(__bf16)v0, (__bf16)v1}, b = {(__bf16)v2, (__bf16)v3};
                    *reinterpret_cast<u32x2*>(static_cast<__bf16*>(Og) + off) =
                        u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
                }
            }
        }
    }
}

template <int D, bool CAUSAL, bool OUT_F32, bool MX, bool QS>
static hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    constexpr int BR = Cfg8<D>::NW * 32;
    const int num_qtiles = (a.N + BR - 1) / BR;
    const long long nblk = (long long)num_qtiles * a.B * a.H;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int nsb = (a.N + kQuantBlockRows - 1) / kQuantBlockRows;
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, OUT_F32, MX, QS>), dim3((unsigned)nblk),
                       dim3(Cfg8<D>::NW * 64), 0, s, static_cast<const uint8_t*>(a.q),
                       static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.o,
                       a.lse, a.N, num_qtiles, (int)nblk, nsb, a.scales_off, a.qscaled ? 1.0f : a.scale * kLog2e);
    return hipGetLastError();
}

template <int D, bool MX, bool QS>
static hipError_t launch_m(const FwdArgs& a, hipStream_t s) {
    if (a.causal)
        return a.out_f32 ? launch_t<D, true, true, MX, QS>(a, s) : launch_t<D, true, false, MX, QS>(a, s);
    return a.out_f32 ? launch_t<D, false, true, MX, QS>(a, s) : launch_t<D, false, false, MX, QS>(a, s);
}

// Prescaled q (FA_FP8_QSCALED): the multiply-free kernel at d = 128; at
// other d the plain kernel, whose logit multiplier sq * sk * c then takes
// c = 1 (q already carries softmax_scale * log2(e)).
template <int D>
static hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    if constexpr (D == 128 && FA8_QS) {
        if (a.qscaled) return a.mx ? launch_m<D, true, true>(a, s) : launch_m<D, false, true>(a, s);
    }
    return a.mx ? launch_m<D, true, false>(a, s) : launch_m<D, false, false>(a, s);
}

hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return launch_d<64>(a, s);
        case 128: return launch_d<128>(a, s);
        case 256: return launch_d<256>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace fa
