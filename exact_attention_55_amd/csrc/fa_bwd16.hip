// fa_bwd16.hip - gradients of the fused attention forward (bf16 / fp16, gfx950).
//
// Method: the attention probabilities are not stored by the forward; they
// are recomputed from Q, K and the saved per-row log-sum-exp ("FlashAttention
// - one, two, three!" (Medium), section "FlashAttention v1.": recomputation
// instead of keeping intermediate results, with a few per-row constants in
// global memory). The gradient is the chain rule through the "Standard
// Attention" definition of O = softmax(scale * Q K^T) V (same page):
//     P  = exp(scale * Q K^T - LSE)        (recomputed per tile)
//     dV = P^T dO,   dP = dO V^T,   D_i = sum_c dO_ic O_ic,
//     dS = P * (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Three kernels, no atomics and no scratch beyond the caller's row-constant
// array (D and -LSE/scale, 2 floats per row):
//  * bwd_delta_kernel: D = rowsum(dO * O) in fp32, and -LSE / scale.
//  * bwd_dq_kernel (one workgroup per 128 query rows, the forward's
//    structure): per key tile S^T = K Q^T and dP^T = V dO^T with K and V
//    rows read from LDS, dS^T in registers, dQ^T += K^T dS^T with K^T read
//    from the same LDS tile by transposing reads.
//  * bwd_dkv_kernel (one workgroup per 128 keys, the mirror image): per
//    query tile S = Q K^T and dP = dO V^T with Q and dO rows from LDS
//    (accumulators started from the row constants),
//    dV^T += dO^T P and dK^T += Q^T dS with dO^T and Q^T by transposing
//    reads. This costs two more GEMMs than a single pass with atomic dQ
//    updates (7 instead of 5 per tile pair) and keeps the result
//    deterministic.
// Tiles go global -> LDS by buffer loads (see fa_fwd16.hip); the LDS
// swizzle, the row permutation of the A operand (krow_perm) and the lane
// layouts are those of the forward.
// At d = 256 both gradient kernels run one wave per SIMD and keep their
// gradient accumulators (dQ^T: 128 registers; dK^T and dV^T: 256) in the
// accumulation registers for the whole kernel, through asm MFMAs
// (mfma_acc); the score and dP MFMAs are compiler builtins that write vector
// registers (this file is built with the VGPR form of the MFMA forced), so
// the exponentials read them directly. Inputs of an asm MFMA written by
// vector instructions (dS, P) pass through a two-wait-state barrier first,
// and the epilogue waits out the last MFMA's latency before reading.
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {
namespace {

template <typename T> struct Bw;
template <> struct Bw<__bf16> {
    using x8 = bf16x8;
    using x2 = bf16x2;
    static __device__ __forceinline__ x2 pack(float a, float b) { return x2{(__bf16)a, (__bf16)b}; }
};
template <> struct Bw<_Float16> {
    using x8 = f16x8;
    using x2 = f16x2;
    static __device__ __forceinline__ x2 pack(float a, float b) { return x2{(_Float16)a, (_Float16)b}; }
};

// Shared tile geometry: rows of 2*D bytes, 16-byte chunks XOR-swizzled with
// lds_swz16<D>. kfrag: A-operand fragment of a 32-row block, rows permuted
// by krow_perm (so that accumulator runs of 8 registers are 8 consecutive
// rows); tfrag: transposed A-operand fragment (d rows x 16 tile rows) by
// two transposing reads.
template <typename T, int D>
struct Tile {
    using X8 = typename Bw<T>::x8;
    static constexpr int RB = 2 * D;
    static constexpr int NCH = D / 16;
    static constexpr int NDB = D / 32;
    static constexpr int NKA = (D == 64) ? 4 : 8;
    static constexpr int NVA = (D == 64) ? 2 : 4;

    // row-fragment lane offsets (ka) and transposed-fragment offsets (va, vstep)
    int ka[NKA], va[NVA], vstep;

    __device__ __forceinline__ void init(int lane) {
        const int l32 = lane & 31, hi = lane >> 5;
        const int kr = krow_perm(l32);
#pragma unroll
        for (int ch = 0; ch < NKA; ++ch) ka[ch] = kr * RB + (((2 * ch + hi) ^ lds_swz16<D>(kr)) * 16);
        const int vr = 8 * hi + (lane & 15) / 4;
#pragma unroll
        for (int db = 0; db < NVA; ++db) {
            const int chunk = 4 * db + 2 * (l32 / 16) + ((lane & 3) >> 1);
            va[db] = vr * RB + ((chunk ^ lds_swz16<D>(vr)) * 16) + 8 * (lane & 1);
        }
        vstep = 4 * RB + (((lane & 3) >> 1) ? -16 : 16);
    }
    __device__ __forceinline__ X8 kfrag(const char* tl, int ch, int blk) const {
        return load16<X8>(tl + ka[ch % NKA] + NKA * 32 * (ch / NKA) + 32 * blk * RB);
    }
    // rows 16*t + 8*hi + (0..7) of d-block db
    __device__ __forceinline__ X8 tfrag(const char* tl, int t, int db) const {
        const char* p = tl + va[db % NVA] + NVA * 64 * (db / NVA) + 16 * t * RB;
        const u32x2 lo = lds_read_tr16(p);
        const u32x2 hi4 = lds_read_tr16(p + vstep);
        return __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
    }
};

// Waves per SIMD: two at d <= 128; one at d = 256, where the two d x 32
// gradient accumulators of the key-parallel kernel alone take 256 of a
// lane's 512 registers (the compiler keeps them in the accumulation
// registers) and the query-parallel kernel holds Q^T and dO^T fragments of
// 256 columns.
template <int D> constexpr int bwd_occupancy() { return D == 256 ? 1 : 2; }
// Fragments of a d-long operand loaded per batch before their MFMAs: the
// whole operand at d <= 128, a quarter of it at d = 256 (bounds the live
// registers).
template <int D> constexpr int bwd_batch() { return D == 256 ? D / 64 : D / 16; }

// acc += A B for a gradient accumulator: asm into the accumulation registers
// at d = 256 (see the file header), the builtin elsewhere.
template <int D, typename X8>
__device__ __forceinline__ void grad_mfma(f32x16& acc, const X8& a, const X8& b) {
    if constexpr (D == 256) mfma_acc(acc, a, b);
    else acc = mfma32(a, b, acc);
}
template <int D, int N>
__device__ __forceinline__ void grad_settle(f32x16 (&acc)[N]) {
    if constexpr (D == 256) {
#pragma unroll
        for (int i = 0; i + 3 < N; i += 4) acc_settle(acc[i], acc[i + 1], acc[i + 2], acc[i + 3]);
    }
}

// Global -> LDS tile copies for a [rows, D] tile of one head (see fa_fwd16).
template <int D, int TROWS, int NW>
struct Copier {
    static constexpr int RB = 2 * D;
    static constexpr int TB = TROWS * RB;
    static constexpr int NIW = TB / 1024 / NW;
    static_assert(TB % (1024 * NW) == 0, "tile must split into 1 KB loads per wave");
    uint32_t voff[NIW];
    uint32_t dst0;
    __device__ __forceinline__ void init(int wave, int lane, uint32_t sbase, int wave_u) {
#pragma unroll
        for (int j = 0; j < NIW; ++j) {
            const int p = (wave * NIW + j) * 1024 + 16 * lane;
            const int row = p / RB;
            voff[j] = row * RB + ((p % RB / 16) ^ lds_swz16<D>(row)) * 16;
        }
        dst0 = sbase + wave_u * NIW * 1024;
    }
    __device__ __forceinline__ void issue(const i32x4& rs, int tile, int slot) const {
#pragma unroll
        for (int j = 0; j < NIW; ++j) buffer_load_lds16(rs, dst0 + slot * TB + j * 1024, voff[j], tile * TB);
    }
};

// 16-bit row of the head-major output for the transposed accumulator of a
// lane (lane = row, register r of d-block db = column 32*db + 8*(r/4) +
// 4*hi + r%4), scaled.
template <typename T, int D, bool OUT_F32>
__device__ __forceinline__ void store_rowT(void* out, size_t off_row, const f32x16 (&acc)[D / 32],
                                           float mul, int hi) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const size_t off = off_row + 32 * db + 8 * j + 4 * hi;
            const float v0 = acc[db][4 * j] * mul, v1 = acc[db][4 * j + 1] * mul;
            const float v2 = acc[db][4 * j + 2] * mul, v3 = acc[db][4 * j + 3] * mul;
            if (OUT_F32) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(out) + off) = f32x4{v0, v1, v2, v3};
            } else {
                const auto a = Bw<T>::pack(v0, v1), b = Bw<T>::pack(v2, v3);
                *reinterpret_cast<u32x2*>(static_cast<T*>(out) + off) =
                    u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, b)};
            }
        }
}

// ---------------------------------------------------------------------------
// Per-row constants: D = rowsum(dO * O) (fp32, 8 lanes of 8 elements for
// d = 64, 16 for d = 128) and Lr = -LSE / scale, the value the key-parallel
// kernel starts its score accumulator from (so that scale * (acc) is the
// log-probability). Both land in the caller's scratch: D at [0, rows),
// Lr at [rows, 2 rows).
template <typename T, int D>
__global__ void __launch_bounds__(256) bwd_delta_kernel(const T* __restrict__ O, const T* __restrict__ dO,
                                                        const float* __restrict__ LSE,
                                                        float* __restrict__ Dout, long long rows,
                                                        float inv_scale) {
    using X8 = typename Bw<T>::x8;
    constexpr int LPR = D / 8;                         // lanes per row
    const long long tid = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long row = tid / LPR;
    const int part = (int)(tid % LPR);
    float acc = 0.f;
    if (row < rows) {
        const X8 a = load16<X8>(O + row * D + 8 * part);
        const X8 b = load16<X8>(dO + row * D + 8 * part);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc = fmaf((float)a[i], (float)b[i], acc);
    }
#pragma unroll
    for (int m = LPR / 2; m >= 1; m /= 2) acc += __shfl_xor(acc, m, 64);
    if (row < rows && part == 0) {
        Dout[row] = acc;
        Dout[rows + row] = -LSE[row] * inv_scale;
    }
}

// ---------------------------------------------------------------------------
// dQ: one workgroup = 4 waves x 32 query rows; key tiles of 64 (32 at
// d = 256, so that the score and dP tiles fit beside the fragments).
template <typename T, int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(256, bwd_occupancy<D>())
bwd_dq_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
              const T* __restrict__ dOg, const float* __restrict__ LSEg, const float* __restrict__ Dg,
              void* __restrict__ dQg, int N, int num_qtiles, int num_blocks, float c, float scale)
{
    using X8 = typename Bw<T>::x8;
    using TL = Tile<T, D>;
    constexpr int NW = 4, QW = 32, BR = NW * QW, BC = D == 256 ? 32 : 64;
    constexpr int NCH = TL::NCH, NDB = TL::NDB, RB = TL::RB;
    constexpr int NKB = BC / 32, NPV = BC / 16;
    constexpr int KB = bwd_batch<D>();       // K / V fragments per batch
    constexpr int TB4 = NDB < 4 ? NDB : 4;   // K^T fragments per batch
    using CP = Copier<D, BC, NW>;
    constexpr int TB = CP::TB;
    __shared__ __attribute__((aligned(1024))) char smem[4 * TB];   // K: slots 0,1; V: 2,3

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    if (num_blocks < 0) smem[tid] = 0;     // keeps the LDS reads alive (tiles come by DMA)

    // Workgroup -> (head, query tile) (see grid_tile); causal: heaviest first.
    int bh, qt;
    grid_tile(num_blocks, num_qtiles, CAUSAL, bh, qt);
    if (CAUSAL) qt = num_qtiles - 1 - qt;
    const size_t head = (size_t)bh * N * D;
    const int qtile0 = qt * BR, q0 = qtile0 + wave * QW;
    const int row = q0 + l32;

    const uint32_t sbase = lds_addr(smem);
    CP cp;
    cp.init(wave, lane, sbase, wave_uniform(wave));
    const i32x4 krs = make_rsrc(Kg + head, N * RB), vrs = make_rsrc(Vg + head, N * RB);
    const int nkt_total = (N + BC - 1) / BC;
    auto load_kv = [&](int t) {
        if (t < nkt_total) {
            cp.issue(krs, t, t & 1);
            cp.issue(vrs, t, 2 + (t & 1));
        }
    };
    auto ktile = [&](int t) -> const char* { return smem + (t & 1) * TB; };
    auto vtile = [&](int t) -> const char* { return smem + (2 + (t & 1)) * TB; };

    // The first tile copies go out before the fragment loads, so the
    // latencies overlap (the wait below covers both).
    load_kv(0);
    // Q^T and dO^T fragments (B operands): lane = query, d = 16*ch + 8*hi .. +7
    X8 qf[NCH], of[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const X8 z = __builtin_bit_cast(X8, u32x4{0, 0, 0, 0});
        qf[ch] = row < N ? load16<X8>(Qg + head + (size_t)row * D + 16 * ch + 8 * hi) : z;
        of[ch] = row < N ? load16<X8>(dOg + head + (size_t)row * D + 16 * ch + 8 * hi) : z;
    }
    const float lse2 = row < N ? LSEg[(size_t)bh * N + row] * kLog2e : 0.f;
    const float dd = row < N ? Dg[(size_t)bh * N + row] : 0.f;
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    TL tl;
    tl.init(lane);
    f32x16 acc[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) acc[db] = f32x16{};

    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const int nkt = (kend + BC - 1) / BC;
    wait_vm_all();
    __syncthreads();
    for (int t = 0; t < nkt; ++t) {
        load_kv(t + 1);
        const int k0 = t * BC;
        // A wave whose rows see none of the tile's keys skips it, except at
        // d = 256: there a branch around the accumulating asm MFMAs splits
        // the accumulators' register live ranges (copies every tile), so the
        // wave runs the tile fully masked instead (at most three tiles).
        if (D == 256 || !CAUSAL || k0 <= q0 + QW - 1) {
            // S^T = K Q^T and dP^T = V dO^T (lane = query, registers = keys)
            f32x16 s[NKB], dp[NKB];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb) s[kb] = dp[kb] = f32x16{};
#pragma unroll
            for (int c0 = 0; c0 < NCH; c0 += KB) {
                X8 kf[NKB][KB];
#pragma unroll
                for (int ch = 0; ch < KB; ++ch)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) kf[kb][ch] = tl.kfrag(ktile(t), c0 + ch, kb);
#pragma unroll
                for (int ch = 0; ch < KB; ++ch)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) s[kb] = mfma32(kf[kb][ch], qf[c0 + ch], s[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
#pragma unroll
            for (int c0 = 0; c0 < NCH; c0 += KB) {
                X8 vf[NKB][KB];
#pragma unroll
                for (int ch = 0; ch < KB; ++ch)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) vf[kb][ch] = tl.kfrag(vtile(t), c0 + ch, kb);
#pragma unroll
                for (int ch = 0; ch < KB; ++ch)
#pragma unroll
                    for (int kb = 0; kb < NKB; ++kb) dp[kb] = mfma32(vf[kb][ch], of[c0 + ch], dp[kb]);
                __builtin_amdgcn_sched_barrier(0);
            }
            // dS^T = P^T (dP^T - D), P^T = exp2(c S^T - lse2); masked keys give 0
            const bool masked = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
            X8 dsf[NPV];
#pragma unroll
            for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    typename Bw<T>::x2 w[4];
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        float x[2];
#pragma unroll
                        for (int e = 0; e < 2; ++e) {
                            const int r = 8 * h + 2 * j + e;
                            float p = exp2_hw(fmaf(s[kb][r], c, -lse2));
                            if (masked) {
                                const int key = k0 + key_of(kb, r, hi);
                                if (key >= N || (CAUSAL && key > row)) p = 0.f;
                            }
                            x[e] = p * (dp[kb][r] - dd);
                        }
                        w[j] = Bw<T>::pack(x[0], x[1]);
                    }
                    dsf[2 * kb + h] = X8{w[0][0], w[0][1], w[1][0], w[1][1],
                                         w[2][0], w[2][1], w[3][0], w[3][1]};
                }
            if constexpr (D == 256) {
#pragma unroll
                for (int tt = 0; tt < NPV; ++tt) asm volatile("s_nop 1" : "+v"(dsf[tt]));
            }
            __builtin_amdgcn_sched_barrier(0);
            // dQ^T += K^T dS^T
#pragma unroll
            for (int tt = 0; tt < NPV; ++tt)
#pragma unroll
                for (int d0 = 0; d0 < NDB; d0 += TB4) {
                    X8 kt[TB4];
#pragma unroll
                    for (int db = 0; db < TB4; ++db) kt[db] = tl.tfrag(ktile(t), tt, d0 + db);
#pragma unroll
                    for (int db = 0; db < TB4; ++db) grad_mfma<D>(acc[d0 + db], kt[db], dsf[tt]);
                }
        }
        wait_vm_all();
        __syncthreads();
    }
    grad_settle<D>(acc);
    if (row < N) store_rowT<T, D, OUT_F32>(dQg, head + (size_t)row * D, acc, scale, hi);
}

// ---------------------------------------------------------------------------
// dK, dV: one workgroup = 4 waves x 32 keys; query tiles of 32, two waves
// per SIMD. Per tile the copies bring the Q and dO rows and the tile's row
// constants Lr = -LSE/scale and D (1 KB each: rows beyond the tile are not
// used) into LDS. The score accumulator starts from Lr and the dP
// accumulator from -D (read from LDS into the accumulator registers), so
// P = exp2(c * S') and dS = P * dP' need no per-row registers.
template <typename T, int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(256, bwd_occupancy<D>())
bwd_dkv_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
               const T* __restrict__ dOg, const float* __restrict__ Cg, void* __restrict__ dKg,
               void* __restrict__ dVg, int N, long long rows, int num_ktiles, int num_blocks,
               float c, float scale)
{
    using X8 = typename Bw<T>::x8;
    using TL = Tile<T, D>;
    constexpr int NW = 4, KW = 32, BK = NW * KW, BQ = 32;
    constexpr int NCH = TL::NCH, NDB = TL::NDB, RB = TL::RB;
    constexpr int NPV = BQ / 16;
    // fragments per batch (d = 256: 2, the d x 32 accumulators leave few registers)
    constexpr int KB = D == 256 ? 2 : NCH / 2;
    constexpr int TB4 = D == 256 ? 2 : NDB;  // transposed fragments per batch
    using CP = Copier<D, BQ, NW>;
    constexpr int TB = CP::TB;
    constexpr int CB = 1024;                 // bytes per row-constant slot
    constexpr int VB = KW * RB;              // bytes of one wave's V rows
    // Q: slots 0,1; dO: 2,3; then [parity][Lr, D] constant slots; then each
    // wave's 32 V rows (B operand of dP, read per tile instead of held in
    // registers)
    __shared__ __attribute__((aligned(1024))) char smem[4 * TB + 4 * CB + NW * VB];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;
    if (num_blocks < 0) smem[tid] = 0;

    // Workgroup -> (head, key tile) (see grid_tile); causal: the first key
    // tiles, which see the most queries, go first.
    int bh, kt;
    grid_tile(num_blocks, num_ktiles, CAUSAL, bh, kt);
    const size_t head = (size_t)bh * N * D;
    const int kblk0 = kt * BK, k0 = kblk0 + wave * KW;
    // lane -> key: permuted within the wave's 32 keys like the A-operand rows,
    // so the K fragments in registers and the V fragments read from LDS (with
    // the row-permuted fragment read) agree
    const int key = k0 + krow_perm(l32);

    const uint32_t sbase = lds_addr(smem);
    const int wave_u = wave_uniform(wave);
    CP cp;
    cp.init(wave, lane, sbase, wave_u);
    const i32x4 qrs = make_rsrc(Qg + head, N * RB), ors = make_rsrc(dOg + head, N * RB);
    const i32x4 lrs = make_rsrc(Cg + rows + (size_t)bh * N, N * 4);     // Lr of this head
    const i32x4 drs = make_rsrc(Cg + (size_t)bh * N, N * 4);            // D of this head
    const uint32_t cslot = sbase + 4 * TB;
    const int nqt = (N + BQ - 1) / BQ;
    auto load_qo = [&](int i) {
        if (i < nqt) {
            cp.issue(qrs, i, i & 1);
            cp.issue(ors, i, 2 + (i & 1));
            if (wave_u == 0) {
                const uint32_t dst = cslot + (i & 1) * 2 * CB;
                buffer_load_lds16(lrs, dst, 16 * lane, i * BQ * 4);
                buffer_load_lds16(drs, dst + CB, 16 * lane, i * BQ * 4);
            }
        }
    };
    auto qtile = [&](int i) -> const char* { return smem + (i & 1) * TB; };
    auto otile = [&](int i) -> const char* { return smem + (2 + (i & 1)) * TB; };
    // accumulator start: register r holds tile row 16*(r/8) + 8*hi + r%8
    auto acc_init = [&](int i, int which, float sign) -> f32x16 {
        const char* base = smem + 4 * TB + (i & 1) * 2 * CB + which * CB;
        f32x16 a;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x4 v = load16<f32x4>(base + 4 * (16 * (g / 2) + 8 * hi + 4 * (g % 2)));
#pragma unroll
            for (int e = 0; e < 4; ++e) a[4 * g + e] = sign * v[e];
        }
        return a;
    };

    // This wave's V rows k0 .. k0+31 into its LDS slot (rows >= N read 0)
    // and the first Q/dO tile go out before the K fragment loads, so the
    // latencies overlap (the wait below covers all of them).
    const char* vw = smem + 4 * TB + 4 * CB + wave * VB;
    {
        Copier<D, KW, 1> vcp;
        vcp.init(0, lane, sbase + 4 * TB + 4 * CB + wave_u * VB, 0);
        const i32x4 vrs = make_rsrc(Vg + head + (size_t)k0 * D, max(N - k0, 0) * RB);
        vcp.issue(vrs, 0, 0);
    }
    const int i0 = CAUSAL ? kblk0 / BQ : 0;
    load_qo(i0);
    // K^T fragments (B operand of S): lane = key, d = 16*ch + 8*hi .. +7
    X8 kf[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch) {
        const X8 z = __builtin_bit_cast(X8, u32x4{0, 0, 0, 0});
        kf[ch] = key < N ? load16<X8>(Kg + head + (size_t)key * D + 16 * ch + 8 * hi) : z;
    }
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    TL tl;
    tl.init(lane);
    f32x16 dk[NDB], dv[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) dk[db] = dv[db] = f32x16{};

    wait_vm_all();
    __syncthreads();
    for (int i = i0; i < nqt; ++i) {
        load_qo(i + 1);
        const int q0 = i * BQ;
        // this wave has a visible pair (d = 256: always run, see bwd_dq_kernel)
        if (D == 256 || !CAUSAL || q0 + BQ - 1 >= k0) {
            // S' = Q K^T + Lr and dP' = dO V^T - D (lane = key, registers =
            // queries); operands in half batches to bound the live registers
            f32x16 s = acc_init(i, 0, 1.0f);
#pragma unroll
            for (int c0 = 0; c0 < NCH; c0 += KB) {
                X8 qa[KB];
#pragma unroll
                for (int ch = 0; ch < KB; ++ch) qa[ch] = tl.kfrag(qtile(i), c0 + ch, 0);
#pragma unroll
                for (int ch = 0; ch < KB; ++ch) s = mfma32(qa[ch], kf[c0 + ch], s);
                __builtin_amdgcn_sched_barrier(0);
            }
            f32x16 dp = acc_init(i, 1, -1.0f);
#pragma unroll
            for (int c0 = 0; c0 < NCH; c0 += KB) {
                X8 oa[KB];
#pragma unroll
                for (int ch = 0; ch < KB; ++ch) oa[ch] = tl.kfrag(otile(i), c0 + ch, 0);
                X8 vb[KB];
#pragma unroll
                for (int ch = 0; ch < KB; ++ch) vb[ch] = tl.kfrag(vw, c0 + ch, 0);
#pragma unroll
                for (int ch = 0; ch < KB; ++ch) dp = mfma32(oa[ch], vb[ch], dp);
                __builtin_amdgcn_sched_barrier(0);
            }
            const bool masked = (q0 + BQ > N) || (CAUSAL && q0 < k0 + KW - 1);
            X8 pf[NPV], dsf[NPV];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                typename Bw<T>::x2 wp[4], wd[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    float p2[2], d2[2];
#pragma unroll
                    for (int e = 0; e < 2; ++e) {
                        const int r = 8 * h + 2 * j + e;
                        float p = exp2_hw(s[r] * c);
                        if (masked) {
                            const int q = q0 + key_of(0, r, hi);
                            if (q >= N || (CAUSAL && key > q)) p = 0.f;
                        }
                        p2[e] = p;
                        d2[e] = p * dp[r];
                    }
                    wp[j] = Bw<T>::pack(p2[0], p2[1]);
                    wd[j] = Bw<T>::pack(d2[0], d2[1]);
                }
                pf[h] = X8{wp[0][0], wp[0][1], wp[1][0], wp[1][1], wp[2][0], wp[2][1], wp[3][0], wp[3][1]};
                dsf[h] = X8{wd[0][0], wd[0][1], wd[1][0], wd[1][1], wd[2][0], wd[2][1], wd[3][0], wd[3][1]};
            }
            if constexpr (D == 256) asm volatile("s_nop 1" : "+v"(pf[0]), "+v"(pf[1]), "+v"(dsf[0]), "+v"(dsf[1]));
            __builtin_amdgcn_sched_barrier(0);
            // dV^T += dO^T P,  dK^T += Q^T dS
#pragma unroll
            for (int tt = 0; tt < NPV; ++tt)
#pragma unroll
                for (int d0 = 0; d0 < NDB; d0 += TB4) {
                    {
                        X8 ot[TB4];
#pragma unroll
                        for (int db = 0; db < TB4; ++db) ot[db] = tl.tfrag(otile(i), tt, d0 + db);
#pragma unroll
                        for (int db = 0; db < TB4; ++db) grad_mfma<D>(dv[d0 + db], ot[db], pf[tt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                    {
                        X8 qt[TB4];
#pragma unroll
                        for (int db = 0; db < TB4; ++db) qt[db] = tl.tfrag(qtile(i), tt, d0 + db);
#pragma unroll
                        for (int db = 0; db < TB4; ++db) grad_mfma<D>(dk[d0 + db], qt[db], dsf[tt]);
                    }
                    __builtin_amdgcn_sched_barrier(0);
                }
        }
        wait_vm_all();
        __syncthreads();
    }
    grad_settle<D>(dk);
    grad_settle<D>(dv);
    if (key < N) {
        store_rowT<T, D, OUT_F32>(dKg, head + (size_t)key * D, dk, scale, hi);
        store_rowT<T, D, OUT_F32>(dVg, head + (size_t)key * D, dv, 1.0f, hi);
    }
}

template <typename T, int D, bool CAUSAL, bool OUT_F32>
hipError_t launch_t(const BwdArgs& a, hipStream_t s) {
    const long long rows = (long long)a.B * a.H * a.N;
    const long long nthr = rows * (D / 8);
    hipLaunchKernelGGL((bwd_delta_kernel<T, D>), dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0, s,
                       static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.lse, a.delta, rows,
                       1.0f / a.scale);
    const float c = a.scale * kLog2e;
    {
        const int nqt = (a.N + 127) / 128;
        const long long nblk = (long long)nqt * a.B * a.H;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_dq_kernel<T, D, CAUSAL, OUT_F32>), dim3((unsigned)nblk), dim3(256), 0, s,
                           static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.lse, a.delta,
                           a.dq, a.N, nqt, (int)nblk, c, a.scale);
    }
    {
        const int nkt = (a.N + 127) / 128;
        const long long nblk = (long long)nkt * a.B * a.H;
        if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
        hipLaunchKernelGGL((bwd_dkv_kernel<T, D, CAUSAL, OUT_F32>), dim3((unsigned)nblk), dim3(256), 0, s,
                           static_cast<const T*>(a.q), static_cast<const T*>(a.k),
                           static_cast<const T*>(a.v), static_cast<const T*>(a.dout), a.delta,
                           a.dk, a.dv, a.N, rows, nkt, (int)nblk, c, a.scale);
    }
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const BwdArgs& a, hipStream_t s) {
    if (a.causal)
        return a.out_f32 ? launch_t<T, D, true, true>(a, s) : launch_t<T, D, true, false>(a, s);
    return a.out_f32 ? launch_t<T, D, false, true>(a, s) : launch_t<T, D, false, false>(a, s);
}

template <typename T>
hipError_t launch_ty(const BwdArgs& a, hipStream_t s) {
    switch (a.d) {
        case 64: return launch_d<T, 64>(a, s);
        case 128: return launch_d<T, 128>(a, s);
        case 256: return launch_d<T, 256>(a, s);
    }
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_bwd16(const BwdArgs& a, bool bf16, hipStream_t s) {
    return bf16 ? launch_ty<__bf16>(a, s) : launch_ty<_Float16>(a, s);
}

}  // namespace fa
