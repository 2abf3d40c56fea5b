// fa_decode16.hip - decode-shaped attention forward (bf16 / fp16, gfx950):
// a few new query rows per head against a long, per-sequence key/value
// history, split over the keys with the partial results merged by their
// log-sum-exp.
//
// Method: the function is the exact attention of "FlashAttention - one, two,
// three!" (Medium), section "Standard Attention"; the split over keys with a
// per-part maximum and sum, recombined afterwards, is the block-wise softmax
// of section "FlashAttention v1." (a part's maximum and denominator are
// rescaled when parts are merged) applied across workgroups instead of across
// loop iterations. "FlashAttention-3: Fast & Accurate Attention with
// Asynchrony & Low-Precision" (Embodied AI 101 transcript), section
// "Performance Results", names autoregressive sampling as a use.
//
// Shape of the work: per (batch, key/value head) the query rows are the
// Nq rows of each of the H/Hkv query heads that share it (at most 32 per
// wave; more rows take more row groups). There is one score column per
// query row, so a 32-key block of S^T = K Q^T is a single 32x32 MFMA tile
// chain and the kernel moves 2*d*2 bytes of K and V per key: it is bound by
// HBM bandwidth, not by the matrix cores. Each wave streams its own range of
// keys (one split) through NST private LDS stages with direct buffer->LDS
// copies, so no workgroup barrier is needed anywhere; only vmcnt waits.
//
// Output: with one split the wave writes O and LSE; otherwise it writes a
// partial (O_s normalised by its own sum, LSE_s) and decode_merge_kernel
// combines them: LSE = log sum_s exp(LSE_s), O = sum_s exp(LSE_s - LSE) O_s.
#include "fa.h"
#include "fa_device.h"
#include "fa_internal.h"

#include <math.h>

#include <mutex>

namespace fa {
namespace {

// Stages per wave: all in flight at the top of a block except the one being
// read. The vmcnt field holds 63 outstanding loads (NST-1 blocks of
// 2*RB/32 loads each). Measured at d = 128: 2, 3 and 4 stages (5, 3 and 2
// waves per CU by LDS) stream within noise of each other and above a plain
// device copy.
#ifndef FA_DEC_NST64
#define FA_DEC_NST64 4
#endif
#ifndef FA_DEC_NST128
#define FA_DEC_NST128 2
#endif
#ifndef FA_DEC_NST256
#define FA_DEC_NST256 2
#endif
template <int D> struct DecCfg;
template <> struct DecCfg<64> { static constexpr int NST = FA_DEC_NST64; };
template <> struct DecCfg<128> { static constexpr int NST = FA_DEC_NST128; };
template <> struct DecCfg<256> { static constexpr int NST = FA_DEC_NST256; };

template <int N>
__device__ __forceinline__ void vm_wait() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Every LDS read of the wave has returned (before a copy overwrites a stage).
__device__ __forceinline__ void lds_reads_done() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

enum { kOutT = 0, kOutF32 = 1, kOutPartial = 2 };

template <typename T, int D, bool CAUSAL, int OUTK>
__global__ void __launch_bounds__(64)
decode16_kernel(const T* __restrict__ Qg, const T* __restrict__ Kg, const T* __restrict__ Vg,
                void* __restrict__ Og, float* __restrict__ LSEg, const int* __restrict__ seqlens,
                int H, int Hkv, int Nq, int Nk, int M, int RG, int S, long long R, float c)
{
    using X8 = typename Elt<T>::x8;
    using X2 = typename Elt<T>::x2;
    constexpr int RB = 2 * D;              // bytes per K / V row
    constexpr int NCH = D / 16;            // k-steps of S^T = K Q^T
    constexpr int NDB = D / 32;            // 32-row blocks of O^T
    constexpr int SB = 32 * RB;            // bytes per 32-row K (or V) block
    constexpr int NL = SB / 1024;          // 1 KB copies per block and tensor
    constexpr int NST = DecCfg<D>::NST;
    constexpr int LPB = 2 * NL;            // copies per block (K and V)
    static_assert(LPB * (NST - 1) <= 63, "outstanding copies exceed vmcnt");
    constexpr int NKA = (D == 64) ? 4 : 8; // distinct K lane offsets (swizzle period)
    constexpr int NVA = (D == 64) ? 2 : 4; // distinct V^T lane offsets

    __shared__ __attribute__((aligned(1024))) char smem[NST * 2 * SB];

    const int lane = threadIdx.x;
    const int l32 = lane & 31, hi = lane >> 5;
    if (Nk < 0) smem[lane] = 0;            // see fa_fwd16_kernel: keeps LDS reads defined

    const int s = blockIdx.x % S;
    const int unit = blockIdx.x / S;
    const int rg = unit % RG;
    const int bk = unit / RG;              // b * Hkv + kv head
    const int b = bk / Hkv, hkv = bk - b * Hkv;
    const int g = H / Hkv;
    int L = Nk;
    if (seqlens) L = min(max(seqlens[b], 0), Nk);
    L = wave_uniform(L);

    // This wave's keys: split s of [0, L) in 32-key multiples.
    const int chunk = ((L + S - 1) / S + 31) / 32 * 32;
    const int k0 = min(L, s * chunk);
    const int k1 = min(L, k0 + chunk);
    const int nblk = (k1 - k0 + 31) / 32;
    // A part of at most 64 keys feeds P to the PV MFMA as the rounded P~
    // plus its rounding residue (two MFMAs per fragment): on a row that sees
    // only a few keys, rounding P to bf16 (2^-8 relative) could otherwise
    // move O by up to ~w(1-w) 2^-8 |v_a - v_b| (above 4e-3 for two keys of
    // comparable weight whose values differ by ~8); over many keys it
    // averages out.
    const bool split_p = k1 - k0 <= 64;

    // Query row of this lane's score column: row r of the group is query
    // i = r % Nq of head hkv*g + r / Nq.
    const int r = 32 * rg + l32;
    const bool rv = r < M;
    const int h = hkv * g + (rv ? r / Nq : 0);
    const int qi = rv ? r % Nq : 0;
    const long long qrow = ((long long)b * H + h) * Nq + qi;
    const int klim = CAUSAL ? L - Nq + qi : L - 1;       // last key this row sees
    const int kfree = CAUSAL ? L - Nq + 1 : L;           // keys below: seen by every row

    // Q^T fragments (B operand): lane holds d = 16 ch + 8 hi .. +7 of its row;
    // rows >= M are zeros. Waited for (a wait the compiler sees) before the
    // first copy is issued.
    X8 qf[NCH];
#pragma unroll
    for (int ch = 0; ch < NCH; ++ch)
        qf[ch] = rv ? load16<X8>(Qg + qrow * D + 16 * ch + 8 * hi)
                    : __builtin_bit_cast(X8, u32x4{0, 0, 0, 0});
    __builtin_amdgcn_s_waitcnt(kVmcnt0);

    // Copies: buffer loads over the sequence's L rows (rows >= L read as
    // zeros) straight into LDS; load j fills bytes [1024 j, +1024) of a block,
    // lane i the 16 bytes at +16 i = physical chunk cp of row p / RB, which
    // holds logical chunk cp ^ lds_swz16(row).
    const size_t head = (size_t)bk * Nk * D;
    const i32x4 krs = make_rsrc(Kg + head, L * RB);
    const i32x4 vrs = make_rsrc(Vg + head, L * RB);
    uint32_t voff[NL];
#pragma unroll
    for (int j = 0; j < NL; ++j) {
        const int p = j * 1024 + 16 * lane;
        const int row = p / RB;
        voff[j] = row * RB + ((p % RB / 16) ^ lds_swz16<D>(row)) * 16;
    }
    const uint32_t sbase = lds_addr(smem);
    auto issue = [&](int j) {
        const uint32_t dst = sbase + (j % NST) * 2 * SB;
        const uint32_t soff = (uint32_t)(k0 + 32 * j) * RB;
#pragma unroll
        for (int i = 0; i < NL; ++i) buffer_load_lds16(krs, dst + i * 1024, voff[i], soff);
#pragma unroll
        for (int i = 0; i < NL; ++i) buffer_load_lds16(vrs, dst + SB + i * 1024, voff[i], soff);
    };

    // Lane offsets into a swizzled block: K fragment ch (row perm(l32), logical
    // chunk 2 ch + hi) and V^T fragment (t, db) as in the forward kernel.
    int ka[NKA];
    int va[NVA];
    int vstep;
    {
        const int kr = krow_perm(l32);
#pragma unroll
        for (int ch = 0; ch < NKA; ++ch) ka[ch] = kr * RB + (((2 * ch + hi) ^ lds_swz16<D>(kr)) * 16);
        const int vr = 8 * hi + (lane & 15) / 4;
#pragma unroll
        for (int db = 0; db < NVA; ++db) {
            const int chunk16 = 4 * db + 2 * (l32 / 16) + ((lane & 3) >> 1);
            va[db] = vr * RB + ((chunk16 ^ lds_swz16<D>(vr)) * 16) + 8 * (lane & 1);
        }
        vstep = 4 * RB + (((lane & 3) >> 1) ? -16 : 16);
    }

    f32x16 o[NDB];
#pragma unroll
    for (int db = 0; db < NDB; ++db) o[db] = f32x16{};
    float m = -INFINITY;   // running maximum, log2 units
    float l = 0.f;         // sum of the rounded P fed to the MFMA
    float lx = 0.f;        // sum of the fp32 p (for the log-sum-exp)

#pragma unroll
    for (int j = 0; j < NST; ++j)
        if (j < nblk) issue(j);

    for (int j = 0; j < nblk; ++j) {
        if (j + NST - 1 < nblk) vm_wait<LPB * (NST - 1)>();
        else vm_wait<0>();
        const char* kl = smem + (j % NST) * 2 * SB;
        const char* vl = kl + SB;
        const int key0 = k0 + 32 * j;

        f32x16 sc = f32x16{};
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch)
            sc = mfma32(load16<X8>(kl + ka[ch % NKA] + NKA * 32 * (ch / NKA)), qf[ch], sc);
        if (key0 + 32 > kfree) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int key = key0 + key_of(0, i, hi);
                if (key >= L || key > klim) sc[i] = -INFINITY;
            }
        }
        float tm = sc[0];
#pragma unroll
        for (int i = 1; i < 16; ++i) tm = fmaxf(tm, sc[i]);
        tm = pair_max(tm) * c;
        const float mnew = fmaxf(m, tm);
        const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(m - mnew);
        const float mref = (mnew == -INFINITY) ? 0.f : mnew;
        m = mnew;
        l *= alpha;
        lx *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[db] *= alpha;

        X8 pf[2];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            X2 pp[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const float p0 = exp2_hw(fmaf(sc[8 * t + 2 * u], c, -mref));
                const float p1 = exp2_hw(fmaf(sc[8 * t + 2 * u + 1], c, -mref));
                pp[u] = pack2<T>(p0, p1);
                lx += p0 + p1;
                l = sum2(pp[u], l);
            }
            pf[t] = X8{pp[0][0], pp[0][1], pp[1][0], pp[1][1], pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
        }
        X8 pr[2];                              // residue p - P~ (split parts only)
        if (split_p) {
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                X2 pp[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const float p0 = exp2_hw(fmaf(sc[8 * t + 2 * u], c, -mref));
                    const float p1 = exp2_hw(fmaf(sc[8 * t + 2 * u + 1], c, -mref));
                    pp[u] = pack2<T>(p0 - (float)pf[t][2 * u], p1 - (float)pf[t][2 * u + 1]);
                    l = sum2(pp[u], l);
                }
                pr[t] = X8{pp[0][0], pp[0][1], pp[1][0], pp[1][1], pp[2][0], pp[2][1], pp[3][0], pp[3][1]};
            }
        }
        // O^T += V^T P^T: k-step t covers keys 16 t .. 16 t + 15 of the block.
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
                const char* vp = vl + va[db % NVA] + NVA * 64 * (db / NVA) + 16 * t * RB;
                const u32x2 lo = lds_read_tr16(vp);
                const u32x2 hi4 = lds_read_tr16(vp + vstep);
                const X8 vf = __builtin_bit_cast(X8, u32x4{lo[0], lo[1], hi4[0], hi4[1]});
                o[db] = mfma32(vf, pf[t], o[db]);
                if (split_p) o[db] = mfma32(vf, pr[t], o[db]);
            }
        if (j + NST < nblk) {
            lds_reads_done();
            issue(j + NST);
        }
    }

    // ---- epilogue ----
    const float lsum = pair_sum(l);
    const float lxs = pair_sum(lx);
    const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
    const float lse = lxs > 0.f ? (m + __builtin_amdgcn_logf(lxs)) * kLn2 : -INFINITY;
    if (!rv) return;
    const long long orow = OUTK == kOutPartial ? (long long)s * R + qrow : qrow;
    if (hi == 0) LSEg[orow] = lse;
#pragma unroll
    for (int db = 0; db < NDB; ++db)
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int dcol = 32 * db + 8 * u + 4 * hi;
            const size_t off = (size_t)orow * D + dcol;
            const float v0 = o[db][4 * u] * inv, v1 = o[db][4 * u + 1] * inv;
            const float v2 = o[db][4 * u + 2] * inv, v3 = o[db][4 * u + 3] * inv;
            if (OUTK != kOutT) {
                *reinterpret_cast<f32x4*>(static_cast<float*>(Og) + off) = f32x4{v0, v1, v2, v3};
            } else {
                const X2 a = pack2<T>(v0, v1), bb = pack2<T>(v2, v3);
                *reinterpret_cast<u32x2*>(static_cast<T*>(Og) + off) =
                    u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, bb)};
            }
        }
}

// Merge of S partial results per query row: D/4 lanes per row, 4 columns
// each. A row whose parts all saw no key gets O = 0 and LSE = -inf.
template <typename T, int D, bool OUT_F32>
__global__ void __launch_bounds__(256)
decode_merge_kernel(const float* __restrict__ Op, const float* __restrict__ LSEp, void* __restrict__ Og,
                    float* __restrict__ LSEg, long long R, int S)
{
    constexpr int TPR = D / 4;
    const long long row = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
    const int col = 4 * (threadIdx.x % TPR);
    if (row >= R) return;
    float mx = -INFINITY;
    for (int s = 0; s < S; ++s) mx = fmaxf(mx, LSEp[(long long)s * R + row]);
    f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mx != -INFINITY) {
        for (int s = 0; s < S; ++s) {
            const float w = expf(LSEp[(long long)s * R + row] - mx);
            const f32x4 x = *reinterpret_cast<const f32x4*>(Op + ((long long)s * R + row) * D + col);
            acc += w * x;
            wsum += w;
        }
        acc *= 1.0f / wsum;
    }
    if (col == 0) LSEg[row] = mx == -INFINITY ? -INFINITY : mx + logf(wsum);
    const size_t off = (size_t)row * D + col;
    if (OUT_F32) {
        *reinterpret_cast<f32x4*>(static_cast<float*>(Og) + off) = acc;
    } else {
        using X2 = typename Elt<T>::x2;
        const X2 a = pack2<T>(acc[0], acc[1]), bb = pack2<T>(acc[2], acc[3]);
        *reinterpret_cast<u32x2*>(static_cast<T*>(Og) + off) =
            u32x2{__builtin_bit_cast(uint32_t, a), __builtin_bit_cast(uint32_t, bb)};
    }
}

template <typename T, int D, bool CAUSAL>
hipError_t launch_t(const DecodeArgs& a, hipStream_t st) {
    const int g = a.H / a.Hkv;
    const int M = g * a.Nq;
    const int RG = (M + 31) / 32;
    const long long R = (long long)a.B * a.H * a.Nq;
    const long long grid = (long long)a.B * a.Hkv * RG * a.splits;
    const float c = a.scale * kLog2e;
    const T* q = static_cast<const T*>(a.q);
    const T* k = static_cast<const T*>(a.k);
    const T* v = static_cast<const T*>(a.v);
    if (a.splits == 1) {
        if (a.out_f32)
            hipLaunchKernelGGL((decode16_kernel<T, D, CAUSAL, kOutF32>), dim3((unsigned)grid), dim3(64), 0, st,
                               q, k, v, a.o, a.lse, a.seqlens, a.H, a.Hkv, a.Nq, a.Nk, M, RG, 1, R, c);
        else
            hipLaunchKernelGGL((decode16_kernel<T, D, CAUSAL, kOutT>), dim3((unsigned)grid), dim3(64), 0, st,
                               q, k, v, a.o, a.lse, a.seqlens, a.H, a.Hkv, a.Nq, a.Nk, M, RG, 1, R, c);
        return hipGetLastError();
    }
    float* op = static_cast<float*>(a.workspace);
    float* lp = reinterpret_cast<float*>(static_cast<char*>(a.workspace) +
                                         decode_partial_o_bytes(R, a.splits, D));
    hipLaunchKernelGGL((decode16_kernel<T, D, CAUSAL, kOutPartial>), dim3((unsigned)grid), dim3(64), 0, st,
                       q, k, v, op, lp, a.seqlens, a.H, a.Hkv, a.Nq, a.Nk, M, RG, a.splits, R, c);
    const unsigned mg = (unsigned)((R + (256 / (D / 4)) - 1) / (256 / (D / 4)));
    if (a.out_f32)
        hipLaunchKernelGGL((decode_merge_kernel<T, D, true>), dim3(mg), dim3(256), 0, st, op, lp, a.o, a.lse,
                           R, a.splits);
    else
        hipLaunchKernelGGL((decode_merge_kernel<T, D, false>), dim3(mg), dim3(256), 0, st, op, lp, a.o, a.lse,
                           R, a.splits);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_d(const DecodeArgs& a, hipStream_t st) {
    return a.causal ? launch_t<T, D, true>(a, st) : launch_t<T, D, false>(a, st);
}

template <typename T>
hipError_t launch_ty(const DecodeArgs& a, hipStream_t st) {
    switch (a.d) {
        case 64: return launch_d<T, 64>(a, st);
        case 128: return launch_d<T, 128>(a, st);
        case 256: return launch_d<T, 256>(a, st);
    }
    return hipErrorInvalidValue;
}

}  // namespace

size_t decode_partial_o_bytes(long long rows, int splits, int d) {
    return round_up((size_t)rows * splits * d * sizeof(float), 256);
}

size_t decode_workspace_bytes(long long rows, int splits, int d) {
    if (splits <= 1) return 0;
    return decode_partial_o_bytes(rows, splits, d) + round_up((size_t)rows * splits * sizeof(float), 256);
}

int decode_default_splits(int B, int H, int Hkv, int Nq, int Nk, int d) {
    // About 1024 waves (four per CU of 256), each split at least 8 blocks
    // of 32 keys, at most 64 splits. Measured on two workloads of 128
    // (batch, key/value head) units: 8 splits beat 4, 6, 12 and 16.
    const int g = H / Hkv;
    const long long units = (long long)B * Hkv * ((g * Nq + 31) / 32);
    const long long waves = 1024;
    long long s = (waves + units - 1) / units;
    const long long by_len = (long long)((Nk + 31) / 32) / 8;
    s = s < by_len ? s : by_len;
    s = s < 64 ? s : 64;
    return s < 1 ? 1 : (int)s;
}

hipError_t launch_decode16(const DecodeArgs& a, bool bf16, hipStream_t st) {
    return bf16 ? launch_ty<__bf16>(a, st) : launch_ty<_Float16>(a, st);
}

// Split partials of fa_fwd_decode_noalloc, for callers that cannot allocate:
// a fixed array in device memory, one per GPU the library runs on, held
// until the process ends. Host code never passes the array's name to a
// kernel (on the host it is only a stand-in for the symbol): its device
// address is looked up once per device and kept.
static __device__ __align__(256) unsigned char scratch[FA_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_addr[kMaxDevices] = {};
}  // namespace

hipError_t decode_scratch(hipStream_t s, void** ptr) {
    int dev = 0;
    hipError_t e = s ? hipStreamGetDevice(s, &dev) : hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_addr[dev]) {
        // with that device current
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_addr[dev] = p;
    }
    *ptr = g_scratch_addr[dev];
    return hipSuccess;
}

}  // namespace fa
