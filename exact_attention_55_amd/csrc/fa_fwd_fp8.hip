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
// transposed output O^T += V^T P^T, lazy rescale, double-buffered LDS), with
// 32x32x64 e4m3 MFMA. Scale handling, per query block i and key tile j:
//  * logits: s = acc * sq_i * sk_j * softmax_scale; in the base-2 domain the
//    product c_j = sq_i * sk_j * softmax_scale * log2(e) is one scalar per
//    tile, folded into the fma that feeds exp2;
//  * P is quantised to e4m3 for the PV MFMA as P' = p * 16 * w_j with
//    w_j = sv_j / sv_max (sv_max = largest V block scale of the head): the
//    factor is folded into the exponent, p' = exp2(s*c - m + log2(16 w_j)), so
//    the V block scale costs no extra VALU work. With the lazy-rescale bound
//    p <= 2^4 this keeps P' <= 256 < 448, and p >= 2^-10 stays normal;
//  * the row sum l accumulates the unquantised p (rowsum(P') / (16 w_j));
//  * epilogue: O = O_acc * sv_max / (16 l).
#include "fa_device.h"
#include "fa_internal.h"

namespace fa {

constexpr float kTau8 = 4.0f;       // lazy-rescale threshold (log2 units)
constexpr float kPScale = 16.0f;    // P multiplier before e4m3 rounding (= 2^(8 - kTau8))

template <int D> struct Cfg8;
template <> struct Cfg8<64>  { static constexpr int NW = 4, QB = 2, BC = 64; };
template <> struct Cfg8<128> { static constexpr int NW = 4, QB = 2, BC = 64; };
template <> struct Cfg8<256> { static constexpr int NW = 4, QB = 1, BC = 64; };

__device__ __forceinline__ uint32_t cvt4_e4m3(float a, float b, float c, float d) {
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, w, true);
    return (uint32_t)w;
}

template <int D, bool CAUSAL, bool OUT_F32>
__global__ void __launch_bounds__(Cfg8<D>::NW * 64, 1)
fa_fwd_fp8_kernel(const uint8_t* __restrict__ Qg, const uint8_t* __restrict__ Kg,
                  const uint8_t* __restrict__ Vg, void* __restrict__ Og, float* __restrict__ LSEg,
                  int N, int num_qtiles, int num_blocks, int nsb, size_t scales_off, float c)
{
    constexpr int NW = Cfg8<D>::NW, QB = Cfg8<D>::QB, BC = Cfg8<D>::BC;
    constexpr int QW = 32 * QB;
    constexpr int BR = NW * QW;
    constexpr int KS = D + 16;              // LDS row stride (bytes)
    constexpr int VS = D + 16;
    constexpr int KT = BC * KS, VT = BC * VS;
    constexpr int NCH = D / 64;             // k-steps of S^T = K Q^T
    constexpr int NDB = D / 32;             // 32-row blocks of O^T
    constexpr int NKB = BC / 32;            // 32-key blocks of S^T
    constexpr int NPV = BC / 64;            // k-steps of O^T += V^T P^T
    constexpr int NT = NW * 64;
    constexpr int CPR = D / 16;             // 16-byte chunks per row
    constexpr int CPT = BC * CPR / NT;
    static_assert(BC * CPR % NT == 0, "tile must split evenly over threads");
    static_assert(NKB == 2 * NPV, "one PV MFMA per two score blocks");
    static_assert(kQuantBlockRows % BC == 0 && kQuantBlockRows % QW == 0, "scale blocks");

    __shared__ __attribute__((aligned(16))) uint8_t smem[2 * (KT + VT)];

    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int l32 = lane & 31, hi = lane >> 5;

    int bid = blockIdx.x;
    if ((num_blocks & 7) == 0) bid = (bid & 7) * (num_blocks >> 3) + (bid >> 3);
    const int bh = bid / num_qtiles;
    int qt = bid - bh * num_qtiles;
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

    // largest V block scale of the head
    float svmax = 0.f;
    for (int i = lane; i < nsb; i += 64) svmax = fmaxf(svmax, Vs[i]);
#pragma unroll
    for (int m = 32; m >= 1; m /= 2) svmax = fmaxf(svmax, __shfl_xor(svmax, m, 64));

    // Q^T fragments: query q0+32*qb+l32, bytes [64*ch + 32*hi, +32)
    i32x8 qf[QB][NCH];
    float cq[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const int row = q0 + 32 * qb + l32;
        const int rowc = min(q0 + 32 * qb, N - 1);          // wave-uniform scale block
        cq[qb] = Qs[rowc / kQuantBlockRows] * c;
#pragma unroll
        for (int ch = 0; ch < NCH; ++ch) {
            u32x4 a = u32x4{0, 0, 0, 0}, b = u32x4{0, 0, 0, 0};
            if (row < N) {
                const uint8_t* p = Q + (size_t)row * D + 64 * ch + 32 * hi;
                a = *reinterpret_cast<const u32x4*>(p);
                b = *reinterpret_cast<const u32x4*>(p + 16);
            }
            qf[qb][ch] = i32x8{(int)a[0], (int)a[1], (int)a[2], (int)a[3],
                               (int)b[0], (int)b[1], (int)b[2], (int)b[3]};
        }
    }

    const int kend = CAUSAL ? min(N, qtile0 + BR) : N;
    const int nkt = (kend + BC - 1) / BC;

    f32x16 o[QB][NDB];
    float m_ref[QB], lsum[QB];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        m_ref[qb] = -INFINITY;
        lsum[qb] = 0.f;
#pragma unroll
        for (int db = 0; db < NDB; ++db) o[qb][db] = f32x16{};
    }

    u32x4 kst[CPT], vst[CPT];
    auto gload = [&](int kt) {
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / CPR, ch = idx % CPR;
            const int key = kt * BC + r;
            if (key < N) {
                kst[i] = *reinterpret_cast<const u32x4*>(K + (size_t)key * D + ch * 16);
                vst[i] = *reinterpret_cast<const u32x4*>(V + (size_t)key * D + ch * 16);
            } else {
                kst[i] = u32x4{0, 0, 0, 0};
                vst[i] = u32x4{0, 0, 0, 0};
            }
        }
    };
    auto swrite = [&](int buf) {
        uint8_t* kl = smem + buf * (KT + VT);
        uint8_t* vl = kl + KT;
#pragma unroll
        for (int i = 0; i < CPT; ++i) {
            const int idx = tid + i * NT;
            const int r = idx / CPR, ch = idx % CPR;
            *reinterpret_cast<u32x4*>(kl + r * KS + ch * 16) = kst[i];
            *reinterpret_cast<u32x4*>(vl + r * VS + ch * 16) = vst[i];
        }
    };

    const int k_off = krow_perm(l32) * KS + 32 * hi;
    const int v_off = (8 * hi + (lane & 15) / 2) * VS + 16 * (l32 / 16) + 8 * (lane & 1);

    gload(0);
    swrite(0);
    __syncthreads();

    for (int kt = 0; kt < nkt; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < nkt) gload(kt + 1);
        const uint8_t* kl = smem + buf * (KT + VT);
        const uint8_t* vl = kl + KT;
        const int k0 = kt * BC;
        const bool active = !CAUSAL || (k0 <= q0 + QW - 1);
        if (active) {
            const int sblk = k0 / kQuantBlockRows;
            const float sk = Ks[sblk];
            const float wv = Vs[sblk] / svmax;                  // (0, 1]
            const float bj = __builtin_amdgcn_logf(kPScale * wv);  // log2(16 w_j)
            const float lscale = 1.0f / (kPScale * wv);
            // ---- S^T = K Q^T ----
            f32x16 s[QB][NKB];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb)
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) s[qb][kb] = f32x16{};
#pragma unroll
            for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb) {
                    const uint8_t* p = kl + k_off + 32 * kb * KS + 64 * ch;
                    const u32x4 a0 = *reinterpret_cast<const u32x4*>(p);
                    const u32x4 a1 = *reinterpret_cast<const u32x4*>(p + 16);
                    const i32x8 a = i32x8{(int)a0[0], (int)a0[1], (int)a0[2], (int)a0[3],
                                          (int)a1[0], (int)a1[1], (int)a1[2], (int)a1[3]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) s[qb][kb] = mfma32_fp8(a, qf[qb][ch], s[qb][kb]);
                }
            }
            const bool need_mask = (k0 + BC > N) || (CAUSAL && k0 + BC - 1 > q0);
            if (need_mask) {
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
            float cj[QB], mt[QB];
            bool need = false;
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                cj[qb] = cq[qb] * sk;
                float mx = s[qb][0][0];
#pragma unroll
                for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
                    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[qb][kb][r]);
                mx = fmaxf(mx, xor32(mx));
                mt[qb] = mx * cj[qb];
                need |= mt[qb] > m_ref[qb] + kTau8;
            }
            if (wave_any(need)) {
#pragma unroll
                for (int qb = 0; qb < QB; ++qb) {
                    const float mnew = fmaxf(m_ref[qb], mt[qb]);
                    const float alpha = (mnew == -INFINITY) ? 1.f : exp2_hw(m_ref[qb] - mnew);
                    m_ref[qb] = mnew;
                    lsum[qb] *= alpha;
#pragma unroll
                    for (int db = 0; db < NDB; ++db) o[qb][db] *= alpha;
                }
            }
            i32x8 pf[QB][NPV];
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) {
                const float nm = bj - m_ref[qb];
                float ls = 0.f;
#pragma unroll
                for (int t = 0; t < NPV; ++t) {
                    uint32_t w[8];
#pragma unroll
                    for (int g = 0; g < 8; ++g) {
                        const int kb = 2 * t + g / 4, r = 4 * (g % 4);
                        float p[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) {
                            p[e] = exp2_hw(fmaf(s[qb][kb][r + e], cj[qb], nm));
                            ls += p[e];
                        }
                        w[g] = cvt4_e4m3(p[0], p[1], p[2], p[3]);
                    }
                    pf[qb][t] = i32x8{(int)w[0], (int)w[1], (int)w[2], (int)w[3],
                                      (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
                }
                lsum[qb] += ls * lscale;
            }
            // ---- O^T += V^T P'^T ----
#pragma unroll
            for (int t = 0; t < NPV; ++t) {
#pragma unroll
                for (int db = 0; db < NDB; ++db) {
                    const uint8_t* vp = vl + v_off + 64 * t * VS + 32 * db;
                    const u32x2 r0 = lds_read_tr8(vp);
                    const u32x2 r1 = lds_read_tr8(vp + 16 * VS);
                    const u32x2 r2 = lds_read_tr8(vp + 32 * VS);
                    const u32x2 r3 = lds_read_tr8(vp + 48 * VS);
                    const i32x8 a = i32x8{(int)r0[0], (int)r0[1], (int)r1[0], (int)r1[1],
                                          (int)r2[0], (int)r2[1], (int)r3[0], (int)r3[1]};
#pragma unroll
                    for (int qb = 0; qb < QB; ++qb) o[qb][db] = mfma32_fp8(a, pf[qb][t], o[qb][db]);
                }
            }
        }
        if (kt + 1 < nkt) swrite(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
        const float l = lsum[qb] + xor32(lsum[qb]);
        const float inv = svmax / (kPScale * l);
        const int row = q0 + 32 * qb + l32;
        if (row < N) {
            if (hi == 0) LSEg[(size_t)bh * N + row] = (m_ref[qb] + __builtin_amdgcn_logf(l)) * kLn2;
#pragma unroll
            for (int db = 0; db < NDB; ++db) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int dcol = 32 * db + 8 * j + 4 * hi;
                    const size_t off = head + (size_t)row * D + dcol;
                    const float v0 = o[qb][db][4 * j] * inv, v1 = o[qb][db][4 * j + 1] * inv;
                    const float v2 = o[qb][db][4 * j + 2] * inv, v3 = o[qb][db][4 * j + 3] * inv;
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
}

template <int D, bool CAUSAL, bool OUT_F32>
static hipError_t launch_t(const FwdArgs& a, hipStream_t s) {
    constexpr int BR = Cfg8<D>::NW * 32 * Cfg8<D>::QB;
    const int num_qtiles = (a.N + BR - 1) / BR;
    const long long nblk = (long long)num_qtiles * a.B * a.H;
    if (nblk > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    const int nsb = (a.N + kQuantBlockRows - 1) / kQuantBlockRows;
    hipLaunchKernelGGL((fa_fwd_fp8_kernel<D, CAUSAL, OUT_F32>), dim3((unsigned)nblk),
                       dim3(Cfg8<D>::NW * 64), 0, s, static_cast<const uint8_t*>(a.q),
                       static_cast<const uint8_t*>(a.k), static_cast<const uint8_t*>(a.v), a.o,
                       a.lse, a.N, num_qtiles, (int)nblk, nsb, a.scales_off, a.scale * kLog2e);
    return hipGetLastError();
}

template <int D>
static hipError_t launch_d(const FwdArgs& a, hipStream_t s) {
    if (a.causal)
        return a.out_f32 ? launch_t<D, true, true>(a, s) : launch_t<D, true, false>(a, s);
    return a.out_f32 ? launch_t<D, false, true>(a, s) : launch_t<D, false, false>(a, s);
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
