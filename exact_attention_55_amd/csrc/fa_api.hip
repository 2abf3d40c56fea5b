// fa_api.hip - the C ABI declared in include/fa.h: argument validation,
// status codes and dispatch to the kernel launchers. All validation happens
// before the first HIP call, so invalid calls work on hosts without a GPU.
#include "fa.h"
#include "fa_internal.h"

#include <math.h>

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_d(int d) { return d == 64 || d == 128 || d == 256; }

// B*H*N*d must stay well inside 64-bit offsets and the grid limits.
bool sizes_ok(int B, int H, int N, int d) {
    if (B < 0 || H < 0 || N < 0 || d <= 0) return false;
    const double elems = (double)B * H * N * d;
    return elems < 4.0e18;
}

int from_hip(hipError_t e) { return e == hipSuccess ? FA_OK : FA_ERR_HIP; }

// Largest K or V of one head in bytes (N * d * 2): the kernels address a
// head through 31-bit buffer offsets, with one tile of headroom.
constexpr long long kMaxHeadBytes = 0x7fffffffLL - (1 << 16);

// Most key splits of one decode call.
constexpr int kMaxSplits = 256;

}  // namespace

extern "C" {

size_t fa_fp8_scales_offset(int B, int H, int N, int d) {
    if (!sizes_ok(B, H, N, d)) return 0;
    return fa::round_up((size_t)B * H * N * d, 256);
}

size_t fa_fp8_packed_bytes(int B, int H, int N, int d) {
    if (!sizes_ok(B, H, N, d)) return 0;
    const size_t nb = ((size_t)N + fa::kQuantBlockRows - 1) / fa::kQuantBlockRows;
    return fa::round_up(fa_fp8_scales_offset(B, H, N, d) + (size_t)B * H * nb * 4, 256);
}

const char* fa_status_string(int status) {
    switch (status) {
        case FA_OK: return "ok";
        case FA_ERR_INVALID_ARG: return "invalid argument";
        case FA_ERR_UNSUPPORTED: return "unsupported configuration";
        case FA_ERR_HIP: return "HIP runtime error";
        case FA_ERR_TOO_LARGE: return "request exceeds the fixed scratch of an allocation-free entry point";
    }
    return "unknown status";
}

int fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
           int d, int causal, float softmax_scale, int dtype, void* stream) {
    const int base = dtype & 0xff;
    const int flags = dtype & ~0xff;
    if ((flags & ~(FA_OUT_F32 | FA_FWD_PIPELINED | FA_FP8_QSCALED)) != 0) return FA_ERR_INVALID_ARG;
    if (base != FA_F16 && base != FA_BF16 && base != FA_FP8_E4M3 && base != FA_FP8_MX)
        return FA_ERR_INVALID_ARG;
    if ((flags & FA_FP8_QSCALED) && base != FA_FP8_E4M3 && base != FA_FP8_MX) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, N, d)) return FA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H > 0x7fffffffLL / 2) return FA_ERR_UNSUPPORTED;
    // K and V of one head are read through 32-bit range-checked offsets.
    if ((long long)N * d * 2 > kMaxHeadBytes) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    const bool fp8 = base == FA_FP8_E4M3 || base == FA_FP8_MX;
    const size_t qa = fp8 ? 256 : 16;
    if (!aligned(q, qa) || !aligned(k, qa) || !aligned(v, qa) || !aligned(o, 16) ||
        !aligned(lse, 4))
        return FA_ERR_INVALID_ARG;

    fa::FwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.causal = causal != 0;
    a.scale = softmax_scale;
    a.out_f32 = (flags & FA_OUT_F32) != 0;
    a.scales_off = fa_fp8_scales_offset(B, H, N, d);
    a.mx = base == FA_FP8_MX;
    a.pipelined = (flags & FA_FWD_PIPELINED) != 0;
    a.qscaled = (flags & FA_FP8_QSCALED) != 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();   // do not report an earlier, unrelated error
    if (fp8) return from_hip(fa::launch_fwd_fp8(a, s));
    return from_hip(fa::launch_fwd16(a, base == FA_BF16, s));
}

int fa_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
           const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int N,
           int d, int causal, float softmax_scale, int dtype, void* stream) {
    const int base = dtype & 0xff;
    const int flags = dtype & ~0xff;
    if ((flags & ~FA_OUT_F32) != 0) return FA_ERR_INVALID_ARG;
    if (base != FA_F16 && base != FA_BF16) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, N, d)) return FA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H > 0x7fffffffLL / 2) return FA_ERR_UNSUPPORTED;
    if ((long long)N * d * 2 > kMaxHeadBytes) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || N == 0) return FA_OK;
    if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta)
        return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(dout, 16) || !aligned(dq, 16) || !aligned(dk, 16) || !aligned(dv, 16) ||
        !aligned(lse, 4) || !aligned(delta, 16))
        return FA_ERR_INVALID_ARG;

    fa::BwdArgs a;
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse; a.dout = dout;
    a.dq = dq; a.dk = dk; a.dv = dv; a.delta = delta;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.causal = causal != 0;
    a.scale = softmax_scale;
    a.out_f32 = (flags & FA_OUT_F32) != 0;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return from_hip(fa::launch_bwd16(a, base == FA_BF16, s));
}

int fa_decode_splits(int B, int H, int H_kv, int Nq, int Nk, int d) {
    if (B <= 0 || H <= 0 || H_kv <= 0 || Nq <= 0 || Nk <= 0 || H % H_kv != 0) return 1;
    if (!supported_d(d)) return 1;
    return fa::decode_default_splits(B, H, H_kv, Nq, Nk, d);
}

size_t fa_decode_workspace_bytes(int B, int H, int Nq, int d, int num_splits) {
    if (!sizes_ok(B, H, Nq, d) || num_splits <= 1 || num_splits > kMaxSplits) return 0;
    return fa::decode_workspace_bytes((long long)B * H * Nq, num_splits, d);
}

}  // extern "C"

namespace {

// Validation shared by the two decode entry points. Returns FA_OK with
// *empty set for a valid empty problem (nothing to launch). With
// caller_ws the caller's workspace must hold the split partials.
int decode_args(const void* q, const void* k, const void* v, void* o, float* lse,
                const int* seqlens_k, void* workspace, size_t workspace_bytes, bool caller_ws,
                int B, int H, int H_kv, int Nq, int Nk, int d, int causal, float softmax_scale,
                int num_splits, int dtype, void* stream, fa::DecodeArgs& a, bool* empty) {
    *empty = false;
    const int base = dtype & 0xff;
    const int flags = dtype & ~0xff;
    if ((flags & ~FA_OUT_F32) != 0) return FA_ERR_INVALID_ARG;
    if (base != FA_F16 && base != FA_BF16) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, Nq, d) || !sizes_ok(B, H_kv, Nk, d)) return FA_ERR_INVALID_ARG;
    if (H > 0 && (H_kv <= 0 || H % H_kv != 0)) return FA_ERR_INVALID_ARG;
    if (!(softmax_scale > 0.0f) || !isfinite(softmax_scale)) return FA_ERR_INVALID_ARG;
    if (num_splits < 1 || num_splits > kMaxSplits) return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if ((long long)Nk * d * 2 > kMaxHeadBytes) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || Nq == 0) {
        *empty = true;
        return FA_OK;
    }
    // the query rows sharing one key/value head are addressed with 31-bit offsets
    if ((long long)(H / H_kv) * Nq * d * 2 > kMaxHeadBytes) return FA_ERR_UNSUPPORTED;
    const long long rgroups = ((long long)(H / H_kv) * Nq + 31) / 32;
    if ((long long)B * H_kv * rgroups * num_splits > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (!q || !k || !v || !o || !lse) return FA_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) ||
        !aligned(lse, 4) || !aligned(seqlens_k, 4))
        return FA_ERR_INVALID_ARG;
    if (caller_ws && num_splits > 1) {
        const size_t need = fa::decode_workspace_bytes((long long)B * H * Nq, num_splits, d);
        if (!workspace || !aligned(workspace, 16) || workspace_bytes < need) return FA_ERR_INVALID_ARG;
    }
    a.q = q; a.k = k; a.v = v; a.o = o; a.lse = lse;
    a.seqlens = seqlens_k;
    a.workspace = workspace;
    a.B = B; a.H = H; a.Hkv = H_kv; a.Nq = Nq; a.Nk = Nk; a.d = d;
    a.causal = causal != 0;
    a.scale = softmax_scale;
    a.out_f32 = (flags & FA_OUT_F32) != 0;
    a.splits = num_splits;
    (void)stream;
    return FA_OK;
}

int prep_rope(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
              int block_rows, int in_dtype, int rope_style, float rope_base, int pos0,
              float prescale, void* stream) {
    const int pow2 = (in_dtype & FA_SCALE_POW2) != 0;
    in_dtype &= ~FA_SCALE_POW2;
    if (in_dtype != FA_BF16 && in_dtype != FA_F16) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, N, d)) return FA_ERR_INVALID_ARG;
    if (rope_style != FA_ROPE_NONE && rope_style != FA_ROPE_INTERLEAVED && rope_style != FA_ROPE_HALF)
        return FA_ERR_INVALID_ARG;
    if (rope_style != FA_ROPE_NONE) {
        if (!(rope_base > 0.0f) || !isfinite(rope_base)) return FA_ERR_INVALID_ARG;
        if (pos0 < 0 || (long long)pos0 + N > (1LL << 24)) return FA_ERR_INVALID_ARG;
    }
    if (block_rows != 0 && block_rows != fa::kQuantBlockRows) return FA_ERR_UNSUPPORTED;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * ((N + 127) / 128) > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || N == 0) return FA_OK;
    if (!x || !x8) return FA_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(x8, 256)) return FA_ERR_INVALID_ARG;

    fa::PrepArgs a;
    a.x = x; a.x8 = static_cast<uint8_t*>(x8); a.signs = signs;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.block_rows = block_rows;
    a.bf16 = in_dtype == FA_BF16;
    a.scales_off = fa_fp8_scales_offset(B, H, N, d);
    a.rope_style = rope_style;
    a.mx = fa::kMxNone;
    a.pow2 = pow2;
    a.prescale = prescale;
    a.rope.pos0 = pos0;
    for (int i = 0; i < 128; ++i)
        a.rope.w[i] = i < d / 2 ? (float)pow((double)rope_base, -2.0 * i / d) : 0.0f;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return from_hip(fa::launch_fp8_prep(a, s));
}

// Shared checks and arguments of the one-launch Q/K/V preps; returns
// FA_OK with a filled, or a status (empty problems: FA_OK with *empty set).
int qkv_args(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8,
             const int8_t* signs, int B, int H, int N, int d, int in_dtype, float q_prescale, bool mx,
             fa::PrepQkvArgs& a, bool* empty) {
    *empty = false;
    in_dtype &= ~FA_SCALE_POW2;
    if (in_dtype != FA_BF16 && in_dtype != FA_F16) return FA_ERR_INVALID_ARG;
    if (!(q_prescale > 0.0f) || !isfinite(q_prescale)) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, N, d)) return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    // workgroups of the launch (bounded above): Q and K one per 128-row
    // block; V the same (block scales) or at most one per 32-row block (MX)
    const long long bh = (long long)B * H;
    const long long wgs = 2 * bh * ((N + 127) / 128) + bh * (mx ? (N + 31) / 32 : (N + 127) / 128);
    if (wgs > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    const size_t out_bytes = mx ? fa_mx_packed_bytes(B, H, N, d) : fa_fp8_packed_bytes(B, H, N, d);
    if (B == 0 || H == 0 || N == 0) {
        *empty = true;
        return FA_OK;
    }
    const void* in[3] = {q, k, v};
    void* out[3] = {q8, k8, v8};
    for (int i = 0; i < 3; ++i) {
        if (!in[i] || !out[i]) return FA_ERR_INVALID_ARG;
        if (!aligned(in[i], 16) || !aligned(out[i], 256)) return FA_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j) {
            const uintptr_t x = (uintptr_t)out[i], y = (uintptr_t)out[j];
            if (x < y + out_bytes && y < x + out_bytes) return FA_ERR_INVALID_ARG;
        }
    a.q = q; a.k = k; a.v = v;
    a.q8 = static_cast<uint8_t*>(q8); a.k8 = static_cast<uint8_t*>(k8); a.v8 = static_cast<uint8_t*>(v8);
    a.signs = signs;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.bf16 = in_dtype == FA_BF16;
    a.scales_off = fa_fp8_scales_offset(B, H, N, d);
    a.q_prescale = q_prescale;
    return FA_OK;
}

}  // namespace

extern "C" {

int fa_fwd_decode(const void* q, const void* k, const void* v, void* o, float* lse,
                  const int* seqlens_k, void* workspace, size_t workspace_bytes, int B, int H,
                  int H_kv, int Nq, int Nk, int d, int causal, float softmax_scale, int num_splits,
                  int dtype, void* stream) {
    fa::DecodeArgs a;
    bool empty;
    const int st = decode_args(q, k, v, o, lse, seqlens_k, workspace, workspace_bytes, true, B, H,
                               H_kv, Nq, Nk, d, causal, softmax_scale, num_splits, dtype, stream, a,
                               &empty);
    if (st != FA_OK || empty) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return from_hip(fa::launch_decode16(a, (dtype & 0xff) == FA_BF16, s));
}

int fa_fwd_decode_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                          const int* seqlens_k, int B, int H, int H_kv, int Nq, int Nk, int d,
                          int causal, float softmax_scale, int num_splits, int dtype, void* stream) {
    fa::DecodeArgs a;
    bool empty;
    const int st = decode_args(q, k, v, o, lse, seqlens_k, nullptr, 0, false, B, H, H_kv, Nq, Nk,
                               d, causal, softmax_scale, num_splits, dtype, stream, a, &empty);
    if (st != FA_OK || empty) return st;
    if (num_splits > 1 &&
        fa::decode_workspace_bytes((long long)B * H * Nq, num_splits, d) > FA_NOALLOC_SCRATCH_BYTES)
        return FA_ERR_TOO_LARGE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    if (num_splits > 1) {
        void* p = nullptr;
        if (fa::decode_scratch(s, &p) != hipSuccess) return FA_ERR_HIP;
        a.workspace = p;
    }
    return from_hip(fa::launch_decode16(a, (dtype & 0xff) == FA_BF16, s));
}

int fa_fp8_prep_scaled(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
                       int block_rows, int in_dtype, int rope_style, float rope_base, int pos0,
                       float prescale, void* stream) {
    if (!(prescale > 0.0f) || !isfinite(prescale)) return FA_ERR_INVALID_ARG;
    return prep_rope(x, x8, signs, B, H, N, d, block_rows, in_dtype | FA_SCALE_POW2, rope_style,
                     rope_base, pos0, prescale, stream);
}

int fa_mx_prep_qkv(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8,
                   const int8_t* signs, int B, int H, int N, int d, int in_dtype, float q_prescale,
                   void* stream) {
    fa::PrepQkvArgs a;
    bool empty;
    const int st = qkv_args(q, k, v, q8, k8, v8, signs, B, H, N, d, in_dtype, q_prescale, true, a, &empty);
    if (st != FA_OK || empty) return st;
    (void)hipGetLastError();
    return from_hip(fa::launch_mx_prep_qkv(a, static_cast<hipStream_t>(stream)));
}

int fa_fp8_prep_qkv(const void* q, const void* k, const void* v, void* q8, void* k8, void* v8,
                    const int8_t* signs, int B, int H, int N, int d, int in_dtype, float q_prescale,
                    void* stream) {
    fa::PrepQkvArgs a;
    bool empty;
    const int st = qkv_args(q, k, v, q8, k8, v8, signs, B, H, N, d, in_dtype, q_prescale, false, a, &empty);
    if (st != FA_OK || empty) return st;
    (void)hipGetLastError();
    return from_hip(fa::launch_fp8_prep_qkv(a, static_cast<hipStream_t>(stream)));
}

int fa_fp8_prep_rope(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
                     int block_rows, int in_dtype, int rope_style, float rope_base, int pos0,
                     void* stream) {
    return prep_rope(x, x8, signs, B, H, N, d, block_rows, in_dtype, rope_style, rope_base, pos0,
                     1.0f, stream);
}

size_t fa_mx_packed_bytes(int B, int H, int N, int d) {
    if (!sizes_ok(B, H, N, d) || d % 32 != 0) return 0;
    const size_t rows = (size_t)B * H * N * (d / 32);
    const size_t cols = (size_t)B * H * ((N + 31) / 32) * d;
    return fa::round_up(fa_fp8_scales_offset(B, H, N, d) + (rows > cols ? rows : cols), 256);
}

static int mx_prep_impl(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
                        int axis, int in_dtype, float prescale, void* stream) {
    if (in_dtype != FA_BF16 && in_dtype != FA_F16) return FA_ERR_INVALID_ARG;
    if (axis != FA_MX_ALONG_D && axis != FA_MX_ALONG_N) return FA_ERR_INVALID_ARG;
    if (axis == FA_MX_ALONG_N && signs) return FA_ERR_INVALID_ARG;
    if (!sizes_ok(B, H, N, d)) return FA_ERR_INVALID_ARG;
    if (!supported_d(d)) return FA_ERR_UNSUPPORTED;
    if ((long long)B * H * ((N + 31) / 32) > 0x7fffffffLL) return FA_ERR_UNSUPPORTED;
    if (B == 0 || H == 0 || N == 0) return FA_OK;
    if (!x || !x8) return FA_ERR_INVALID_ARG;
    if (!aligned(x, 16) || !aligned(x8, 256)) return FA_ERR_INVALID_ARG;

    fa::PrepArgs a;
    a.x = x; a.x8 = static_cast<uint8_t*>(x8); a.signs = signs;
    a.B = B; a.H = H; a.N = N; a.d = d;
    a.block_rows = fa::kQuantBlockRows;
    a.bf16 = in_dtype == FA_BF16;
    a.scales_off = fa_fp8_scales_offset(B, H, N, d);
    a.rope_style = 0;
    a.rope.pos0 = 0;
    for (int i = 0; i < 128; ++i) a.rope.w[i] = 0.0f;
    a.mx = axis == FA_MX_ALONG_D ? fa::kMxAlongD : fa::kMxAlongN;
    a.prescale = prescale;
    hipStream_t s = static_cast<hipStream_t>(stream);
    (void)hipGetLastError();
    return from_hip(fa::launch_fp8_prep(a, s));
}

int fa_mx_prep(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d, int axis,
               int in_dtype, void* stream) {
    return mx_prep_impl(x, x8, signs, B, H, N, d, axis, in_dtype, 1.0f, stream);
}

int fa_mx_prep_scaled(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
                      int axis, int in_dtype, float prescale, void* stream) {
    if (!(prescale > 0.0f) || !isfinite(prescale)) return FA_ERR_INVALID_ARG;
    if (axis != FA_MX_ALONG_D) return FA_ERR_INVALID_ARG;
    return mx_prep_impl(x, x8, signs, B, H, N, d, axis, in_dtype, prescale, stream);
}

int fa_fp8_prep(const void* x, void* x8, const int8_t* signs, int B, int H, int N, int d,
                int block_rows, int in_dtype, void* stream) {
    return fa_fp8_prep_rope(x, x8, signs, B, H, N, d, block_rows, in_dtype, FA_ROPE_NONE, 1.0f, 0,
                            stream);
}

}  // extern "C"
