// fa_internal.h - host-side launchers shared between the C-ABI layer and the
// kernel translation units. Arguments are validated by fa_api.hip before any
// launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

constexpr int kQuantBlockRows = 128;   // rows per FP8 scale block
constexpr int kMxNone = -1, kMxAlongD = 0, kMxAlongN = 1;   // PrepArgs::mx

struct FwdArgs {
    const void* q;
    const void* k;
    const void* v;
    void* o;
    float* lse;
    int B, H, N, d;
    bool causal;
    float scale;        // softmax scale
    bool out_f32;
    // FP8 only: byte offset of the scale array inside q/k/v
    size_t scales_off;
    bool mx = false;    // FP8: microscaled inputs (E8M0 scales per 32 elements)
    bool qscaled = false;   // FP8: q carries softmax_scale * log2(e) (power-of-two block scales)
    bool pipelined = false;   // 16-bit, d = 128: the 64-rows-per-wave pipelined kernel
};

// 16-bit forward (bf16 = true: bfloat16, else float16).
hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t s);
// 16-bit forward at d = 128 with 64 query rows per wave and the in-wave
// three-stage pipeline (fa_fwd16_pipe.hip).
hipError_t launch_fwd16_pipe(const FwdArgs& a, bool bf16, hipStream_t s);
// FP8 e4m3 forward on packed tensors.
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t s);

// Rotary frequencies w_i (float32, i < d/2) and the first row's position,
// passed to the prep kernel by value.
struct RopeFreqs {
    float w[128];
    int pos0;
};

struct PrepArgs {
    const void* x;
    uint8_t* x8;
    const int8_t* signs;
    int B, H, N, d;
    int block_rows;     // 128 or 0 (per tensor)
    bool bf16;
    size_t scales_off;
    int rope_style;     // 0 none, 1 interleaved pairs, 2 half pairs
    RopeFreqs rope;
    int mx;             // kMxNone: fp32 block scales; microscaling along d or n
    int pow2 = 0;       // fp32 block scales rounded up to powers of two
    float prescale = 1.0f;   // factor on the (rotated) values before the block maximum
};
hipError_t launch_fp8_prep(const PrepArgs& a, hipStream_t s);

// Q, K and V prepared in one launch (block scales, powers of two; Q and K
// through the transform when signs is set, Q times q_prescale).
struct PrepQkvArgs {
    const void* q;
    const void* k;
    const void* v;
    uint8_t* q8;
    uint8_t* k8;
    uint8_t* v8;
    const int8_t* signs;
    int B, H, N, d;
    bool bf16;
    size_t scales_off;
    float q_prescale;
};
hipError_t launch_fp8_prep_qkv(const PrepQkvArgs& a, hipStream_t s);
// The same for microscaled inputs (q, k along d; v along the sequence).
hipError_t launch_mx_prep_qkv(const PrepQkvArgs& a, hipStream_t s);

struct BwdArgs {
    const void* q;
    const void* k;
    const void* v;
    const void* o;
    const float* lse;
    const void* dout;
    void* dq;
    void* dk;
    void* dv;
    float* delta;       // caller scratch [2][B][H][N]: rowsum(dO * O), -LSE / scale
    int B, H, N, d;
    bool causal;
    float scale;
    bool out_f32;       // gradients as float32
};
// 16-bit backward (bf16 = true: bfloat16, else float16), d = 64 or 128.
hipError_t launch_bwd16(const BwdArgs& a, bool bf16, hipStream_t s);

inline size_t round_up(size_t x, size_t m) { return (x + m - 1) / m * m; }

struct DecodeArgs {
    const void* q;      // [B][H][Nq][d]
    const void* k;      // [B][Hkv][Nk][d]
    const void* v;
    void* o;            // [B][H][Nq][d]
    float* lse;         // [B][H][Nq]
    const int* seqlens; // [B] keys per sequence (clamped to [0, Nk]), or null: Nk
    void* workspace;    // partial results when splits > 1
    int B, H, Hkv, Nq, Nk, d;
    bool causal;
    float scale;
    bool out_f32;
    int splits;
};
// Bytes of the partial-O block at the start of the workspace, and of the
// whole workspace (partial O, then partial LSE), for rows = B*H*Nq.
size_t decode_partial_o_bytes(long long rows, int splits, int d);
size_t decode_workspace_bytes(long long rows, int splits, int d);
int decode_default_splits(int B, int H, int Hkv, int Nq, int Nk, int d);
// Decode-shaped 16-bit forward (bf16 = true: bfloat16, else float16).
hipError_t launch_decode16(const DecodeArgs& a, bool bf16, hipStream_t s);
// Device address of the fixed decode scratch (FA_NOALLOC_SCRATCH_BYTES) on
// the device of stream s (the current device for a null stream), looked up
// once per device.
hipError_t decode_scratch(hipStream_t s, void** ptr);

}  // namespace fa
