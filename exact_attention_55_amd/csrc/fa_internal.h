// fa_internal.h - host-side launchers shared between the C-ABI layer and the
// kernel translation units. Arguments are validated by fa_api.hip before any
// launcher runs.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fa {

constexpr int kQuantBlockRows = 128;   // rows per FP8 scale block

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
    // FP8 only: byte offset of the float32 scale array inside q/k/v
    size_t scales_off;
};

// 16-bit forward (bf16 = true: bfloat16, else float16).
hipError_t launch_fwd16(const FwdArgs& a, bool bf16, hipStream_t s);
// FP8 e4m3 forward on packed tensors.
hipError_t launch_fwd_fp8(const FwdArgs& a, hipStream_t s);

struct PrepArgs {
    const void* x;
    uint8_t* x8;
    const int8_t* signs;
    int B, H, N, d;
    int block_rows;     // 128 or 0 (per tensor)
    bool bf16;
    size_t scales_off;
};
hipError_t launch_fp8_prep(const PrepArgs& a, hipStream_t s);

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

}  // namespace fa
