// fa_device.h - gfx950 device primitives shared by the attention kernels.
//
// Thin wrappers over the CDNA4 matrix-core, LDS and cross-lane builtins, plus
// the register-fragment types they use. Nothing here knows about attention.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace fa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(8))) int32_t i32x8;
typedef __attribute__((vector_size(2 * sizeof(int)))) int i32x2v;

#define FA_LDS __attribute__((address_space(3)))

// Element-type traits for the two 16-bit input types.
template <typename T> struct Elt;
template <> struct Elt<__bf16> {
    using x8 = bf16x8;
    using x2 = bf16x2;
};
template <> struct Elt<_Float16> {
    using x8 = f16x8;
    using x2 = f16x2;
};

// Two floats rounded (RNE) to the 16-bit type, packed.
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

// D(32x32 f32) += A(32x16) * B(16x32), 16-bit operands, fp32 accumulate.
// Operand layout (wave64): lane l holds row/column (l % 32) and 8 consecutive
// k values of k-group (l / 32). Accumulator: lane l holds column l % 32,
// register r holds row 8*(r/4) + 4*(l/32) + (r%4).
__device__ __forceinline__ f32x16 mfma32(const bf16x8& a, const bf16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma32(const f16x8& a, const f16x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// acc += A B with acc bound to the accumulation registers (AGPRs) through
// inline asm, for kernels that keep large accumulators there for their whole
// life (one wave per SIMD). The compiler does not treat these as MFMAs: the
// caller makes sure their vector inputs were written at least two wait
// states before (or by loads the compiler waits for), and that vector
// instructions read acc only after the MFMA's result latency.
__device__ __forceinline__ void mfma_acc(f32x16& acc, const bf16x8& a, const bf16x8& b) {
    asm("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc(f32x16& acc, const f16x8& a, const f16x8& b) {
    asm("v_mfma_f32_32x32x16_f16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}
// Waits out the result latency of the asm MFMAs that last wrote the given
// accumulators before vector instructions read them.
__device__ __forceinline__ void acc_settle(f32x16& a0, f32x16& a1, f32x16& a2, f32x16& a3) {
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4" : "+a"(a0), "+a"(a1), "+a"(a2), "+a"(a3));
}

// o *= a on accumulators that live in the accumulation registers (AGPRs):
// each element is read out, scaled and written back in one asm block. A
// plain vector multiply there makes the compiler keep a VGPR copy of every
// accumulator across the key loop (copied in at every iteration) because
// VALU instructions cannot name AGPRs; with this form the accumulators stay
// in AGPRs and only the rarely taken rescale moves them. The compiler adds no
// wait states for an asm read of an MFMA result, so the first read carries
// them itself: 21 (s_nop 7, 7, 4) cover the longest MFMA write -> VALU read
// distance of gfx950 (a 16-pass 32x32 MFMA needs 18), whatever the caller
// issued just before. Later reads come after it in program order. The last
// write is followed by 3 more so that an MFMA reading o as its accumulator
// input right after the call sees the written value.
__device__ __forceinline__ void scale_acc(f32x16& o, float a) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        float x = o[i], t;
        if (i == 0)
            asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 4\n\t"
                         "v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t) : "v"(a));
        else if (i == 15)
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1\n\t"
                         "s_nop 2"
                         : "+a"(x), "=&v"(t) : "v"(a));
        else
            asm volatile("v_accvgpr_read_b32 %1, %0\n\tv_mul_f32 %1, %1, %2\n\tv_accvgpr_write_b32 %0, %1"
                         : "+a"(x), "=&v"(t) : "v"(a));
        o[i] = x;
    }
}

// D(32x32 f32) += A(32x64) * B(64x32) with OCP e4m3 operands (32 bytes per
// lane per operand) and unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ f32x16 mfma32_fp8(const i32x8& a, const i32x8& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// Same with per-lane E8M0 scales: lane l's 32 A values (row l % 32, k-half
// l / 32) are multiplied by 2^(sa - 127), its 32 B values by 2^(sb - 127).
__device__ __forceinline__ f32x16 mfma32_fp8s(const i32x8& a, const i32x8& b, const f32x16& c, int sa,
                                              int sb) {
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, sa, 0, sb);
}

// Transposing LDS read of 16-bit data. Within each group of 16 lanes the 16
// eight-byte reads form a 4 x 16 tile (lane j supplies row j/4, columns
// 4*(j%4) .. +3); lane i of the group receives column i, rows 0..3.
__device__ __forceinline__ u32x2 lds_read_tr16(const void* p) {
    bf16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((FA_LDS bf16x4*)(p));
    return __builtin_bit_cast(u32x2, v);
}

// Same for 8-bit data: the 16 reads form an 8 x 16 tile (lane j supplies row
// j/2, columns 8*(j%2) .. +7); lane i receives column i, rows 0..7.
__device__ __forceinline__ u32x2 lds_read_tr8(const void* p) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr8_b64_v2i32((FA_LDS i32x2v*)(p)));
}

// The same two reads issued through inline asm, with no wait attached. The
// compiler cannot tell the LDS tiles apart, so after any direct-to-LDS copy
// it makes a transposing-read builtin wait for every outstanding copy, a
// full memory latency in the middle of the key loop. The tiles read here are
// ordered against the copies by explicit waits and barriers instead. The
// result is valid only after lgkm_wait() covers the read and lgkm_bind()
// ties the registers to that wait. OFF is a byte offset < 65536.
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr16_async(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x2 lds_tr8_async(uint32_t addr) {
    u32x2 r;
    asm volatile("ds_read_b64_tr_b8 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "n"(OFF));
    return r;
}
// Wait until at most N LDS (and scalar-memory) requests of the wave are in
// flight. LDS requests complete in issue order, so this covers every read
// issued before the last N.
template <int N>
__device__ __forceinline__ void lgkm_wait() {
    static_assert(N >= 0 && N <= 15, "lgkmcnt is a 4-bit field");
    asm volatile("s_waitcnt lgkmcnt(%0)" ::"n"(N));
}
// Orders every use of x after the preceding lgkm_wait (both are volatile asm,
// which the compiler keeps in order).
__device__ __forceinline__ void lgkm_bind(u32x2& x) { asm volatile("" : "+v"(x)); }

// 32-bit LDS address of a pointer into a __shared__ array.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(const FA_LDS char*)(p);
}

// Compile-time loop: f(std::integral_constant<int, i>) for i in [I, N).
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (I < N) {
        f(std::integral_constant<int, I>{});
        static_for<I + 1, N>(f);
    }
}

// Hardware base-2 exponential (v_exp_f32).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Value held by lane (l ^ 32).
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over the lane pair (l, l ^ 32), on the VALU: permlane32_swap
// of (x, x) returns the lower half-wave's values in the first result and the
// upper half-wave's in the second, in every lane.
__device__ __forceinline__ float pair_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

template <typename V>
__device__ __forceinline__ V load16(const void* p) {
    return __builtin_bit_cast(V, *reinterpret_cast<const u32x4*>(p));
}

constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kLog2e = 1.44269504088896340736f;

// Score tiles are computed transposed (S^T = K Q^T) with 32x32 MFMA. The key
// row fed to MFMA row m of a 32-key block is perm(m) = m with bits 2 and 3
// swapped, so that accumulator register r of a lane in half-wave hi holds key
//   32*kb + perm(8*(r/4) + 4*hi + r%4) = 32*kb + 16*(r/8) + 8*hi + (r%8):
// every run of 8 registers is 8 consecutive keys, which is what the
// transposing LDS reads of V deliver for the P V product.
__device__ __forceinline__ int krow_perm(int m) {
    return (m & ~12) | ((m >> 1) & 4) | ((m << 1) & 8);
}
__device__ __forceinline__ int key_of(int kb, int r, int hi) {
    return 32 * kb + 16 * (r >> 3) + 8 * hi + (r & 7);
}

// LDS tiles hold rows unpadded; the 16-byte chunk c of row r is stored at
// chunk position c ^ swz(r). The LDS serves 64 four-byte banks (256 bytes)
// per cycle: 16 lanes of a 16-byte read or 32 lanes of an 8-byte read. The
// swizzle makes both access patterns of the kernels hit 16 distinct bank
// groups: the score MFMA's K reads (one chunk from 16 rows {0..15} of a
// 32-key block) and the transposing V reads (4 rows x 4 chunks for 16-bit,
// 8 rows x 2 chunks for 8-bit data, per 32 lanes).
//   16-bit rows of 2*D bytes:  D = 64 (two rows per 256 bytes):
//     swz = 4*((r>>1)&1) + ((r>>2)&3);  D >= 128: swz = 4*(r&3) + ((r>>2)&3)
template <int D> __device__ __forceinline__ int lds_swz16(int r) {
    if (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
    return ((r & 3) << 2) | ((r >> 2) & 3);
}
//   8-bit rows of D bytes: D = 64 (four rows per 256 bytes), 128 (two), 256.
template <int D> __device__ __forceinline__ int lds_swz8(int r) {
    if (D == 64) return (((r >> 2) & 1) << 1) | ((r >> 3) & 1);
    if (D == 128) return (((r >> 1) & 3) << 1) | ((r >> 3) & 1);
    return ((r & 7) << 1) | ((r >> 3) & 1);
}

// Buffer resource over [base, base + bytes): raw (stride 0) byte-addressed
// loads, range-checked against bytes. On gfx950 the check covers the whole
// offset (VGPR offset + SGPR offset): a 16-byte read at or past the end
// returns zeros, also into LDS. bytes must be < 2^31; base wave-uniform.
typedef __attribute__((ext_vector_type(4))) int i32x4;
__device__ __forceinline__ i32x4 make_rsrc(const void* base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane((int)(uint32_t)a),
                 __builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32) & 0xffff),
                 __builtin_amdgcn_readfirstlane(bytes), 0x00020000};
}
// 16 bytes per lane from a buffer straight into LDS: lane i's bytes come
// from offset voff + soff and land at LDS address lds + 16*i (lds and soff
// wave-uniform). Issued through inline asm so that the compiler does not
// track it: otherwise it makes LDS reads wait for every outstanding copy,
// because it cannot tell the tiles apart. Completion is awaited explicitly
// (wait_vm_all) before the barrier that publishes the tile. The LDS address
// goes through M0, which the statement declares clobbered: M0 is reserved
// (never given to an "s" operand), and the clobber keeps any value the
// compiler holds in it from being assumed live across the copy (clang warns
// that a reserved register is named; the warning is silenced here only).
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void buffer_load_lds16(i32x4 rsrc, uint32_t lds, uint32_t voff,
                                                  uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
// 4 bytes per lane (lane i at lds + 4*i), otherwise as buffer_load_lds16.
__device__ __forceinline__ void buffer_load_lds4(i32x4 rsrc, uint32_t lds, uint32_t voff, uint32_t soff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
                 :: "s"(lds), "v"(voff), "s"(rsrc), "s"(soff) : "memory", "m0");
}
#pragma clang diagnostic pop

// Workgroup -> (head, tile level) for a grid of heads x tiles workgroups.
// Balanced (non-causal): consecutive workgroups land on different XCDs, so
// they are regrouped to let each XCD walk whole heads (a head's K/V then stay
// in that XCD's L2). Unbalanced (causal): workgroup i takes level i / heads
// of head i % heads, so level 0 (the caller's heaviest tile) of every head is
// dispatched before any lighter one; a head's tiles still share one XCD when
// the head count is a multiple of 8.
__device__ __forceinline__ void grid_tile(int num_blocks, int num_tiles, bool unbalanced, int& bh,
                                          int& level) {
    const int i = blockIdx.x;
    if (unbalanced) {
        const int heads = num_blocks / num_tiles;
        level = i / heads;
        bh = i - level * heads;
        return;
    }
    const int bid = ((num_blocks & 7) == 0) ? (i & 7) * (num_blocks >> 3) + (i >> 3) : i;
    bh = bid / num_tiles;
    level = bid - bh * num_tiles;
}

__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ float uniform_f(float x) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(x)));
}

// E8M0 byte (127 + k) of f = 2^k, a normal float32 power of two; -1 for any
// other value (frexp: f = 0.5 * 2^(k + 1), k + 1 in [-125, 128] when normal).
__device__ __forceinline__ int e8m0_of_pow2(float f) {
    const int e = __builtin_amdgcn_frexp_expf(f);
    return (__builtin_amdgcn_frexp_mantf(f) == 0.5f && e >= -125 && e <= 128) ? 126 + e : -1;
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt(0), other counters ignored.
constexpr int kVmcnt0 = 0x0f70;

// Wait until this wave's global loads (including direct-to-LDS ones) landed.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
// Wait until at most N of this wave's global loads are still in flight (they
// complete in issue order for this count).
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N <= 63, "vmcnt is a 6-bit field");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Workgroup barrier after this wave's global->LDS copies, except the newest
// VM of them, have landed. Nothing is scheduled across it and memory
// accesses are not moved across it.
template <int VM>
__device__ __forceinline__ void sync_tiles() {
    static_assert(VM >= 0 && VM <= 63, "vmcnt is a 6-bit field");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_barrier" ::"n"(VM) : "memory");
    __builtin_amdgcn_sched_barrier(0);
}

}  // namespace fa
