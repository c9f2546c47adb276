// kd_common.hpp -- device helpers shared by the gfx950 kernels of the fused
// top-K KL loss: element types, raw buffer loads with hardware bounds checks,
// LDS tile swizzle, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kd {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Storage tag of a bfloat16 element (raw 16 bits).
struct bf16_t { uint16_t bits; };

constexpr int kThreads = 256;          // 4 wave64 per workgroup
constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Byte offset that every buffer resource below treats as out of range: loads
// from it return zero (operand extents are kept below 2^31 bytes on the host).
constexpr uint32_t kOOB = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    // gfx9 raw buffer: stride 0, num_records = bytes, dword3 = 32-bit data format.
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ u32x4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

// Two fp32 -> packed bf16x2 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// Combine lanes l and l ^ 32 with one VALU swap of the two 32-lane halves
// (v_permlane32_swap) instead of an LDS permute: x[l] and x[l ^ 32] end up in
// the two results, in some order, on every lane.
__device__ __forceinline__ float halves_max(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float halves_sum(float v) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS operand tiles are ROWS x 128 bytes (one row = 128 bytes of the K
// extent).  The 16-byte chunk c of row r lives at chunk position
// c ^ ((r ^ (r >> 3)) & 7): rows that differ in their low three bits, or in
// bits 3..5 at a fixed low part, land in different banks, which keeps both
// the row-wise fragment reads and the column-wise transposed stores free of
// bank conflicts.
__device__ __forceinline__ int lds_off(int r, int c) {
    return (r << 7) + ((c ^ ((r ^ (r >> 3)) & 7)) << 4);
}

// Clamp an untrusted id into [0, V).
__device__ __forceinline__ int clamp_id(int v, int V) {
    return v < 0 ? 0 : (v >= V ? V - 1 : v);
}

}  // namespace kd
