// Device-side helpers shared by the MoE kernels (gfx950 / CDNA4, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

namespace moe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// bf16 <-> fp32 on raw bits.  fp32 -> bf16 rounds to nearest even (finite inputs).
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand a: lane l holds row (l % 16) of the
// 16-row tile, 8 consecutive k of the lane group (l / 16); operand b likewise for the
// 16 columns.  Result: lane l holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ floatx4 mfma16(const u32x4& a, const u32x4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Order-preserving map of an fp32 to uint32 (larger float -> larger integer).
__device__ __forceinline__ uint32_t f32_ordered(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  return v;
}

// Map a linear block id to a work id so that consecutive work ids run on the same
// XCD: the hardware deals blocks round-robin over the 8 XCDs, so block b lands on
// XCD b % 8.  `nblocks` must be a multiple of 8.
__device__ __forceinline__ int xcd_major(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

}  // namespace moe
