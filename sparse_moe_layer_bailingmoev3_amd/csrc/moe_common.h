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
// two fp32 -> two fp16 (round to nearest even), saturated at +-65504 (finite inputs), low
// half first
__device__ __forceinline__ uint32_t pack_f16x2_sat(float lo, float hi) {
  lo = fminf(fmaxf(lo, -65504.f), 65504.f);
  hi = fminf(fmaxf(hi, -65504.f), 65504.f);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}

// 16x16x32 bf16 MFMA, fp32 accumulate.  Operand a: lane l holds row (l % 16) of the
// 16-row tile, 8 consecutive k of the lane group (l / 16); operand b likewise for the
// 16 columns.  Result: lane l holds column (l % 16), rows 4*(l/16) .. 4*(l/16)+3.
__device__ __forceinline__ floatx4 mfma16(const u32x4& a, const u32x4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// 16x16x32 fp16 MFMA, fp32 accumulate; same operand and result layout as mfma16
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ floatx4 mfma16_f16(const u32x4& a, const u32x4& b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// eight bf16 -> eight fp16: exact for magnitudes from 2^-17 (fp16 keeps the 8 significant bits
// of bf16 down to there) up to 65504; smaller ones lose low bits toward zero (an absolute
// error below 2^-24), larger ones (never bf16 model weights) become infinite
__device__ __forceinline__ u32x4 bf16x8_to_f16x8(const u32x4& w) {
  u32x4 r;
#pragma unroll
  for (int i = 0; i < 4; ++i)
    r[i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__uint_as_float(w[i] << 16),
                                                                     __uint_as_float(w[i] & 0xFFFF0000u)));
  return r;
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

// ---- MXFP8 (OCP MX v1.0, E4M3 elements, one e8m0 scale per 32 values) ----------------
// Shared-scale byte of a block from its largest magnitude: X = floor(log2 amax) - 8 (8 = the
// exponent of E4M3's largest normal, 448), clamped to [-127, 127], stored as X + 127; an
// all-zero block (or one below fp32's normal range) gets X = -127.
__device__ __forceinline__ int mx8_scale_byte(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 0xFFu);  // biased exponent: floor(log2) + 127
  if (ef == 0) return 0;
  return min(254, max(0, ef - 8));
}

// Four values of a block with shared exponent X (= scale byte - 127) -> four E4M3 codes, low
// byte first: v * 2^-X (exact), clamped to +-448 so nothing overflows, then gfx950's fp32 ->
// E4M3 conversion (round to nearest even).
__device__ __forceinline__ uint32_t mx8_pack4(float v0, float v1, float v2, float v3, int X) {
  const float c = 448.0f;
  v0 = fminf(fmaxf(__builtin_amdgcn_ldexpf(v0, -X), -c), c);
  v1 = fminf(fmaxf(__builtin_amdgcn_ldexpf(v1, -X), -c), c);
  v2 = fminf(fmaxf(__builtin_amdgcn_ldexpf(v2, -X), -c), c);
  v3 = fminf(fmaxf(__builtin_amdgcn_ldexpf(v3, -X), -c), c);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(v0, v1, 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(v2, v3, w, true);
  return (uint32_t)w;
}

// Map a linear block id to a work id so that consecutive work ids run on the same
// XCD: the hardware deals blocks round-robin over the 8 XCDs, so block b lands on
// XCD b % 8.  `nblocks` must be a multiple of 8.
__device__ __forceinline__ int xcd_major(int b, int nblocks) {
  return (b & 7) * (nblocks >> 3) + (b >> 3);
}

}  // namespace moe
