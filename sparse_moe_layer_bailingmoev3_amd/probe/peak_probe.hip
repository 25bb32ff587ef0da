// Achievable-rate probes for the benchmark: what this GPU sustains for a plain HBM read, a
// plain copy and a loop of bf16 MFMAs, so that kernel figures can be set against measured
// rates beside the nominal peaks.  Built as libmoe_probe.so, separate from libmoe's ABI; only
// the benchmark loads it.  Every launch is bounded by its arguments (grid-stride loops over n
// elements; a fixed number of MFMA iterations) and writes only the sink it is given.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr uint32_t NEVER = 0x9E3779B9u;  // a sink value the data never produces in practice

// xor of n 16-byte elements: each workgroup reads spans of 8 x 4 KB (a wave instruction covers
// 1 KB), the 8 loads of a span in flight together; one word per workgroup is written only if
// the xor of its data equals NEVER, which keeps every load live
constexpr int RU = 8;
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n, uint32_t* __restrict__ sink) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t span = (size_t)RU * 256, stride = (size_t)gridDim.x * span;
  for (size_t base = (size_t)blockIdx.x * span; base < n; base += stride) {
    u32x4 v[RU];
#pragma unroll
    for (int j = 0; j < RU; ++j) {
      const size_t i = base + j * 256 + threadIdx.x;
      v[j] = i < n ? src[i] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int j = 0; j < RU; ++j) acc ^= v[j];
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == NEVER) sink[blockIdx.x] = r;
}

__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n; i += 4 * stride) {
    const u32x4 a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
    dst[i] = a;
    dst[i + stride] = b;
    dst[i + 2 * stride] = c;
    dst[i + 3 * stride] = d;
  }
  for (; i < n; i += stride) dst[i] = src[i];
}

// `iters` rounds of NACC independent 16x16x32 bf16 MFMAs per wave (operands from the lane id,
// so nothing folds; measured at 4096 workgroups: 8 chains 1.47, 16 chains 2.06, 32 chains 2.16
// PFLOP/s, so fewer chains are latency-bound); one float per workgroup is written only if the
// sum equals a value it never takes in practice
constexpr int PROBE_NACC = 32;
__global__ __launch_bounds__(256) void mfma_bf16_kernel(int iters, float* __restrict__ sink) {
  const uint32_t l = threadIdx.x;
  const u32x4 ab = {0x3F803F80u ^ (l & 7u), 0x3F003F00u ^ (l & 3u), 0x3E803E80u, 0x3F803F80u};
  const bf16x8 a = __builtin_bit_cast(bf16x8, ab);
  floatx4 acc[PROBE_NACC];
#pragma unroll
  for (int j = 0; j < PROBE_NACC; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, (float)j};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < PROBE_NACC; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, a, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < PROBE_NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == -1234.5f) sink[blockIdx.x] = s;
}

// The same loop on the scaled MFMA, 16x16x128 with both operands in FMT (0 = E4M3, 4 = E2M1,
// whose operand uses the low four dwords) and unit block scales (e8m0 127)
typedef int i32x8 __attribute__((ext_vector_type(8)));
template <int FMT>
__global__ __launch_bounds__(256) void mfma_scale_kernel(int iters, float* __restrict__ sink) {
  const int l = (int)threadIdx.x;
  const i32x8 a = {0x38383838 ^ (l & 7), 0x30303030 ^ (l & 3), 0x34343434, 0x38383838,
                   0x38383838, 0x30303030, 0x34343434 ^ (l & 1), 0x38383838};
  floatx4 acc[PROBE_NACC];
#pragma unroll
  for (int j = 0; j < PROBE_NACC; ++j) acc[j] = floatx4{0.f, 0.f, 0.f, (float)j};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < PROBE_NACC; ++j)
      acc[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, a, acc[j], FMT, FMT, 0, 127, 0, 127);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < PROBE_NACC; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  if (s == -1234.5f) sink[blockIdx.x] = s;
}

// The weight stream of the few-token expert kernel, alone: each wave reads 16 rows of a
// [rows, K] bf16 matrix in 256-value steps (8 loads of 16 bytes per lane, two steps in
// flight), lane (r, q) taking values 32i + 8q .. +7 of row r for load i.  Row-major layout:
// a load instruction covers 64 contiguous bytes of each of the 16 rows.  Blocked layout: the
// same 16 x 256 values stored as one contiguous 8 KB block per (row block, step), so a load
// instruction covers 1 KB.  Both read the same bytes; a word is written only if their xor
// equals NEVER.
template <bool BLOCKED>
__global__ __launch_bounds__(256) void frag_read_kernel(const uint16_t* __restrict__ w, int rows, int K,
                                                        uint32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int row0 = (blockIdx.x * 4 + wave) * 16;
  if (row0 >= rows) return;
  const int nsteps = K / 256;
  auto at = [&](int st, int i) {
    const size_t off = BLOCKED ? ((size_t)(row0 / 16) * nsteps + st) * 4096 + (size_t)i * 512 + lane * 8
                               : (size_t)(row0 + r16) * K + (size_t)st * 256 + i * 32 + q * 8;
    return *(const u32x4*)(w + off);
  };
  u32x4 acc = {0u, 0u, 0u, 0u};
  u32x4 v0[8], v1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) v0[i] = at(0, i);
  for (int st = 0; st < nsteps; st += 2) {  // nsteps is even
#pragma unroll
    for (int i = 0; i < 8; ++i) v1[i] = at(st + 1, i);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v0[i];
    if (st + 2 < nsteps) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v0[i] = at(st + 2, i);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) acc ^= v1[i];
  }
  const uint32_t r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == NEVER) sink[blockIdx.x] = r;
}

}  // namespace

extern "C" {

// plain HBM read of n16 16-byte elements from src; sink: device, >= grid words
int moe_probe_read(const void* src, size_t n16, void* sink, int grid, void* stream) {
  if (!src || !sink || grid <= 0) return -1;
  hipLaunchKernelGGL(read_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, n16,
                     (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// plain copy of n16 16-byte elements
int moe_probe_copy(const void* src, void* dst, size_t n16, int grid, void* stream) {
  if (!src || !dst || grid <= 0) return -1;
  hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, (const u32x4*)src, (u32x4*)dst, n16);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// independent MFMA chains per wave of the probes below
int moe_probe_mfma_chains(void) { return PROBE_NACC; }

// grid workgroups of 4 waves, each wave PROBE_NACC * iters bf16 MFMAs of 16x16x32 (2*16*16*32
// = 16384 flops each); sink: device, >= grid floats
int moe_probe_mfma_bf16(int iters, int grid, void* sink, void* stream) {
  if (!sink || grid <= 0 || iters <= 0) return -1;
  hipLaunchKernelGGL(mfma_bf16_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// the same with scaled MFMAs of 16x16x128 (65536 flops each) on E4M3 (fmt 0) or E2M1 (fmt 4)
// operands
int moe_probe_mfma_scaled(int fmt, int iters, int grid, void* sink, void* stream) {
  if (!sink || grid <= 0 || iters <= 0 || (fmt != 0 && fmt != 4)) return -1;
  if (fmt == 0)
    hipLaunchKernelGGL(mfma_scale_kernel<0>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, (float*)sink);
  else
    hipLaunchKernelGGL(mfma_scale_kernel<4>, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters, (float*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

// the few-token expert kernel's weight stream over a [rows, K] bf16 matrix, row-major
// (blocked = 0) or in contiguous 16 x 256-value blocks (blocked = 1); rows a multiple of 64, K
// of 512; one workgroup of 4 waves per 64 rows; sink: device, >= rows / 64 words
int moe_probe_frag_read(const void* w, int rows, int K, int blocked, void* sink, void* stream) {
  if (!w || !sink || rows <= 0 || rows % 64 || K <= 0 || K % 512) return -1;
  const dim3 grid(rows / 64);
  if (blocked)
    hipLaunchKernelGGL(frag_read_kernel<true>, grid, dim3(256), 0, (hipStream_t)stream, (const uint16_t*)w, rows, K,
                       (uint32_t*)sink);
  else
    hipLaunchKernelGGL(frag_read_kernel<false>, grid, dim3(256), 0, (hipStream_t)stream, (const uint16_t*)w, rows, K,
                       (uint32_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : -5;
}

}  // extern "C"
