// Combine: the layer output of each token is the weighted sum of its routed experts'
// outputs plus the shared expert's output (routing walk-through page, lqnn.cn, section 二:
// the shared expert sees every token; section 四: routed weights renormalised and scaled by
// routed_scaling_factor).  Deterministic: fp32 sum of the fp32 expert outputs over the slots
// in their stored order (ascending expert id), shared expert last, one rounding to bf16.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// one workgroup per token; each thread owns 8 consecutive hidden values (16 bytes)
__global__ __launch_bounds__(512) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int K, int H, int S,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int64_t shared_row = (int64_t)T * K + t;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int p = inv[(size_t)t * K + k];
      if (p < 0) continue;
      const float wk = w[(size_t)t * K + k];
      const float4 v0 = *(const float4*)(y + (size_t)p * H + c);
      const float4 v1 = *(const float4*)(y + (size_t)p * H + c + 4);
      acc[0] = fmaf(wk, v0.x, acc[0]);
      acc[1] = fmaf(wk, v0.y, acc[1]);
      acc[2] = fmaf(wk, v0.z, acc[2]);
      acc[3] = fmaf(wk, v0.w, acc[3]);
      acc[4] = fmaf(wk, v1.x, acc[4]);
      acc[5] = fmaf(wk, v1.y, acc[5]);
      acc[6] = fmaf(wk, v1.z, acc[6]);
      acc[7] = fmaf(wk, v1.w, acc[7]);
    }
    if (S) {
      const float4 v0 = *(const float4*)(y + (size_t)shared_row * H + c);
      const float4 v1 = *(const float4*)(y + (size_t)shared_row * H + c + 4);
      acc[0] += v0.x;
      acc[1] += v0.y;
      acc[2] += v0.z;
      acc[3] += v0.w;
      acc[4] += v1.x;
      acc[5] += v1.y;
      acc[6] += v1.z;
      acc[7] += v1.w;
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(u32x4*)(out + (size_t)t * H + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const float* y_sorted, const int32_t* inv_perm, const float* topk_w, int T, int K, int H,
                          int S, uint16_t* out, hipStream_t s, Tracer* tr) {
  int threads = ((H / 8 + 63) / 64) * 64;
  threads = std::min(threads, 512);
  hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(threads), 0, s, y_sorted, inv_perm, topk_w, T, K, H, S, out);
  hipError_t err = hipGetLastError();
  if (tr) tr->mark("combine", s);
  return err;
}

}  // namespace moe
