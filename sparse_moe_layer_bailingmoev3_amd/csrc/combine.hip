// Combine: the layer output of each token is the weighted sum of its routed experts'
// outputs plus the shared expert's output (routing walk-through page, lqnn.cn, section 二:
// the shared expert sees every token; section 四: routed weights renormalised and scaled by
// routed_scaling_factor).  Deterministic: fp32 sum of the expert outputs (fp32, or fp16 as the
// 256-position tile kernels write them inside moe_forward) over the slots
// in their stored order (ascending expert id), shared expert last, one rounding to bf16.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// one workgroup per token; each thread owns 8 consecutive hidden values.  The rows of 8 slots
// are loaded in one batch (a slot without a row loads row 0 and is skipped in the sum), so a
// token costs one round trip per 8 slots instead of one per slot.  Y16: y holds fp16 values
// (8 per 16-byte load), else fp32 (8 per two 16-byte loads); both are summed in fp32.
constexpr int CB = 8;

template <bool Y16>
__device__ __forceinline__ void load8(const void* y, size_t idx, float (&r)[8]) {
  if constexpr (Y16) {
    const u32x4 v = *(const u32x4*)((const uint16_t*)y + idx);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      r[2 * i] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] & 0xFFFFu));
      r[2 * i + 1] = (float)__builtin_bit_cast(_Float16, (uint16_t)(v[i] >> 16));
    }
  } else {
    const float4 a = *(const float4*)((const float*)y + idx);
    const float4 b = *(const float4*)((const float*)y + idx + 4);
    r[0] = a.x; r[1] = a.y; r[2] = a.z; r[3] = a.w;
    r[4] = b.x; r[5] = b.y; r[6] = b.z; r[7] = b.w;
  }
}

template <bool Y16>
__global__ __launch_bounds__(512) void combine_kernel(const void* __restrict__ y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int K, int H, int S,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int64_t shared_row = (int64_t)T * K + t;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // the shared expert's row does not depend on the slot indices: load it first
    float sh[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sh[i] = 0.f;
    if (S) load8<Y16>(y, (size_t)shared_row * H + c, sh);
    for (int k0 = 0; k0 < K; k0 += CB) {
      // slot indices and weights read unconditionally (clamped to the last slot) so that
      // they go out as one batch
      int p[CB];
      float wt[CB];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        const int k = min(k0 + u, K - 1);
        p[u] = inv[(size_t)t * K + k];
        wt[u] = w[(size_t)t * K + k];
      }
      float v[CB][8];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (k0 + u >= K) p[u] = -1;
        load8<Y16>(y, (size_t)(p[u] < 0 ? 0 : p[u]) * H + c, v[u]);
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        // a skipped slot keeps the sum as it is (a select, not a branch, so that the weight
        // loads stay in the batch)
        const float wk = wt[u];
        const bool use = p[u] >= 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = use ? fmaf(wk, v[u][i], acc[i]) : acc[i];
      }
    }
    if (S) {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += sh[i];
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pack_bf16x2(acc[2 * i], acc[2 * i + 1]);
    *(u32x4*)(out + (size_t)t * H + c) = o;
  }
}

}  // namespace

hipError_t launch_combine(const void* y_sorted, const int32_t* inv_perm, const float* topk_w, int T, int K, int H,
                          int S, uint16_t* out, hipStream_t s, Tracer* tr, bool y16) {
  int threads = ((H / 8 + 63) / 64) * 64;
  threads = std::min(threads, 512);
  if (y16)
    launch(tr, combine_kernel<true>, dim3(T), dim3(threads), s, y_sorted, inv_perm, topk_w, T, K, H, S, out);
  else
    launch(tr, combine_kernel<false>, dim3(T), dim3(threads), s, y_sorted, inv_perm, topk_w, T, K, H, S, out);
  hipError_t err = hipGetLastError();
  if (tr) tr->mark("combine", s);
  return err;
}

}  // namespace moe
