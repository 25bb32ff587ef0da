// Combine: the layer output of each token is the weighted sum of its routed experts'
// outputs plus the shared expert's output (routing walk-through page, lqnn.cn, section 二:
// the shared expert sees every token; section 四: routed weights renormalised and scaled by
// routed_scaling_factor).  Deterministic: fp32 sum of the fp32 expert outputs over the slots
// in their stored order (ascending expert id), shared expert last, one rounding to bf16.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

// one workgroup per token; each thread owns 8 consecutive hidden values (16 bytes).  The
// rows of 8 slots are loaded in one batch (a slot without a row loads row 0 and is skipped
// in the sum), so a token costs one round trip per 8 slots instead of one per slot.
constexpr int CB = 8;

__global__ __launch_bounds__(512) void combine_kernel(const float* __restrict__ y, const int32_t* __restrict__ inv,
                                                      const float* __restrict__ w, int T, int K, int H, int S,
                                                      uint16_t* __restrict__ out) {
  const int t = blockIdx.x;
  const int64_t shared_row = (int64_t)T * K + t;
  for (int c = threadIdx.x * 8; c < H; c += blockDim.x * 8) {
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // the shared expert's row does not depend on the slot indices: load it first
    float4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
    if (S) {
      s0 = *(const float4*)(y + (size_t)shared_row * H + c);
      s1 = *(const float4*)(y + (size_t)shared_row * H + c + 4);
    }
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
      float4 v[CB][2];
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        if (k0 + u >= K) p[u] = -1;
        const float* row = y + (size_t)(p[u] < 0 ? 0 : p[u]) * H + c;
        v[u][0] = *(const float4*)row;
        v[u][1] = *(const float4*)(row + 4);
      }
#pragma unroll
      for (int u = 0; u < CB; ++u) {
        // a skipped slot keeps the sum as it is (a select, not a branch, so that the weight
        // loads stay in the batch)
        const float wk = wt[u];
        const bool use = p[u] >= 0;
        const float r[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w, v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = use ? fmaf(wk, r[i], acc[i]) : acc[i];
      }
    }
    if (S) {
      acc[0] += s0.x;
      acc[1] += s0.y;
      acc[2] += s0.z;
      acc[3] += s0.w;
      acc[4] += s1.x;
      acc[5] += s1.y;
      acc[6] += s1.z;
      acc[7] += s1.w;
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
  launch(tr, combine_kernel, dim3(T), dim3(threads), s, y_sorted, inv_perm, topk_w, T, K, H, S, out);
  hipError_t err = hipGetLastError();
  if (tr) tr->mark("combine", s);
  return err;
}

}  // namespace moe
