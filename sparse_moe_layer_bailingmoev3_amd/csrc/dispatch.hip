// Dispatch: group the (token, slot) pairs chosen by the router by expert, so the expert
// FFNs can run as a grouped GEMM over contiguous row blocks (the routing walk-through page,
// lqnn.cn, section 三.2, ends with 8 experts per token; each expert then serves its tokens).
//
// Deterministic and atomic-order independent:
//   1. mark     one bit per (expert, token) in a bitmap [E][ceil(T/32)] (atomicOr only sets
//               bits, so the result does not depend on the order of the atomics);
//   2. count    one wave per expert: popcount of its bitmap row -> counts[e];
//   3. scan     one wave: exclusive prefix sum of counts -> offsets;
//   4. scatter  one wave per expert walks its row in ascending token order and writes
//               sorted_token and inv_perm; the shared expert's block is the identity.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void dispatch_mark_kernel(const int32_t* __restrict__ topk_idx, int T, int K, int E, int words,
                                     uint32_t* __restrict__ bitmap, int32_t* __restrict__ inv_perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * K) return;
  const int e = topk_idx[i];
  const int t = (int)(i / K);
  if (e >= 0 && e < E)
    atomicOr(&bitmap[(size_t)e * words + (t >> 5)], 1u << (t & 31));
  else
    inv_perm[i] = -1;  // ignored pair
}

// one wave per expert (plus one wave that writes the shared expert's count)
__global__ __launch_bounds__(256) void dispatch_count_kernel(const uint32_t* __restrict__ bitmap, int E, int words,
                                                             int T, int S, int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e > E) return;
  if (e == E) {
    if (lane == 0) counts[E] = T * S;
    return;
  }
  const uint32_t* row = bitmap + (size_t)e * words;
  int c = 0;
  for (int w = lane; w < words; w += WAVE) c += __popc(row[w]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, WAVE);
  if (lane == 0) counts[e] = c;
}

// single wave: offsets[0] = 0, offsets[i+1] = offsets[i] + counts[i] for i < n
__global__ __launch_bounds__(64) void exclusive_scan_kernel(const int32_t* __restrict__ counts, int n,
                                                            int32_t* __restrict__ offsets) {
  const int lane = threadIdx.x;
  const int per = (n + WAVE - 1) / WAVE;
  const int b = lane * per, e = min(n, b + per);
  int sum = 0;
  for (int i = b; i < e; ++i) sum += counts[i];
  int incl = sum;
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) {
    int o = __shfl_up(incl, m, WAVE);
    if (lane >= m) incl += o;
  }
  int run = incl - sum;
  if (lane == 0) offsets[0] = 0;
  for (int i = b; i < e; ++i) {
    run += counts[i];
    offsets[i + 1] = run;
  }
}

// one wave per expert; expert E (if S) writes the identity block
__global__ __launch_bounds__(256) void dispatch_scatter_kernel(const uint32_t* __restrict__ bitmap,
                                                               const int32_t* __restrict__ offsets,
                                                               const int32_t* __restrict__ topk_idx, int T, int K,
                                                               int E, int words, int S,
                                                               int32_t* __restrict__ sorted_token,
                                                               int32_t* __restrict__ inv_perm) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e > E || (e == E && !S)) return;
  int base = offsets[e];
  if (e == E) {
    for (int t = lane; t < T; t += WAVE) sorted_token[base + t] = t;
    return;
  }
  const uint32_t* row = bitmap + (size_t)e * words;
  for (int w0 = 0; w0 < words; w0 += WAVE) {
    const int w = w0 + lane;
    uint32_t bits = w < words ? row[w] : 0u;
    const int c = __popc(bits);
    int incl = c;
#pragma unroll
    for (int m = 1; m < WAVE; m <<= 1) {
      int o = __shfl_up(incl, m, WAVE);
      if (lane >= m) incl += o;
    }
    int pos = base + incl - c;
    while (bits) {
      const int bit = __ffs(bits) - 1;
      bits &= bits - 1;
      const int t = w * 32 + bit;
      sorted_token[pos] = t;
      const int32_t* ti = topk_idx + (size_t)t * K;
      for (int k = 0; k < K; ++k)
        if (ti[k] == e) inv_perm[(size_t)t * K + k] = pos;
      ++pos;
    }
    base += __shfl(incl, WAVE - 1, WAVE);
  }
}

}  // namespace

size_t dispatch_bitmap_words(int64_t T, int E) { return (size_t)E * (size_t)((T + 31) / 32); }

hipError_t launch_dispatch(const int32_t* topk_idx, int T, int K, int E, int S, uint32_t* bitmap, int32_t* counts,
                           int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm, hipStream_t s, Tracer* tr) {
  const int words = (T + 31) / 32;
  const size_t nbits = (size_t)E * words;
  int zb = (int)std::min<size_t>((nbits + 255) / 256, 1024);
  hipLaunchKernelGGL(fill_u32_kernel, dim3(zb), dim3(256), 0, s, bitmap, nbits, 0u);
  if (tr) tr->mark("dispatch_clear", s);
  const int64_t pairs = (int64_t)T * K;
  hipLaunchKernelGGL(dispatch_mark_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), 0, s, topk_idx, T, K, E,
                     words, bitmap, inv_perm);
  if (tr) tr->mark("dispatch_mark", s);
  const int eb = (E + 1 + 3) / 4;
  hipLaunchKernelGGL(dispatch_count_kernel, dim3(eb), dim3(256), 0, s, bitmap, E, words, T, S, counts);
  if (tr) tr->mark("dispatch_count", s);
  hipLaunchKernelGGL(exclusive_scan_kernel, dim3(1), dim3(64), 0, s, counts, E + 1, offsets);
  if (tr) tr->mark("dispatch_scan", s);
  hipLaunchKernelGGL(dispatch_scatter_kernel, dim3(eb), dim3(256), 0, s, bitmap, offsets, topk_idx, T, K, E, words, S,
                     sorted_token, inv_perm);
  if (tr) tr->mark("dispatch_scatter", s);
  return hipGetLastError();
}

}  // namespace moe
