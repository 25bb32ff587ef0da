// Dispatch: group the (token, slot) pairs chosen by the router by expert, so the expert
// FFNs can run as a grouped GEMM over contiguous row blocks (the routing walk-through page,
// lqnn.cn, section 三.2, ends with 8 experts per token; each expert then serves its tokens).
//
// Deterministic and independent of the order of atomics:
//   1. mark     one bit per (expert, token) in a bitmap [E][ceil(T/32)] (atomicOr on
//               integers: the final bits do not depend on the order).  moe_dispatch marks
//               here and counts with atomicAdd; the fused forward marks inside the router's
//               top-k kernel (after its logits kernel cleared the bitmap), and the histogram
//               is then the popcount of each bitmap row (dispatch_count_kernel).  Up to 256
//               tokens the fused forward does all of the dispatch in the top-k kernel's last
//               workgroup (router.hip) instead.
//   2. finish   one wave per (expert, 2048-token chunk of its row): the chunk's first
//               position is the sum of the counts before the expert plus the row's earlier
//               bits; it walks the set bits in ascending token order and writes sorted_token
//               and inv_perm.  One more wave writes the offsets, the counts with the shared
//               expert's entry, the shared expert's identity block and, for the fused
//               forward, the expert FFN's tile prefix and tile records.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

__global__ void fill_u32_kernel(uint32_t* __restrict__ p, size_t n, uint32_t v) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x) p[i] = v;
}

__global__ void dispatch_mark_kernel(const int32_t* __restrict__ topk_idx, int T, int K, int E, int words,
                                     uint32_t* __restrict__ bitmap, int32_t* __restrict__ counts,
                                     int32_t* __restrict__ inv_perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)T * K) return;
  const int e = topk_idx[i];
  const int t = (int)(i / K);
  if (e >= 0 && e < E) {
    atomicOr(&bitmap[(size_t)e * words + (t >> 5)], 1u << (t & 31));
    atomicAdd(&counts[e], 1);
  } else {
    inv_perm[i] = -1;  // ignored pair
  }
}

// dense FFN as a one-expert layer: every token is routed to expert 0 in slot 0 with weight 1
__global__ __launch_bounds__(256) void dense_dispatch_kernel(int T, int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_token,
                                                             int32_t* __restrict__ inv_perm, float* __restrict__ topk_w) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    offsets[0] = 0;
    offsets[1] = T;
    offsets[2] = T;
  }
  if (i < T) {
    sorted_token[i] = i;
    inv_perm[i] = i;
    topk_w[i] = 1.0f;
  }
}

// marked bitmap (no expert twice for a token): counts[e] = set bits of row e, one wave per row
__global__ __launch_bounds__(256) void dispatch_count_kernel(const uint32_t* __restrict__ bitmap, int words, int E,
                                                             int32_t* __restrict__ counts) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const uint32_t* row = bitmap + (size_t)e * words;
  int c = 0;
  for (int w = lane; w < words; w += WAVE) c += __popc(row[w]);
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, WAVE);
  if (lane == 0) counts[e] = c;
}

// sum of v[0 .. n) over one wave (lane-strided)
__device__ __forceinline__ int wave_sum_prefix(const int32_t* __restrict__ v, int n, int lane) {
  int c = 0;
  for (int i = lane; i < n; i += WAVE) c += v[i];
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, WAVE);
  return c;
}

// Waves 0 .. E*nchunks-1: expert e = wave / nchunks, chunk c = wave % nchunks of 64 bitmap
// words (2048 tokens) of its row; the chunk's first position is the sum of the counts of
// the experts before e plus the bits of the row's earlier chunks.  Wave E*nchunks: offsets,
// counts_out (a copy of the histogram plus the shared expert's T*S), the shared expert's
// identity block and (if tile_prefix) the tile prefix of the E + S experts for tiles of bm
// positions.
__global__ __launch_bounds__(256) void dispatch_finish_kernel(const uint32_t* __restrict__ bitmap,
                                                              const int32_t* __restrict__ counts,
                                                              int32_t* __restrict__ counts_out,
                                                              const int32_t* __restrict__ topk_idx, int T, int K,
                                                              int E, int words, int S,
                                                              int32_t* __restrict__ offsets,
                                                              int32_t* __restrict__ sorted_token,
                                                              int32_t* __restrict__ inv_perm,
                                                              int32_t* __restrict__ tile_prefix, int bm) {
  const int lane = threadIdx.x & 63;
  const int nchunks = (words + WAVE - 1) / WAVE;
  const int wv = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wv > E * nchunks) return;
  if (wv == E * nchunks) {
    // exclusive scan of counts[0..E) plus the shared expert
    const int per = (E + WAVE - 1) / WAVE;
    const int b = lane * per, en = min(E, b + per);
    int sum = 0, tsum = 0;
    for (int i = b; i < en; ++i) {
      sum += counts[i];
      if (tile_prefix) tsum += (counts[i] + bm - 1) / bm;
    }
    int incl = sum, tincl = tsum;
#pragma unroll
    for (int m = 1; m < WAVE; m <<= 1) {
      int o = __shfl_up(incl, m, WAVE), to = __shfl_up(tincl, m, WAVE);
      if (lane >= m) {
        incl += o;
        tincl += to;
      }
    }
    int run = incl - sum, trun = tincl - tsum;
    int4* info = tile_prefix ? (int4*)(tile_prefix + tile_info_offset(E)) : nullptr;
    for (int i = b; i < en; ++i) {
      const int c = counts[i];
      offsets[i] = run;
      counts_out[i] = c;
      if (tile_prefix) {
        tile_prefix[i] = trun;
        for (int j = 0; j * bm < c; ++j) info[trun + j] = int4{i, run + j * bm, min(bm, c - j * bm), 0};
        trun += (c + bm - 1) / bm;
      }
      run += c;
    }
    // the shared expert's block starts at T*K even when pairs were ignored (out-of-range
    // ids): positions routed .. T*K-1 then hold no token
    const int routed = __shfl(incl, WAVE - 1, WAVE);
    const int trouted = __shfl(tincl, WAVE - 1, WAVE);
    const int sh0 = T * K;
    if (lane == 0) {
      counts_out[E] = T * S;
      offsets[E] = sh0;
      offsets[E + 1] = sh0 + T * S;
      if (tile_prefix) {
        tile_prefix[E] = trouted;
        tile_prefix[E + 1] = trouted + (S ? (T + bm - 1) / bm : 0);
      }
    }
    if (tile_prefix && S)  // the shared expert's tiles: all T tokens in order
      for (int j = lane; j * bm < T; j += WAVE) info[trouted + j] = int4{E, sh0 + j * bm, min(bm, T - j * bm), 0};
    for (int p = routed + lane; p < sh0; p += WAVE) sorted_token[p] = -1;
    if (S)
      for (int t = lane; t < T; t += WAVE) sorted_token[sh0 + t] = t;
    return;
  }
  const int e = wv / nchunks, chunk = wv - e * nchunks;
  const uint32_t* row = bitmap + (size_t)e * words;
  const int w0 = chunk * WAVE;
  // start of this chunk: experts before e, then the row's earlier words
  int base = wave_sum_prefix(counts, e, lane);
  {
    int c = 0;
    for (int w = lane; w < w0; w += WAVE) c += __popc(row[w]);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) c += __shfl_xor(c, m, WAVE);
    base += c;
  }
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
  // the set bits in token order, 4 tokens at a time: their slot rows (8 slots per batch,
  // clamped loads) go out in one batch, and every slot that lists e gets the position
  constexpr int TB = 4, KB = 8;
  while (bits) {
    int tt[TB];
#pragma unroll
    for (int i = 0; i < TB; ++i) {
      tt[i] = -1;
      if (bits) {
        tt[i] = w * 32 + __ffs(bits) - 1;
        bits &= bits - 1;
      }
    }
#pragma unroll
    for (int i = 0; i < TB; ++i)
      if (tt[i] >= 0) sorted_token[pos + i] = tt[i];
    for (int k0 = 0; k0 < K; k0 += KB) {
      int v[TB][KB];
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int u = 0; u < KB; ++u) v[i][u] = topk_idx[(size_t)(tt[i] >= 0 ? tt[i] : tt[0]) * K + min(k0 + u, K - 1)];
#pragma unroll
      for (int i = 0; i < TB; ++i)
#pragma unroll
        for (int u = 0; u < KB; ++u)
          if (tt[i] >= 0 && k0 + u < K && v[i][u] == e) inv_perm[(size_t)tt[i] * K + k0 + u] = pos + i;
    }
    pos += TB;
  }
  if (chunk == nchunks - 1) {
    // a token listing the same expert twice is counted twice but has one bit: mark the
    // positions that no token fills (the expert FFN skips negative tokens)
    const int filled = base + __shfl(incl, WAVE - 1, WAVE);
    const int end = wave_sum_prefix(counts, e, lane) + counts[e];
    for (int p = filled + lane; p < end; p += WAVE) sorted_token[p] = -1;
  }
}

}  // namespace

size_t dispatch_bitmap_words(int64_t T, int E) { return (size_t)E * (size_t)((T + 31) / 32); }


hipError_t launch_dense_dispatch(int T, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm, float* topk_w,
                                 hipStream_t s) {
  if (T <= 0) return hipErrorInvalidValue;
  hipLaunchKernelGGL(dense_dispatch_kernel, dim3((T + 255) / 256), dim3(256), 0, s, T, offsets, sorted_token, inv_perm,
                     topk_w);
  return hipGetLastError();
}

hipError_t launch_dispatch(const int32_t* topk_idx, int T, int K, int E, int S, uint32_t* bitmap, int32_t* counts,
                           int32_t* counts_out, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm, bool marked,
                           int32_t* tile_prefix, int bm, hipStream_t s, Tracer* tr) {
  const int words = (T + 31) / 32;
  if (!marked) {
    const size_t nbits = (size_t)E * words;
    int zb = (int)std::min<size_t>((nbits + 255) / 256, 1024);
    launch(tr, fill_u32_kernel, dim3(zb), dim3(256), s, bitmap, nbits, 0u);
    launch(tr, fill_u32_kernel, dim3(1), dim3(256), s, (uint32_t*)counts, (size_t)E, 0u);
    if (tr) tr->mark("dispatch_clear", s);
    const int64_t pairs = (int64_t)T * K;
    launch(tr, dispatch_mark_kernel, dim3((unsigned)((pairs + 255) / 256)), dim3(256), s, topk_idx, T, K, E,
           words, bitmap, counts, inv_perm);
    if (tr) tr->mark("dispatch_mark", s);
  } else {
    launch(tr, dispatch_count_kernel, dim3((E + 3) / 4), dim3(256), s, (const uint32_t*)bitmap, words, E, counts);
    if (tr) tr->mark("dispatch_count", s);
  }
  const int nchunks = (words + WAVE - 1) / WAVE;
  const int eb = (E * nchunks + 1 + 3) / 4;
  launch(tr, dispatch_finish_kernel, dim3(eb), dim3(256), s, bitmap, counts, counts_out, topk_idx, T, K, E, words,
         S, offsets, sorted_token, inv_perm, tile_prefix, bm);
  if (tr) tr->mark("dispatch_finish", s);
  return hipGetLastError();
}

}  // namespace moe
