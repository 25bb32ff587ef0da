// Router of the BailingMoeV3 sparse MoE block.
//
// Ling-3.0-flash-VL routing walk-through page (lqnn.cn), section 三.1: one raw score per
// routed expert from the hidden state, then an element-wise sigmoid; section 三.3: a
// per-expert bias is added for selection; section 三.2: keep the topk_group groups with the
// largest in-group maximum and pick the top-k experts inside them; section 四: the router
// runs in fp32, the chosen scores are renormalised and scaled by routed_scaling_factor.
//
// Kernels:
//   router_logits_kernel  fp32-accurate logits on bf16 MFMA.  x is bf16, so splitting each
//                         fp32 router weight exactly into three bf16 pieces (hi + mid + lo,
//                         8 significand bits each) makes every product x * piece exact in
//                         fp32; three 16x16x32 bf16 MFMAs with fp32 accumulation then give
//                         fp32-GEMM logits at a fraction of the cost of fp32 MFMA (the
//                         split-precision idea of Markidis et al. 2018 / Ootomo & Yokota
//                         2022).  The hidden dimension may be split across workgroups for
//                         small token counts; partial sums are added later in a fixed order.
//   router_logits_kwaves_kernel  the same logits for up to 256 tokens: 16-expert workgroups
//                         whose four waves split their slice of the hidden dimension.
//   router_topk_kernel    one wave per token: sigmoid, bias, group max, group ranking and the
//                         top-k selection entirely in registers with wave shuffles; for up to
//                         256 tokens the last workgroup to finish also builds the dispatch.
//   expert_bias_update_kernel  the sign-rule bias step from a step's expert counts.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

__device__ __forceinline__ void split3(float w0, float w1, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  // exact split by truncation: w = hi + mid + lo, each a bf16
  uint32_t u0 = __float_as_uint(w0), u1 = __float_as_uint(w1);
  uint32_t h0 = u0 & 0xFFFF0000u, h1 = u1 & 0xFFFF0000u;
  float r0 = w0 - __uint_as_float(h0), r1 = w1 - __uint_as_float(h1);
  uint32_t m0 = __float_as_uint(r0) & 0xFFFF0000u, m1 = __float_as_uint(r1) & 0xFFFF0000u;
  float s0 = r0 - __uint_as_float(m0), s1 = r1 - __uint_as_float(m1);
  uint32_t l0 = __float_as_uint(s0) & 0xFFFF0000u, l1 = __float_as_uint(s1) & 0xFFFF0000u;
  hi = (h0 >> 16) | h1;
  mid = (m0 >> 16) | m1;
  lo = (l0 >> 16) | l1;
}

// partial[split][t][e] = sum over the split's slice of h of x[t][h] * W[e][h].
// Workgroup: 4 waves; wave w owns RF 16-row blocks of experts (the MFMA a operands),
// tokens m0 .. m0 + 16*MF - 1 are the b operands.  Lane (r, q) of a 16x32 operand holds
// row r, k = kb + 8q .. kb + 8q + 7.
template <int MF, int RF>
__global__ __launch_bounds__(256) void router_logits_kernel(const uint16_t* __restrict__ x,
                                                            const float* __restrict__ w, int T, int H,
                                                            int E, int kchunk, float* __restrict__ partial,
                                                            uint32_t* __restrict__ clear, int64_t clear_words) {
  constexpr int WG_EXPERTS = 4 * RF * 16;
  // zero the dispatch bitmap and counters that the top-k kernel fills (used by the fused
  // forward; independent of the logits)
  if (clear) {
    const int64_t nth = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < clear_words;
         i += nth)
      clear[i] = 0u;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int n_tiles = E / WG_EXPERTS;
  const int nt = blockIdx.x % n_tiles, split = blockIdx.x / n_tiles;
  const int m0 = blockIdx.y * 16 * MF;
  const int e_base = nt * WG_EXPERTS + wave * RF * 16;
  const int k0 = split * kchunk;

  const float* wr[RF];
#pragma unroll
  for (int f = 0; f < RF; ++f) wr[f] = w + (size_t)(e_base + f * 16 + r16) * H + k0 + q * 8;
  floatx4 acc[RF][MF];
#pragma unroll
  for (int f = 0; f < RF; ++f)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) acc[f][mf] = floatx4{0.f, 0.f, 0.f, 0.f};

  // The workgroup's token tile (16*MF rows x 32 k per step) is loaded once, by all threads, and
  // shared through LDS (each wave used to load all of it itself: two thirds of the loads);
  // weights go straight to registers.  Loads run D steps ahead in a register ring, issued
  // unconditionally (steps past the end reload the last one) so the waits stay exact.
  constexpr int BMX = 16 * MF, LX = 40;  // 80-byte LDS rows: 8 consecutive rows hit distinct banks
  constexpr int XCH = BMX * 4;           // 16-byte pieces of the tile per step
  constexpr int XPT = (XCH + 255) / 256;
  constexpr int D = 3;
  __shared__ __align__(16) uint16_t xs[2][BMX * LX];
  const int nsteps = kchunk / 32;
  const uint16_t* xsrc[XPT];
  int xdst[XPT];
#pragma unroll
  for (int i = 0; i < XPT; ++i) {
    const int c = threadIdx.x + i * 256;
    const int row = c < XCH ? c >> 2 : 0, col = (c & 3) * 8;
    xsrc[i] = x + (size_t)min(m0 + row, T - 1) * H + k0 + col;
    xdst[i] = c < XCH ? row * LX + col : -1;
  }
  struct Stage {
    u32x4 xv[XPT];
    float4 a[RF][2];
  };
  auto load = [&](Stage& st, int step) {
    const int kk = min(step, nsteps - 1) * 32;
#pragma unroll
    for (int i = 0; i < XPT; ++i) st.xv[i] = *(const u32x4*)(xsrc[i] + kk);
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      st.a[f][0] = *(const float4*)(wr[f] + kk);
      st.a[f][1] = *(const float4*)(wr[f] + kk + 4);
    }
  };
  auto store_x = [&](const Stage& st, int buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i)
      if (xdst[i] >= 0) *(u32x4*)(xs[buf] + xdst[i]) = st.xv[i];
  };
  auto compute = [&](const Stage& st, int buf) {
    u32x4 hi[RF], mid[RF], lo[RF];
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      const float v[8] = {st.a[f][0].x, st.a[f][0].y, st.a[f][0].z, st.a[f][0].w,
                          st.a[f][1].x, st.a[f][1].y, st.a[f][1].z, st.a[f][1].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        uint32_t h, m, l;
        split3(v[2 * i], v[2 * i + 1], h, m, l);
        hi[f][i] = h;
        mid[f][i] = m;
        lo[f][i] = l;
      }
    }
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const u32x4 xv = *(const u32x4*)(xs[buf] + (mf * 16 + r16) * LX + q * 8);
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        acc[f][mf] = mfma16(lo[f], xv, acc[f][mf]);
        acc[f][mf] = mfma16(mid[f], xv, acc[f][mf]);
        acc[f][mf] = mfma16(hi[f], xv, acc[f][mf]);
      }
    }
  };
  Stage ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) load(ring[j], j);
  store_x(ring[0], 0);
  __syncthreads();
  for (int s0 = 0; s0 < nsteps; s0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int st = s0 + j;
      if (st < nsteps) {
        compute(ring[j], st & 1);
        store_x(ring[(j + 1) % D], (st + 1) & 1);
      }
      load(ring[j], st + D);
      __syncthreads();
    }
  }
  // result: lane holds token r16 of each fragment, experts 4q .. 4q+3 of each 16-row block
  float* out = partial + (size_t)split * T * E;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    int t = m0 + mf * 16 + r16;
    if (t < T) {
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        float4 v = {acc[f][mf][0], acc[f][mf][1], acc[f][mf][2], acc[f][mf][3]};
        *(float4*)(out + (size_t)t * E + e_base + f * 16 + 4 * q) = v;
      }
    }
  }
}

// Few tokens: the same partial sums from more, shorter workgroups.  A workgroup owns 16
// experts, tokens m0 .. m0 + 16*MF - 1 and one split of h; its 4 waves take consecutive
// quarters of the split, issue all their loads at once (two 32-wide k steps per round), and
// their sums are added through LDS in wave order.  Needs kchunk % 128 == 0.
template <int MF>
__global__ __launch_bounds__(256) void router_logits_kwaves_kernel(const uint16_t* __restrict__ x,
                                                                   const float* __restrict__ w, int T, int H,
                                                                   int E, int kchunk, float* __restrict__ partial,
                                                                   uint32_t* __restrict__ clear,
                                                                   int64_t clear_words) {
  __shared__ floatx4 red[4][MF][64];
  if (clear) {
    const int64_t nth = (int64_t)gridDim.x * gridDim.y * blockDim.x;
    for (int64_t i = ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * blockDim.x + threadIdx.x; i < clear_words;
         i += nth)
      clear[i] = 0u;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int n_tiles = E / 16;
  const int nt = blockIdx.x % n_tiles, split = blockIdx.x / n_tiles;
  const int m0 = blockIdx.y * 16 * MF;
  const int e_base = nt * 16;
  const int kw = kchunk / 4;  // this wave's k range
  const int k0 = split * kchunk + wave * kw;

  const float* wr = w + (size_t)(e_base + r16) * H + k0 + q * 8;
  const uint16_t* xr[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int t = min(m0 + mf * 16 + r16, T - 1);
    xr[mf] = x + (size_t)t * H + k0 + q * 8;
  }
  floatx4 acc[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) acc[mf] = floatx4{0.f, 0.f, 0.f, 0.f};

  auto step = [&](const float4 (&a)[2], const u32x4 (&xv)[MF]) {
    const float v[8] = {a[0].x, a[0].y, a[0].z, a[0].w, a[1].x, a[1].y, a[1].z, a[1].w};
    u32x4 hi, mid, lo;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t h, m, l;
      split3(v[2 * i], v[2 * i + 1], h, m, l);
      hi[i] = h;
      mid[i] = m;
      lo[i] = l;
    }
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      acc[mf] = mfma16(lo, xv[mf], acc[mf]);
      acc[mf] = mfma16(mid, xv[mf], acc[mf]);
      acc[mf] = mfma16(hi, xv[mf], acc[mf]);
    }
  };
  for (int kk = 0; kk + 64 <= kw; kk += 64) {
    float4 a[2][2];
    u32x4 xv[2][MF];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      a[u][0] = *(const float4*)(wr + kk + 32 * u);
      a[u][1] = *(const float4*)(wr + kk + 32 * u + 4);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) xv[u][mf] = *(const u32x4*)(xr[mf] + kk + 32 * u);
    }
    step(a[0], xv[0]);
    step(a[1], xv[1]);
  }
  if (kw % 64) {  // one 32-wide step left
    const int kk = kw - 32;
    float4 a[2];
    u32x4 xv[MF];
    a[0] = *(const float4*)(wr + kk);
    a[1] = *(const float4*)(wr + kk + 4);
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) xv[mf] = *(const u32x4*)(xr[mf] + kk);
    step(a, xv);
  }
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) red[wave][mf][lane] = acc[mf];
  __syncthreads();
  // lane holds token r16 of each fragment, experts 4q .. 4q+3; fragment mf is summed (waves
  // 0, 1, 2, 3 in order) and stored by wave mf % 4
  float* out = partial + (size_t)split * T * E;
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    if (mf % 4 != wave) continue;
    const int t = m0 + mf * 16 + r16;
    if (t < T) {
      const floatx4 s = ((red[0][mf][lane] + red[1][mf][lane]) + red[2][mf][lane]) + red[3][mf][lane];
      *(float4*)(out + (size_t)t * E + e_base + 4 * q) = float4{s[0], s[1], s[2], s[3]};
    }
  }
}

// One token (one wave): the top-k of the routing walk-through page's sections 三.1-三.3.
// Cross-lane steps of the selection without an LDS round trip.  Inside rows of 16 lanes, DPP
// moves: quad_perm [1,0,3,2] and [2,3,0,1] (lane ^ 1, lane ^ 2), row_half_mirror (lane i of 8
// <-> 7 - i) and row_mirror (lane i of 16 <-> 15 - i); after these four steps of a maximum
// (exact, so the pairing order does not matter) every lane holds its row's maximum, and the
// four rows are combined from wave-uniform lane reads.
constexpr int DPP_XOR1 = 0xB1, DPP_XOR2 = 0x4E, DPP_ROW_HALF_MIRROR = 0x141, DPP_ROW_MIRROR = 0x140;

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {
  return ((uint64_t)dpp_u32<CTRL>((uint32_t)(v >> 32)) << 32) | dpp_u32<CTRL>((uint32_t)v);
}
__device__ __forceinline__ uint32_t readlane_u32(uint32_t v, int l) {
  return (uint32_t)__builtin_amdgcn_readlane((int)v, l);
}
__device__ __forceinline__ uint64_t readlane_u64(uint64_t v, int l) {
  return ((uint64_t)readlane_u32((uint32_t)(v >> 32), l) << 32) | readlane_u32((uint32_t)v, l);
}
__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

// maximum over the wave, the same in every lane
__device__ __forceinline__ uint64_t wave_max_u64_dpp(uint64_t v) {
  v = max_u64(v, dpp_u64<DPP_XOR1>(v));
  v = max_u64(v, dpp_u64<DPP_XOR2>(v));
  v = max_u64(v, dpp_u64<DPP_ROW_HALF_MIRROR>(v));
  v = max_u64(v, dpp_u64<DPP_ROW_MIRROR>(v));
  return max_u64(max_u64(readlane_u64(v, 0), readlane_u64(v, 16)), max_u64(readlane_u64(v, 32), readlane_u64(v, 48)));
}

// maximum over aligned groups of lpg consecutive lanes (a power of two), in every lane
__device__ __forceinline__ float group_max_f32(float v, int lpg) {
  if (lpg >= 2) v = fmaxf(v, __uint_as_float(dpp_u32<DPP_XOR1>(__float_as_uint(v))));
  if (lpg >= 4) v = fmaxf(v, __uint_as_float(dpp_u32<DPP_XOR2>(__float_as_uint(v))));
  if (lpg >= 8) v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_HALF_MIRROR>(__float_as_uint(v))));
  if (lpg >= 16) v = fmaxf(v, __uint_as_float(dpp_u32<DPP_ROW_MIRROR>(__float_as_uint(v))));
  for (int m = 16; m < lpg; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, WAVE));
  return v;
}

template <int EPL>
__device__ __forceinline__ void route_token(const float* __restrict__ partial, int nsplit, int T, int E,
                                            const float* __restrict__ bias, int G, int TG, int K, int norm,
                                            float scale, int32_t* __restrict__ topk_idx, float* __restrict__ topk_w,
                                            uint32_t* __restrict__ bitmap, int words, int t, int lane) {
  const int e0 = lane * EPL;

  // logits: split partial sums added in split order
  float l[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) l[i] = 0.f;
#pragma unroll 4
  for (int p = 0; p < nsplit; ++p) {
    const float* src = partial + ((size_t)p * T + t) * E + e0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) l[i] += src[i];
  }

  // sigmoid score s and biased choice score c
  float s[EPL], c[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i) {
    s[i] = 1.0f / (1.0f + expf(-l[i]));
    float b = bias ? bias[e0 + i] : 0.0f;
    c[i] = (s[i] + b) + 0.0f;  // + 0 turns a -0 into +0 so equal scores compare as ties
  }

  // group score: maximum biased score inside the group
  const int lpg = WAVE / G;
  float gm = c[0];
#pragma unroll
  for (int i = 1; i < EPL; ++i) gm = fmaxf(gm, c[i]);
  gm = group_max_f32(gm, lpg);

  // rank of this lane's group among all groups (ties: lower group index first)
  const int g = lane / lpg;
  int rank = 0;
  for (int h = 0; h < G; ++h) {
    const float o = __uint_as_float(readlane_u32(__float_as_uint(gm), h * lpg));
    rank += (o > gm) || (o == gm && h < g);
  }
  const bool kept = rank < TG;

  // selection keys: ordered score in the high word, reversed index in the low word, so
  // the maximum key is the best score and, among equal scores, the lowest index.
  // Experts of dropped groups get key 0 and can never be chosen.
  uint64_t key[EPL];
#pragma unroll
  for (int i = 0; i < EPL; ++i)
    key[i] = kept ? (((uint64_t)f32_ordered(c[i]) << 32) | (uint32_t)(0xFFFFFFFFu - (uint32_t)(e0 + i))) : 0ull;

  int my_idx = 0;
  float my_s = 0.f;
  for (int r = 0; r < K; ++r) {
    uint64_t best = key[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) best = key[i] > best ? key[i] : best;
    best = wave_max_u64_dpp(best);
    const int idx = (int)(0xFFFFFFFFu - (uint32_t)best);
    const int owner = idx / EPL, slot = idx - owner * EPL;
    float sv = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
      if (i == slot) {
        sv = s[i];
        if (lane == owner) key[i] = 0ull;
      }
    }
    sv = __uint_as_float(readlane_u32(__float_as_uint(sv), owner));
    if (lane == r) {
      my_idx = idx;
      my_s = sv;
    }
  }

  // renormalise (unbiased scores) and scale; write in ascending expert order
  const float sum = wave_sum_f32(lane < K ? my_s : 0.f);
  int pos = 0;
  for (int j = 0; j < K; ++j) pos += (int)readlane_u32((uint32_t)my_idx, j) < my_idx;
  if (lane < K) {
    const float wv = norm ? (my_s / sum) * scale : my_s * scale;
    topk_idx[(size_t)t * K + pos] = my_idx;
    topk_w[(size_t)t * K + pos] = wv;
    if (bitmap) {
      // dispatch: one bit per (expert, token) (an integer atomic, so the final bitmap does
      // not depend on the order).  The histogram is the popcount of the bitmap rows, taken
      // later: one atomic per pair on 512 counters serialised on the hot ones (30 us of this
      // kernel at 8192 tokens, 100 us on skewed routing).
      atomicOr(&bitmap[(size_t)my_idx * words + (t >> 5)], 1u << (t & 31));
    }
  }
}

// The dispatch of the fused forward for few tokens, run by the last top-k workgroup to finish
// (the one that brings `done` to the grid size): the same results as the dispatch kernels'
// finish step.  Every workgroup first makes its top-k stores visible (release fence before
// the counter); the last one reads all of topk_idx once after an acquire fence, through
// loads that bypass the non-coherent L1, and builds the bitmap and the histogram in LDS.
__device__ __forceinline__ int load_acq(const int32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

constexpr int FD_WORDS = FUSED_DISPATCH_MAX_T / 32;                // bitmap words per expert
constexpr int FD_PER_THREAD = FUSED_DISPATCH_MAX_PAIRS / 256;      // (token, slot) pairs per thread

__device__ __forceinline__ void fused_dispatch_finish(const FusedDispatch& fd, const int32_t* topk_idx, int T,
                                                   int K, int E) {
  __shared__ int last;
  __shared__ int offs[FUSED_DISPATCH_MAX_E + 1];
  __shared__ int cnt[FUSED_DISPATCH_MAX_E];
  __shared__ uint32_t bits[FUSED_DISPATCH_MAX_E * FD_WORDS];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) last = atomicAdd(fd.done, 1) == (int)gridDim.x - 1;
  __syncthreads();
  if (!last) return;
  __threadfence();
  const int tid = threadIdx.x, TK = T * K;
  int ev[FD_PER_THREAD];
#pragma unroll
  for (int u = 0; u < FD_PER_THREAD; ++u) {
    const int p = tid + u * 256;
    ev[u] = p < TK ? load_acq(topk_idx + p) : -1;
  }
  for (int i = tid; i < E; i += 256) cnt[i] = 0;
  for (int i = tid; i < E * FD_WORDS; i += 256) bits[i] = 0u;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < FD_PER_THREAD; ++u) {
    const int p = tid + u * 256, e = ev[u];
    if (p < TK && e >= 0 && e < E) {
      const int t = p / K;
      atomicOr(&bits[e * FD_WORDS + (t >> 5)], 1u << (t & 31));
      atomicAdd(&cnt[e], 1);
    }
  }
  __syncthreads();
  const int lane = tid & 63;
  if (tid < 64) {
    // exclusive scans of the expert counts and of their FFN tiles
    const int per = (E + 63) / 64;
    const int b = lane * per, en = min(E, b + per);
    int sum = 0, tsum = 0;
    for (int i = b; i < en; ++i) {
      const int c = cnt[i];
      sum += c;
      tsum += (c + fd.bm - 1) / fd.bm;
    }
    int incl = sum, tincl = tsum;
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const int o = __shfl_up(incl, m, 64), to = __shfl_up(tincl, m, 64);
      if (lane >= m) {
        incl += o;
        tincl += to;
      }
    }
    int run = incl - sum, trun = tincl - tsum;
    int4* info = fd.tile_prefix ? (int4*)(fd.tile_prefix + tile_info_offset(E)) : nullptr;
    for (int i = b; i < en; ++i) {
      const int c = cnt[i];
      offs[i] = run;
      fd.offsets[i] = run;
      fd.counts_out[i] = c;
      if (fd.tile_prefix) {
        fd.tile_prefix[i] = trun;
        for (int j = 0; j * fd.bm < c; ++j) info[trun + j] = int4{i, run + j * fd.bm, min(fd.bm, c - j * fd.bm), 0};
      }
      run += c;
      trun += (c + fd.bm - 1) / fd.bm;
    }
    // the shared expert's block starts at T*K even when pairs were ignored (out-of-range
    // ids): positions routed .. T*K-1 then hold no token
    const int routed = __shfl(incl, 63, 64), trouted = __shfl(tincl, 63, 64);
    const int sh0 = T * K;
    if (lane == 0) {
      offs[E] = sh0;
      fd.counts_out[E] = T * fd.S;
      fd.offsets[E] = sh0;
      fd.offsets[E + 1] = sh0 + T * fd.S;
      if (fd.tile_prefix) {
        fd.tile_prefix[E] = trouted;
        fd.tile_prefix[E + 1] = trouted + (fd.S ? (T + fd.bm - 1) / fd.bm : 0);
      }
    }
    if (fd.tile_prefix && fd.S)  // the shared expert's tiles: all T tokens in order
      for (int j = lane; j * fd.bm < T; j += 64)
        info[trouted + j] = int4{E, sh0 + j * fd.bm, min(fd.bm, T - j * fd.bm), 0};
    for (int p = routed + lane; p < sh0; p += 64) fd.sorted_token[p] = -1;
  }
  __syncthreads();
  // each (token, slot): its position is the expert's offset plus the number of the expert's
  // tokens before it (set bits of the expert's bitmap row below the token)
#pragma unroll
  for (int u = 0; u < FD_PER_THREAD; ++u) {
    const int p = tid + u * 256, e = ev[u];
    if (p >= TK) continue;
    if (e < 0 || e >= E) {
      fd.inv_perm[p] = -1;
      continue;
    }
    const int t = p / K;
    const uint32_t* row = bits + e * FD_WORDS;
    int rank = __popc(row[t >> 5] & ((1u << (t & 31)) - 1u));
    for (int w = 0; w < (t >> 5); ++w) rank += __popc(row[w]);
    const int pos = offs[e] + rank;
    fd.sorted_token[pos] = t;
    fd.inv_perm[p] = pos;
  }
  if (fd.S)
    for (int t = tid; t < T; t += 256) fd.sorted_token[offs[E] + t] = t;
}

// One wave per token.  Lane l holds experts l*EPL .. l*EPL + EPL - 1, so a group of E/G
// experts is 64/G consecutive lanes.
template <int EPL, bool FUSED>
__global__ __launch_bounds__(256) void router_topk_kernel(const float* __restrict__ partial, int nsplit,
                                                          int T, int E, const float* __restrict__ bias, int G,
                                                          int TG, int K, int norm, float scale,
                                                          int32_t* __restrict__ topk_idx,
                                                          float* __restrict__ topk_w,
                                                          uint32_t* __restrict__ bitmap, int words,
                                                          FusedDispatch fd) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  // the fused dispatch builds its bitmap and histogram from topk_idx itself
  if (t < T) route_token<EPL>(partial, nsplit, T, E, bias, G, TG, K, norm, scale, topk_idx, topk_w,
                              FUSED ? nullptr : bitmap, words, t, lane);
  if constexpr (FUSED) fused_dispatch_finish(fd, topk_idx, T, K, E);
}


int pick_router_mf(int64_t T) { return T <= 16 ? 1 : T <= 32 ? 2 : T <= 64 ? 4 : 8; }

// Expert-bias update (routing walk-through page, section 三.3: the selection bias of a busy
// expert is lowered and that of an idle one raised, with no auxiliary loss; the page gives no
// rule or rate, the sign rule is taken): one workgroup; the total count is summed in 64 bits
// and each expert compares count * E with it, so the decision involves no rounding.
__global__ __launch_bounds__(1024) void expert_bias_update_kernel(const int32_t* __restrict__ counts, int E,
                                                                  float gamma, float* __restrict__ bias) {
  __shared__ long long wsum[16];
  const int e = threadIdx.x, lane = e & 63, wave = e >> 6;
  const long long c = e < E ? (long long)counts[e] : 0;
  long long v = c;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, WAVE);
  if (lane == 0) wsum[wave] = v;
  __syncthreads();
  long long total = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) total += wsum[w];
  if (e < E) {
    const long long d = total - (long long)E * c;  // > 0: below the mean
    const float side = d > 0 ? 1.0f : d < 0 ? -1.0f : 0.0f;
    bias[e] = bias[e] + gamma * side;
  }
}

}  // namespace

hipError_t launch_expert_bias_update(const int32_t* counts, int E, float gamma, float* bias, hipStream_t s) {
  if (E <= 0 || E > 1024) return hipErrorInvalidValue;
  hipLaunchKernelGGL(expert_bias_update_kernel, dim3(1), dim3((E + 63) / 64 * 64), 0, s, counts, E, gamma, bias);
  return hipGetLastError();
}

RouterPlan router_plan(int64_t T, int H, int E) {
  RouterPlan p;
  p.mf = pick_router_mf(T);
  p.m_tiles = (int)((T + 16 * p.mf - 1) / (16 * p.mf));
  // 128 experts per workgroup (x re-read E/128 times) once that still gives ~512 workgroups,
  // else 64 (measured: 512 workgroups of 64 experts at T = 8192, 512 of 128 at T = 16384)
  p.rf = (E % 128 == 0 && (int64_t)p.m_tiles * (E / 128) >= 512) ? 2 : 1;
  p.n_tiles = E / (64 * p.rf);
  // split the hidden dimension while there are fewer than ~256 workgroups (the chip has
  // 256 CUs); each split is a multiple of 32 that divides H, and at most 10 splits keep
  // the partial sums the top-k kernel adds small
  const int kb = H / 32;
  int best = 1;
  for (int ns = 1; ns <= std::min(kb, 10); ++ns) {
    if (kb % ns) continue;
    if ((int64_t)p.m_tiles * p.n_tiles * best >= 256) break;
    best = ns;
  }
  p.nsplit = best;
  p.kwaves = false;
  if (T <= 256 && p.m_tiles * p.n_tiles < 256 && E % 16 == 0) {
    // few tokens: 16-expert workgroups whose waves split the k range (each wave's share a
    // multiple of 32); the fewest splits (at most 10) that give ~256 workgroups.  (More
    // tokens keep 64-expert workgroups, which read each token row E/64 times instead of E/16.)
    int ks = 0;
    for (int ns = 1; ns <= std::min(kb, 10); ++ns) {
      if (kb % ns || (kb / ns) % 4) continue;
      ks = ns;
      if ((int64_t)p.m_tiles * (E / 16) * ns >= 256) break;
    }
    if (ks) {
      p.kwaves = true;
      p.nsplit = ks;
      p.n_tiles = E / 16;
    }
  }
  return p;
}

size_t router_partial_bytes(int64_t T, int H, int E) {
  RouterPlan p = router_plan(T, H, E);
  return (size_t)p.nsplit * (size_t)T * (size_t)E * sizeof(float);
}

hipError_t launch_router_logits(const RouterPlan& p, const uint16_t* x, const float* w, int T, int H, int E,
                                float* partial, uint32_t* clear, int64_t clear_words, hipStream_t s, Tracer* tr) {
  dim3 grid(p.n_tiles * p.nsplit, p.m_tiles), block(256);
  const int kchunk = H / p.nsplit;
  if (p.kwaves) {
    if (kchunk % 128 || E % 16) return hipErrorInvalidValue;
#define MOE_RLK(M) \
  launch(tr, router_logits_kwaves_kernel<M>, grid, block, s, x, w, T, H, E, kchunk, partial, clear, clear_words)
    switch (p.mf) {
      case 1: MOE_RLK(1); break;
      case 2: MOE_RLK(2); break;
      case 4: MOE_RLK(4); break;
      default: MOE_RLK(8); break;
    }
#undef MOE_RLK
    hipError_t err = hipGetLastError();
    if (tr) tr->mark("router_logits", s);
    return err;
  }
#define MOE_RL(M, R) \
  launch(tr, router_logits_kernel<M, R>, grid, block, s, x, w, T, H, E, kchunk, partial, clear, clear_words)
  if (p.rf == 2) {
    switch (p.mf) {
      case 1: MOE_RL(1, 2); break;
      case 2: MOE_RL(2, 2); break;
      case 4: MOE_RL(4, 2); break;
      default: MOE_RL(8, 2); break;
    }
  } else {
    switch (p.mf) {
      case 1: MOE_RL(1, 1); break;
      case 2: MOE_RL(2, 1); break;
      case 4: MOE_RL(4, 1); break;
      default: MOE_RL(8, 1); break;
    }
  }
#undef MOE_RL
  hipError_t err = hipGetLastError();
  if (tr) tr->mark("router_logits", s);
  return err;
}

hipError_t launch_router_topk(const float* partial, int nsplit, int T, int E, const float* bias, int G, int TG,
                              int K, int norm, float scale, int32_t* topk_idx, float* topk_w, uint32_t* bitmap,
                              const FusedDispatch& fd, hipStream_t s, Tracer* tr) {
  if (fd.done && (T > FUSED_DISPATCH_MAX_T || (int64_t)T * K > FUSED_DISPATCH_MAX_PAIRS || E > FUSED_DISPATCH_MAX_E))
    return hipErrorInvalidValue;
  const int words = (T + 31) / 32;
  dim3 grid((T + 3) / 4), block(256);
  const int epl = E / WAVE;
#define MOE_TOPK(N)                                                                                        \
  if (fd.done)                                                                                             \
    launch(tr, router_topk_kernel<N, true>, grid, block, s, partial, nsplit, T, E, bias, G, TG, K, norm, scale, \
           topk_idx, topk_w, bitmap, words, fd);                                                          \
  else                                                                                                     \
    launch(tr, router_topk_kernel<N, false>, grid, block, s, partial, nsplit, T, E, bias, G, TG, K, norm, scale, \
           topk_idx, topk_w, bitmap, words, fd)
  switch (epl) {
    case 1: MOE_TOPK(1); break;
    case 2: MOE_TOPK(2); break;
    case 4: MOE_TOPK(4); break;
    case 8: MOE_TOPK(8); break;
    case 16: MOE_TOPK(16); break;
    default: return hipErrorInvalidValue;
  }
#undef MOE_TOPK
  hipError_t err = hipGetLastError();
  if (tr) tr->mark("router_topk", s);
  return err;
}

}  // namespace moe
