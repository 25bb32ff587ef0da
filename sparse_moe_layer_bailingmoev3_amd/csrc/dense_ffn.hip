// Dense SwiGLU FFN for a few tokens (the dense FFN layers of the model: Ling-3.0-flash-VL
// routing walk-through page, lqnn.cn, section 二, first_k_dense_replace; the same SwiGLU form as
// the experts, with the optional clamp of section 四).
//
// With one weight set and at most 10 tokens the work is a stream of the three weight matrices,
// and parallelism can only come from the weight rows and the reduction dimension.  Design for
// gfx950:
//   * a workgroup owns a block of 16 weight rows (of gate and up together, or of down) and the
//     16-token tile; its NWK waves split the reduction range into NWK contiguous pieces, so the
//     grid holds N/16 * NWK waves (1728 for gate/up, 640 for down at hidden 2560 and
//     intermediate 6912) instead of one wave per 16 rows of a full-length reduction;
//   * each wave streams its weight rows and its slice of the token rows straight from global
//     memory into registers (the token rows are small and stay in L2), with no LDS and no
//     barrier in the loop; every load of a step is issued unconditionally;
//   * few bytes in flight: one 64-value step (gate/up) or two 96-value steps (down) per wave,
//     about 7 MB over the chip; the same reads with four times as much in flight measured
//     1.6x slower (28 -> 47 us per call at T = 1): the memory system congests;
//   * the NWK partial sums are added once through LDS, in wave order (deterministic), and the
//     first wave runs the epilogue: SwiGLU, clamp and the two bf16 planes of h (hi = bf16(h),
//     lo = bf16(h - hi); the expert FFN kernels keep one fp16 plane instead) after gate/up;
//     after down, the bf16 output
//     itself (a dense FFN has one slot per token with weight 1, so no combine is needed);
//   * k permutation: lane group q of a 16-row operand owns the contiguous slice
//     [q*KS/4, (q+1)*KS/4) of a step and MFMA sub-step s takes its s-th 8-value piece, the
//     same for both operands, so every lane loads one contiguous run per row.
// Every wave reads the token rows of its own slice, so the token traffic grows with T (down
// reads two h planes per token); above 10 tokens the expert FFN kernels, which share a token
// tile between the waves of a workgroup through LDS and split the down reduction over
// workgroups, measured faster.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int DN_GATEUP = 0, DN_DOWN = 1;

struct DenseArgs {
  const uint16_t* act;     // gate/up: x [T,K]; down: h hi plane [T,K]
  const uint16_t* act_lo;  // down: h lo plane [T,K]
  const uint16_t* w0;      // gate [N,K] (gate/up) or down [N,K]
  const uint16_t* w1;      // up [N,K] (gate/up)
  uint16_t* out;           // gate/up: h hi plane [T,N]; down: the layer output [T,N]
  uint16_t* out_lo;        // gate/up: h lo plane [T,N]
  int T, K, N;
  float limit;             // SwiGLU clamp (gate/up), 0 = none
};

template <int MODE, int NWK, int KS, int D>
__global__ __launch_bounds__(NWK * 64) void dense_ffn_kernel(DenseArgs a) {
  constexpr int NMAT = MODE == DN_GATEUP ? 2 : 1;
  constexpr int NTP = MODE == DN_GATEUP ? 1 : 2;  // token planes (h hi and lo for down)
  constexpr int SUB = KS / 32;
  __shared__ floatx4 red[(NWK - 1) * NMAT * 64];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int nrb = a.N / 16;  // row blocks; consecutive ones run on one XCD
  const int per_xcd = (nrb + 7) >> 3;
  const int rb = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
  if ((blockIdx.x >> 3) >= per_xcd || rb >= nrb) return;  // uniform over the workgroup

  const int K = a.K, kw = K / NWK, nsteps = kw / KS;
  const int k0 = wave * kw + q * (KS / 4);
  const uint16_t* wp[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) wp[m] = (m == 0 ? a.w0 : a.w1) + (size_t)(rb * 16 + r16) * K + k0;
  // lanes of token rows past T read row T - 1 (their results are never stored)
  const int tok = min(r16, a.T - 1);
  const uint16_t* tp[NTP];
#pragma unroll
  for (int p = 0; p < NTP; ++p) tp[p] = (p == 0 ? a.act : a.act_lo) + (size_t)tok * K + k0;

  struct Stage {
    u32x4 w[NMAT][SUB];
    u32x4 t[NTP][SUB];
  };
  // loads of step `step`; past the last step they repeat its addresses into a ring slot that
  // is not read again (every step issues the same loads: the compiler's wait counts stay exact)
  auto load = [&](Stage& st, int step) {
    const int ko = min(step, nsteps - 1) * KS;
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m) st.w[m][s] = *(const u32x4*)(wp[m] + ko + s * 8);
#pragma unroll
      for (int p = 0; p < NTP; ++p) st.t[p][s] = *(const u32x4*)(tp[p] + ko + s * 8);
    }
  };
  floatx4 acc[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) acc[m] = floatx4{0.f, 0.f, 0.f, 0.f};
  auto compute = [&](const Stage& st) {
#pragma unroll
    for (int s = 0; s < SUB; ++s)
#pragma unroll
      for (int p = NTP - 1; p >= 0; --p)
#pragma unroll
        for (int m = 0; m < NMAT; ++m) acc[m] = mfma16(st.w[m][s], st.t[p][s], acc[m]);
  };

  Stage ring[D];
#pragma unroll
  for (int j = 0; j < D; ++j) load(ring[j], j);
  const int padded = (nsteps + D - 1) / D * D;
  for (int s0 = 0; s0 < padded; s0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      if (s0 + j < nsteps) compute(ring[j]);
      load(ring[j], s0 + j + D);
    }
  }

  // partial sums of waves 1 .. NWK-1 through LDS (lane-contiguous: no bank conflicts), added
  // to wave 0's in wave order
  if (wave > 0) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m) red[((wave - 1) * NMAT + m) * 64 + lane] = acc[m];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int v = 1; v < NWK; ++v)
#pragma unroll
    for (int m = 0; m < NMAT; ++m) acc[m] += red[((v - 1) * NMAT + m) * 64 + lane];

  // epilogue: lane holds token r16 and rows 4q .. 4q+3 of the 16-row block
  if (r16 < a.T) {
    const size_t o = (size_t)r16 * a.N + rb * 16 + 4 * q;
    if constexpr (MODE == DN_GATEUP) {
      float hv[4], lv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float g = acc[0][r], u = acc[1][r];
        float h = g / (1.0f + __expf(-g)) * u;
        if (a.limit > 0.f) h = fminf(fmaxf(h, -a.limit), a.limit);
        hv[r] = bf16_bits_to_f32(f32_to_bf16_bits(h));
        lv[r] = h - hv[r];  // exact in fp32
      }
      *(u32x2*)(a.out + o) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
      *(u32x2*)(a.out_lo + o) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
    } else {
      *(u32x2*)(a.out + o) = u32x2{pack_bf16x2(acc[0][0], acc[0][1]), pack_bf16x2(acc[0][2], acc[0][3])};
    }
  }
}

// Configurations (measured on MI355X, hidden 2560, intermediate 6912): NWK waves splitting the
// reduction, KS values per step, D steps in flight; a 32-value step (D32 in flight) where KS
// does not divide a wave's slice.  Alternatives measured slower at T = 1 / 16: gate/up with
// 128-value steps (42.8 / 64.7 us per call) or eight waves (43.1 / 61.9); down with eight waves
// (30.1 / 48.5), three steps in flight (28.4 / 46.1), two row blocks per wave (35.9 / 56.0) or
// 192-value steps (31.4 / 50.4); against 28.2 / 45.2 us for these.
struct GateUpCfg { static constexpr int NWK = 4, KS = 64, D = 1, D32 = 2; };
struct DownCfg { static constexpr int NWK = 4, KS = 96, D = 2, D32 = 4; };

template <int MODE, int NWK, int KS, int D>
hipError_t launch_cfg(const DenseArgs& a, hipStream_t s) {
  const int total = a.N / 16;
  const int grid = (total + 7) / 8 * 8;
  hipLaunchKernelGGL((dense_ffn_kernel<MODE, NWK, KS, D>), dim3(grid), dim3(NWK * 64), 0, s, a);
  return hipGetLastError();
}

template <int MODE, int NWK, int KS, int D, int D32>
hipError_t launch_ks(const DenseArgs& a, hipStream_t s) {
  if (a.N % 16 || a.K % NWK || (a.K / NWK) % 32) return hipErrorInvalidValue;
  if ((a.K / NWK) % KS == 0) return launch_cfg<MODE, NWK, KS, D>(a, s);
  return launch_cfg<MODE, NWK, 32, D32>(a, s);
}

}  // namespace

bool dense_ffn_small_supported(int64_t T, int H, int I) {
  return T >= 1 && T <= DENSE_SMALL_MAX_T && H % 128 == 0 && I % 128 == 0;
}

hipError_t launch_dense_ffn_small(const uint16_t* x, const uint16_t* gate, const uint16_t* up, const uint16_t* down,
                                  int T, int H, int I, float limit, uint16_t* h_hi, uint16_t* h_lo, uint16_t* out,
                                  hipStream_t s) {
  if (!dense_ffn_small_supported(T, H, I)) return hipErrorInvalidValue;
  DenseArgs gu{};
  gu.act = x; gu.w0 = gate; gu.w1 = up; gu.out = h_hi; gu.out_lo = h_lo;
  gu.T = T; gu.K = H; gu.N = I; gu.limit = limit;
  DenseArgs dn{};
  dn.act = h_hi; dn.act_lo = h_lo; dn.w0 = down; dn.out = out;
  dn.T = T; dn.K = I; dn.N = H;
  hipError_t e = launch_ks<DN_GATEUP, GateUpCfg::NWK, GateUpCfg::KS, GateUpCfg::D, GateUpCfg::D32>(gu, s);
  if (e != hipSuccess) return e;
  return launch_ks<DN_DOWN, DownCfg::NWK, DownCfg::KS, DownCfg::D, DownCfg::D32>(dn, s);
}

}  // namespace moe
