// Expert FFNs of the BailingMoeV3 sparse MoE block as a grouped GEMM on bf16 MFMA.
//
// Each expert is a SwiGLU FFN of three matrices, gate and up (hidden -> intermediate) and
// down (intermediate -> hidden) (Ling-3.0-flash-VL routing walk-through page, lqnn.cn,
// section 二); activations may be clamped to +-limit (section 四, expert_swiglu_limit_list);
// routed-expert weights may be MXFP4 (hybrid-attention page, lpnh.cn, table 模型一览).
//
// Work unit (one workgroup): expert e, a tile of up to 16*MF consecutive sorted positions
// of that expert, and a block of NW*RF*16 weight rows.  Design for gfx950:
//   * weights are the MFMA a operand and stream from HBM straight into registers, each
//     wave owning RF 16-row blocks (no LDS round trip, every weight byte is read by exactly
//     one wave); two steps of loads are kept in flight;
//   * the token rows (gathered x rows for gate/up, contiguous h rows for down) are the b
//     operand, staged once per workgroup in double-buffered LDS and shared by all waves;
//   * the reduction dimension is consumed KS values per step.  bf16: MFMA sub-step s takes
//     k = 32s + 8q .. +7 for lane group q of both operands, so one load instruction covers
//     64 contiguous bytes of each of its 16 rows; MXFP4: lane group q owns the 32-value
//     scale block q of a step and sub-step s its s-th 8-value piece, for both operands (the
//     same permutation of k on both sides leaves the dot products unchanged);
//   * gate and up share the token operand; SwiGLU and the clamp run on the accumulators;
//     the activation h is stored as two bf16 planes, hi = bf16(h) and lo = bf16(h - hi),
//     and the down projection runs one MFMA per plane, so h keeps ~16 significand bits
//     through the down GEMM; the down projection writes fp32 expert outputs;
//   * MXFP4 weights (KS = 128: one 16-byte load = 32 codes = one scale block per lane) are
//     decoded exactly to bf16 in registers by the gfx950 scaled fp4 -> bf16 conversion;
//   * the work list (tiles per expert) lives on the device; consecutive work ids are placed
//     on the same XCD so the row blocks of one tile share its token rows in that XCD's L2.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int MODE_GATEUP = 0, MODE_DOWN = 1;

struct FfnArgs {
  const uint16_t* act;          // gate/up: x [T,K]; down: h hi plane [P,K]
  const uint16_t* act_lo;       // down: h lo plane [P,K]
  const int32_t* sorted_token;  // gate/up: token of each sorted position
  const int32_t* offsets;       // [E+2]
  const int32_t* tile_prefix;   // [E+2] tiles of all experts before e
  const void* w0;               // routed gate (gate/up) or down
  const void* w1;               // routed up (gate/up)
  const uint8_t* s0;            // MXFP4 scales of w0
  const uint8_t* s1;            // MXFP4 scales of w1
  const void* sw0;              // shared expert gate or down
  const void* sw1;              // shared expert up
  void* out;                    // gate/up: h hi plane bf16 [P,N]; down: y fp32 [P,N]
  uint16_t* out_lo;             // gate/up: h lo plane bf16 [P,N]
  int T, E, S;
  int K;                        // reduction length
  int N;                        // output columns per expert
  int nrb;                      // row blocks per expert (N / rows per workgroup)
  int rbw;                      // row blocks one workgroup streams back to back
  int ngroups;                  // ceil(nrb / rbw): row-block groups per tile
  int bm_list;                  // positions per tile of the device tile list (a multiple of 16*MF)
  int group_major;              // 1: work id = group * tiles + tile (else tile * groups + group)
  int dense;                    // 1: one weight set and the identity permutation (a dense FFN): tiles
                                // follow from T, no dispatch arrays are read, down writes bf16 out [T,N]
  int ksplit;                   // workgroups splitting the reduction (down of a dense FFN; else 1)
  float* part;                  // ksplit > 1: fp32 partial sums [ksplit,T,N], added in order later
  float limit, shared_limit;
};

__device__ __forceinline__ void block_sync_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// 8 e2m1 codes (low nibble first) times a power of two -> 8 bf16 (exact).  gfx950 converts
// one byte (two codes, low nibble to the low half) per instruction.
__device__ __forceinline__ u32x4 fp4x8_to_bf16x8(uint32_t v, float scale) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 0));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 1));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 2));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(v, scale, 3));
  return o;
}

__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);  // 2^(s-127)
}

template <int NMAT, int RF, int WREGS>
struct WStage {
  u32x4 w[NMAT][RF][WREGS];
  uint32_t sc[NMAT][RF];
};

template <int NTP, int CPT>
struct TStage {
  u32x4 t[NTP][CPT];
};

// One work unit.  D = prefetch distance: the loads of step s + D (weights and the token
// tile) are issued while step s computes, all in one batch, so that waiting for the token
// tile of the next step (loads complete in issue order) never waits for younger weights.
template <int NW, int RF, int MF, int D, int MODE, int KS, bool FP4, bool PADDED>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, int e, int pos0, int nrows, int rb0, int nrb_here,
                                         int ksp, uint16_t* lds) {
  constexpr int NMAT = MODE == MODE_GATEUP ? 2 : 1;
  constexpr int NTP = MODE == MODE_GATEUP ? 1 : 2;  // token planes (h hi and lo for down)
  constexpr int BM = MF * 16;
  constexpr int SUB = KS / 32;       // MFMA sub-steps per step
  constexpr int LROW = KS + 16;      // LDS row stride (bf16); the 32-byte pad measured fewest bank conflicts
  constexpr int NTH = NW * 64;
  constexpr int CHUNKS = BM * KS / 8;  // 16-byte pieces of one token plane per step
  constexpr int CPT = (CHUNKS + NTH - 1) / NTH;
  constexpr int ROWS = NW * RF * 16;
  constexpr int WREGS = FP4 ? 1 : SUB;
  // PADDED, the loop form (each measured fastest for its kernels): tiles of 64+ tokens and
  // the MXFP4 kernel issue every load unconditionally; 16- and 32-token tiles do not

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int kspan = K / a.ksplit, k0 = ksp * kspan;  // this workgroup's part of the reduction
  const int nsteps = kspan / KS;             // k-steps per row block
  const int total_steps = nsteps * nrb_here;  // the pipeline runs through all row blocks
  const bool shared = e == a.E;

  // token tile: per-thread 16-byte pieces (row, col).  Every piece is loaded from a valid
  // address (pieces past the tile or of a position without a token read the tile's first
  // position, or token 0) and the invalid ones are written to LDS as zeros, so every step
  // issues the same loads and the compiler's wait counting stays exact.
  const uint16_t* tsrc[NTP][CPT];
  bool tvalid[CPT];
  int tdst[CPT];
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    const int c = tid + i * NTH;
    const int row = c < CHUNKS ? c / (KS / 8) : 0, col = (c % (KS / 8)) * 8;
    tdst[i] = c < CHUNKS ? row * LROW + col : -1;
    bool ok = c < CHUNKS && row < nrows;
    const int prow = row < nrows ? row : 0;
    if (MODE == MODE_GATEUP) {
      const int tok = a.dense ? pos0 + prow : a.sorted_token[pos0 + prow];
      ok = ok && (unsigned)tok < (unsigned)a.T;
      tsrc[0][i] = a.act + (size_t)((unsigned)tok < (unsigned)a.T ? tok : 0) * K + k0 + col;
    } else {
      tsrc[0][i] = a.act + (size_t)(pos0 + prow) * K + k0 + col;
      tsrc[NTP - 1][i] = a.act_lo + (size_t)(pos0 + prow) * K + k0 + col;
    }
    tvalid[i] = ok;
  }

  // weight rows of this lane.  bf16: sub-step s of a step reads k = 32s + 8q .. +7, so
  // one load instruction covers 64 contiguous bytes of each of the 16 rows.  MXFP4: lane
  // group q owns the 32-value block q of the step (16 bytes of codes, one scale byte) and
  // sub-step s uses its codes 8s .. 8s+7.
  const int nbase = rb0 * ROWS + wave * RF * 16;
  const uint16_t* wp[NMAT][RF];
  const uint8_t* wq[NMAT][RF];
  const uint8_t* wsc[NMAT][RF];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      const size_t row = (size_t)(nbase + f * 16 + r16);
      if constexpr (FP4) {
        const uint8_t* base = (const uint8_t*)(m == 0 ? a.w0 : a.w1) + (size_t)e * N * (K / 2);
        const uint8_t* sbase = (m == 0 ? a.s0 : a.s1) + (size_t)e * N * (K / 32);
        wq[m][f] = base + row * (K / 2) + k0 / 2 + q * (KS / 8);
        wsc[m][f] = sbase + row * (K / 32) + k0 / 32 + q * (KS / 128);
        wp[m][f] = nullptr;
      } else {
        const uint16_t* base = shared ? (const uint16_t*)(m == 0 ? a.sw0 : a.sw1)
                                      : (const uint16_t*)(m == 0 ? a.w0 : a.w1) + (size_t)e * N * K;
        wp[m][f] = base + row * K + k0 + q * 8;
        wq[m][f] = nullptr;
        wsc[m][f] = nullptr;
      }
    }

  floatx4 acc[NMAT][RF][MF];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) acc[m][f][mf] = floatx4{0.f, 0.f, 0.f, 0.f};

  // loads of step `step`; past the last step they repeat the last step's addresses into a
  // ring slot that is not read again
  auto load_t = [&](TStage<NTP, CPT>& ts, int step) {
    const int ks = min(step, total_steps - 1) % nsteps;
#pragma unroll
    for (int p = 0; p < NTP; ++p)
#pragma unroll
      for (int i = 0; i < CPT; ++i) {
        if constexpr (PADDED)
          ts.t[p][i] = *(const u32x4*)(tsrc[p][i] + ks * KS);
        else
          ts.t[p][i] = tvalid[i] ? *(const u32x4*)(tsrc[p][i] + ks * KS) : u32x4{0u, 0u, 0u, 0u};
      }
  };
  auto store_t = [&](const TStage<NTP, CPT>& ts, int buf) {
#pragma unroll
    for (int p = 0; p < NTP; ++p)
#pragma unroll
      for (int i = 0; i < CPT; ++i)
        if (tdst[i] >= 0)
          *(u32x4*)(lds + (buf * NTP + p) * BM * LROW + tdst[i]) = tvalid[i] ? ts.t[p][i] : u32x4{0u, 0u, 0u, 0u};
  };
  // (plain loads: nontemporal loads measured ~25% slower on these streams)
  auto load_w = [&](WStage<NMAT, RF, WREGS>& st, int step) {
    step = min(step, total_steps - 1);
    const int rbi = step / nsteps, ks = step - rbi * nsteps;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int f = 0; f < RF; ++f) {
        if constexpr (FP4) {
          st.w[m][f][0] = *(const u32x4*)(wq[m][f] + (size_t)rbi * ROWS * (K / 2) + (size_t)ks * (KS / 2));
          st.sc[m][f] = wsc[m][f][(size_t)rbi * ROWS * (K / 32) + (size_t)ks * (KS / 32)];
        } else {
#pragma unroll
          for (int s = 0; s < WREGS; ++s)
            st.w[m][f][s] = *(const u32x4*)(wp[m][f] + (size_t)rbi * ROWS * K + (size_t)ks * KS + s * 32);
        }
      }
  };
  auto compute_at_use = [&](const WStage<NMAT, RF, WREGS>& st, int buf) {
    const uint16_t* L = lds + buf * NTP * BM * LROW + r16 * LROW;
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      const int col = FP4 ? q * 32 + s * 8 : s * 32 + q * 8;
      u32x4 wf[NMAT][RF];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if constexpr (FP4) {
            wf[m][f] = fp4x8_to_bf16x8(st.w[m][f][0][s], e8m0_to_f32(st.sc[m][f]));
          } else {
            wf[m][f] = st.w[m][f][s];
          }
        }
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
        for (int p = NTP - 1; p >= 0; --p) {
          const u32x4 tf = *(const u32x4*)(L + p * BM * LROW + mf * 16 * LROW + col);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int f = 0; f < RF; ++f) acc[m][f][mf] = mfma16(wf[m][f], tf, acc[m][f][mf]);
        }
      }
    }
  };
  // The token fragments of sub-step s + 1 are read from LDS while sub-step s runs its MFMAs
  // (scheduling barriers keep the compiler from sinking each read to its first use, which
  // left every pair of MFMAs waiting on an LDS round trip).  256-token tiles, which have no
  // registers to spare, read each fragment where it is used.
  auto compute = [&](const WStage<NMAT, RF, WREGS>& st, int buf) {
    if constexpr (MF > 8) {
      compute_at_use(st, buf);
      return;
    }
    const uint16_t* L = lds + buf * NTP * BM * LROW + r16 * LROW;
    u32x4 tf[2][NTP][MF];
    auto read_frags = [&](u32x4 (&t)[NTP][MF], int s) {
      const int col = FP4 ? q * 32 + s * 8 : s * 32 + q * 8;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int p = 0; p < NTP; ++p) t[p][mf] = *(const u32x4*)(L + p * BM * LROW + mf * 16 * LROW + col);
    };
    // MXFP4: the weights of sub-step s + 1 are also decoded while sub-step s multiplies
    u32x4 wf[2][NMAT][RF];
    auto weights = [&](u32x4 (&w)[NMAT][RF], int s) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if constexpr (FP4) {
            w[m][f] = fp4x8_to_bf16x8(st.w[m][f][0][s], e8m0_to_f32(st.sc[m][f]));
          } else {
            w[m][f] = st.w[m][f][s];
          }
        }
    };
    read_frags(tf[0], 0);
    weights(wf[0], 0);
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      if (s + 1 < SUB) read_frags(tf[(s + 1) & 1], s + 1);
      __builtin_amdgcn_sched_barrier(0);
      if (s + 1 < SUB) weights(wf[(s + 1) & 1], s + 1);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
#pragma unroll
        for (int p = NTP - 1; p >= 0; --p) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int f = 0; f < RF; ++f) acc[m][f][mf] = mfma16(wf[s & 1][m][f], tf[s & 1][p][mf], acc[m][f][mf]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // epilogue of one row block: lane holds token r16 of each fragment and rows 4q .. 4q+3 of
  // each 16-row block
  const float limit = shared ? a.shared_limit : a.limit;
  auto epilogue = [&](int rbi) {
    const int ncol = nbase + rbi * ROWS + 4 * q;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const int j = mf * 16 + r16;
      if (j < nrows) {
        const size_t obase = (size_t)(pos0 + j) * N + ncol;
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if (MODE == MODE_GATEUP) {
            float hv[4], lv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = acc[0][f][mf][r], u = acc[NMAT - 1][f][mf][r];
              float h = g / (1.0f + __expf(-g)) * u;
              if (limit > 0.f) h = fminf(fmaxf(h, -limit), limit);
              hv[r] = bf16_bits_to_f32(f32_to_bf16_bits(h));
              lv[r] = h - hv[r];  // exact in fp32
            }
            *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
            *(u32x2*)(a.out_lo + obase + f * 16) = u32x2{pack_bf16x2(lv[0], lv[1]), pack_bf16x2(lv[2], lv[3])};
          } else if (a.ksplit > 1) {
            *(floatx4*)(a.part + ((size_t)ksp * a.T + pos0 + j) * N + ncol + f * 16) = acc[0][f][mf];
          } else if (a.dense) {
            const floatx4 v = acc[0][f][mf];
            *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else {
            *(floatx4*)((float*)a.out + obase + f * 16) = acc[0][f][mf];
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int mf = 0; mf < MF; ++mf) acc[m][f][mf] = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  WStage<NMAT, RF, WREGS> ws[D];
  TStage<NTP, CPT> ts[D];
#pragma unroll
  for (int j = 0; j < D; ++j) {
    load_t(ts[j], j);
    load_w(ws[j], j);
  }
  store_t(ts[0], 0);
  block_sync_lds();
  if constexpr (PADDED) {
    // the loop runs to a multiple of D steps, every step issuing its loads unconditionally
    // (the steps past the end repeat the last loads into slots nobody reads), so the
    // compiler's own wait counting stays exact
    const int padded_steps = (total_steps + D - 1) / D * D;
    for (int s0 = 0; s0 < padded_steps; s0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int s = s0 + j;
        const bool real = s < total_steps;
        if (real && s + 1 < total_steps) store_t(ts[(j + 1) % D], (s + 1) & 1);
        if (real) compute(ws[j], s & 1);
        load_t(ts[j], s + D);
        load_w(ws[j], s + D);
        if (real && (s + 1) % nsteps == 0) epilogue(s / nsteps);
        block_sync_lds();
      }
    }
  } else {
    // short blocks of a few tokens (decode): no repeated loads past the end, and only the
    // positions that hold a token are loaded
    for (int s0 = 0; s0 < total_steps; s0 += D) {
#pragma unroll
      for (int j = 0; j < D; ++j) {
        const int s = s0 + j;
        if (s < total_steps) {
          if (s + 1 < total_steps) store_t(ts[(j + 1) % D], (s + 1) & 1);
          compute(ws[j], s & 1);
          if (s + D < total_steps) {
            load_t(ts[j], s + D);
            load_w(ws[j], s + D);
          }
          if ((s + 1) % nsteps == 0) epilogue(s / nsteps);
          block_sync_lds();
        }
      }
    }
  }
}

template <int NW, int RF, int MF, int D, int MODE, int FMT, int KS>
__global__ __launch_bounds__(NW * 64) void ffn_kernel(FfnArgs a) {
  constexpr bool PADDED = FMT == FMT_MXFP4 || MF >= 4;
  constexpr int BM = MF * 16;
  constexpr int NTP = MODE == MODE_GATEUP ? 1 : 2;
  __shared__ __align__(16) uint16_t lds[2 * NTP * BM * (KS + 16)];

  // device work list: work id -> (tile, sub-tile, row-block group); consecutive work ids
  // run on the same XCD.  A tile of the list holds bm_list positions and splits into
  // bm_list / BM sub-tiles of this kernel's size (empty sub-tiles exit at once).  Tile-major
  // order puts the row-block groups of a tile side by side (they share its token rows in
  // L2); group-major order, for a single weight set, the tiles of a row-block group (they
  // share its weight rows).
  const int subs = a.bm_list / BM;
  const int ntsub = (a.dense ? (a.T + a.bm_list - 1) / a.bm_list : a.tile_prefix[a.E + a.S]) * subs;
  const int total = ntsub * a.ngroups * a.ksplit;
  const int per_xcd = (total + 7) >> 3;
  const int slot = blockIdx.x >> 3;
  if (slot >= per_xcd) return;
  const int wk = (blockIdx.x & 7) * per_xcd + slot;
  if (wk >= total) return;
  // the parts of a split reduction are consecutive work ids
  const int w = wk / a.ksplit, ksp = wk - w * a.ksplit;
  int tsub, grp;
  if (a.group_major) {
    grp = w / ntsub;
    tsub = w - grp * ntsub;
  } else {
    tsub = w / a.ngroups;
    grp = w - tsub * a.ngroups;
  }
  const int tile = tsub / subs, sub = tsub - tile * subs;
  const int rb0 = grp * a.rbw, nrb_here = min(a.rbw, a.nrb - rb0);
  const int4 info = a.dense ? int4{0, tile * a.bm_list, min(a.bm_list, a.T - tile * a.bm_list), 0}
                            : ((const int4*)(a.tile_prefix + tile_info_offset(a.E)))[tile];
  const int e = info.x, m0 = sub * BM;
  if (m0 >= info.z) return;
  const int nrows = min(BM, info.z - m0);
  if constexpr (FMT == FMT_MXFP4) {
    if (e < a.E) {
      ffn_tile<NW, RF, MF, D, MODE, KS, true, PADDED>(a, e, info.y + m0, nrows, rb0, nrb_here, ksp, lds);
      return;
    }
  }
  ffn_tile<NW, RF, MF, D, MODE, KS, false, PADDED>(a, e, info.y + m0, nrows, rb0, nrb_here, ksp, lds);
}

// out[i] = bf16(sum over s of part[s][i]), the parts of a split reduction added in order;
// four values per thread
__global__ __launch_bounds__(256) void ksplit_sum_kernel(const float* __restrict__ part, int ksplit, int64_t n4,
                                                         uint16_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
  floatx4 v = ((const floatx4*)part)[i];
  for (int s = 1; s < ksplit; ++s) v += ((const floatx4*)part)[s * n4 + i];
  ((u32x2*)out)[i] = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
}

// single wave: tiles of expert i = ceil(count_i / bm); tile_prefix = exclusive scan, and the
// tile records after it (n = E + S experts, the tile_info block at tile_info_offset(n - S))
__global__ __launch_bounds__(64) void tile_prefix_kernel(const int32_t* __restrict__ offsets, int n, int bm,
                                                         int32_t* __restrict__ tile_prefix, int info_off) {
  const int lane = threadIdx.x;
  const int per = (n + WAVE - 1) / WAVE;
  const int b = lane * per, e = min(n, b + per);
  int sum = 0;
  for (int i = b; i < e; ++i) sum += (offsets[i + 1] - offsets[i] + bm - 1) / bm;
  int incl = sum;
#pragma unroll
  for (int m = 1; m < WAVE; m <<= 1) {
    int o = __shfl_up(incl, m, WAVE);
    if (lane >= m) incl += o;
  }
  int run = incl - sum;
  if (lane == 0) tile_prefix[0] = 0;
  int4* info = (int4*)(tile_prefix + info_off);
  for (int i = b; i < e; ++i) {
    const int o = offsets[i], c = offsets[i + 1] - o;
    for (int j = 0; j * bm < c; ++j) info[run + j] = int4{i, o + j * bm, min(bm, c - j * bm), 0};
    run += (c + bm - 1) / bm;
    tile_prefix[i + 1] = run;
  }
}

// Kernel configuration per (tile size, weight format, GEMM): NW waves, RF 16-row weight
// blocks per wave (rows per workgroup and matrix NW*RF*16: 128, or 64 for the 16-token bf16
// tiles of decode, whose smaller workgroups measured faster: gate/up 4 %, down 1.5 %), KS
// values of k per step, D steps of loads in flight.  Otherwise the down GEMM, which reads two
// h planes per token fragment, keeps two weight blocks per wave to halve its LDS reads per
// MFMA.  16-token bf16 tiles (decode) take 256-value steps, two in flight, in 64-row
// workgroups: each weight row then goes out in 512-byte runs (measured: decode gate/up 311 ->
// 297 us, down 161 -> 159 us against 64-value steps); so does the gate/up of 32-token tiles
// (T = 1024: 683 -> 655 us; their down GEMM measured slower that way).  The down GEMM of
// 16-token tiles takes 384-value steps, so that a 768-long reduction is two steps, both in
// flight from the start (decode down 155.4 -> 153.9 us).  Where K is not a multiple of the
// step they fall back to 256-value steps (KS_MID), then to 128-value steps, four in flight
// (KS_ALT, D_ALT).
template <int MF, int FMT, int MODE> struct FfnCfg {
  static constexpr bool FP4 = FMT == FMT_MXFP4;
  static constexpr bool DOWN = MODE == MODE_DOWN;
  static constexpr bool WIDE = !FP4 && (MF == 1 || (MF == 2 && !DOWN));
  static constexpr int NW = (MF <= 2 || DOWN) ? 4 : 8;
  static constexpr int RF = WIDE ? 1 : (MF <= 2 || DOWN) ? 2 : 1;
  static constexpr int KS = FP4 ? 128 : WIDE ? ((MF == 1 && DOWN) ? 384 : 256) : 64;
  static constexpr int D = WIDE ? 2
                         : MF <= 2 ? (FP4 ? 3 : 4)
                         : MF == 4 ? (FP4 ? 2 : 4)
                         : MF == 8 ? (FP4 ? 2 : (DOWN ? 3 : 4))
                                   : 2;
  static constexpr int KS_MID = WIDE ? 256 : KS;  // where K is not a multiple of KS
  static constexpr int KS_ALT = WIDE ? 128 : KS, D_ALT = WIDE ? 4 : D;
};

template <int MF, int MODE, int FMT>
hipError_t launch_one(FfnArgs a, int rbw, int64_t max_tiles, hipStream_t s, Tracer* tr) {
  using C = FfnCfg<MF, FMT, MODE>;
  constexpr int ROWS = C::NW * C::RF * 16;  // weight rows per block of each matrix
  if (a.bm_list % (16 * MF) || a.N % ROWS || a.ksplit < 1 || a.K % a.ksplit) return hipErrorInvalidValue;
  const int kspan = a.K / a.ksplit;
  a.nrb = a.N / ROWS;
  a.rbw = std::min(a.nrb, rbw);
  a.ngroups = (a.nrb + a.rbw - 1) / a.rbw;
  int64_t work = max_tiles * (a.bm_list / (16 * MF)) * a.ngroups * a.ksplit;
  int64_t grid = (work + 7) / 8 * 8;
  if (grid <= 0) return hipSuccess;
  if (kspan % C::KS == 0)
    launch(tr, ffn_kernel<C::NW, C::RF, MF, C::D, MODE, FMT, C::KS>, dim3((unsigned)grid), dim3(C::NW * 64), s, a);
  else if (C::KS_MID != C::KS && kspan % C::KS_MID == 0)
    launch(tr, ffn_kernel<C::NW, C::RF, MF, C::D, MODE, FMT, C::KS_MID>, dim3((unsigned)grid), dim3(C::NW * 64), s,
           a);
  else if (C::KS_ALT != C::KS && kspan % C::KS_ALT == 0)
    launch(tr, ffn_kernel<C::NW, C::RF, MF, C::D_ALT, MODE, FMT, C::KS_ALT>, dim3((unsigned)grid), dim3(C::NW * 64), s,
           a);
  else
    return hipErrorInvalidValue;
  hipError_t err = hipGetLastError();
  if (tr) tr->mark(MODE == MODE_GATEUP ? "expert_gate_up" : "expert_down", s);
  return err;
}

template <int MODE>
hipError_t launch_mode(int mf, const FfnArgs& a, int rbw, int fmt, int64_t max_tiles, hipStream_t s, Tracer* tr) {
  if (fmt == FMT_MXFP4) {
    switch (mf) {
      case 1: return launch_one<1, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      case 2: return launch_one<2, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      case 4: return launch_one<4, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      case 8: return launch_one<8, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      default: return hipErrorInvalidValue;  // the plan never picks 16 for MXFP4
    }
  }
  switch (mf) {
    case 1: return launch_one<1, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr);
    case 2: return launch_one<2, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr);
    case 4: return launch_one<4, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr);
    case 8: return launch_one<8, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr);
    default: return launch_one<16, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr);
  }
}

}  // namespace

FfnPlan ffn_plan(int64_t T, int K, int E, int S, int fmt, int H, int I) {
  FfnPlan p;
  const double avg = (double)T * K / E;  // routed tokens per expert on average
  // tile list of 16*mf positions; gate/up runs whole tiles, down runs sub-tiles of 16*mf_down
  // (measured: the down GEMM, which reads two h planes, is fastest with 64-token tiles at
  // two waves per SIMD; gate/up with 128, or 256 when experts average well above 128 tokens;
  // MXFP4 experts with up to 96 tokens on average take 64-token tiles: at 64 per expert,
  // gate/up 0.694 -> 0.731 ms but down 0.606 -> 0.548 ms)
  p.mf = avg <= 12 ? 1 : avg <= 24 ? 2 : (avg <= 48 || (fmt == FMT_MXFP4 && avg <= 96)) ? 4
       : (avg <= 192 || fmt == FMT_MXFP4) ? 8 : 16;
  p.mf_gate_up = p.mf;
  p.mf_down = std::min(p.mf, 4);
  // more than 12 tokens per expert and bf16 weights: the 256-token tile kernel (ffn_tile.hip)
  // (measured against the small tiles: T = 1024 (16 per expert) 1.094 -> 1.074 ms, T = 1536
  // 1.297 -> 1.215, T = 2048 1.446 -> 1.294, T = 4096 1.89 -> 1.57)
  p.tiles = fmt == FMT_BF16 && avg > 12 && ffn_tiles_supported(H, I);
  p.group_major = false;
  p.ksplit_down = 1;
  if (p.tiles) p.mf = 16;
  p.bm = 16 * p.mf;
  // row blocks streamed back to back by one workgroup: long-lived workgroups amortise the
  // pipeline start; few tokens per expert keep more, shorter workgroups for parallelism
  p.rbw_gate_up = p.mf >= 4 ? 3 : 1;
  p.rbw_down = p.mf >= 4 ? 5 : 1;  // decode: one row block per workgroup (measured)
  if (E == 1 && S == 0 && avg <= 4096) {
    // a single expert (the dense FFN) has no experts to spread over the CUs: one row block per
    // workgroup, so that token tiles x row blocks fill the chip, with tiles of 16 to 256 tokens
    // growing with T (measured at hidden 2560, intermediate 6912, against 16-token tiles up to
    // 128 tokens: T = 64 67 -> 49 us, T = 128 125 -> 78; against 64-token tiles up to 512:
    // T = 512 175 -> 141 us); up to 512 tokens the tiles of one row block run side by side on
    // one XCD (group-major work order), so that its weight rows come from L2 for all but the
    // first.  Above 4096 tokens the 256-position tile kernel is faster (T = 4096 0.76 against
    // 0.90 ms, T = 8192 1.47 against 1.26 ms).
    p.mf = avg <= 32 ? 1 : avg <= 128 ? 2 : avg <= 256 ? 4 : avg <= 2048 ? 8 : 16;
    p.mf_gate_up = p.mf;
    p.mf_down = std::min(p.mf, 4);
    p.tiles = false;
    p.bm = 16 * p.mf;
    p.rbw_gate_up = p.rbw_down = 1;
    p.group_major = avg <= 512;  // measured: T = 64 88 -> 83 us, 128 158 -> 144, 512 206 -> 198; 1024 279 -> 282
    // few tokens: the down GEMM (H / 64 or H / 128 row blocks per tile) also splits its
    // reduction over up to DENSE_MAX_KSPLIT workgroups, toward ~768 workgroups; the split
    // must leave a whole number of 128-value (one 16-token fragment) or 64-value steps
    if (avg <= DENSE_KSPLIT_MAX_T) {
      const int64_t tiles = (T + 16 * p.mf_down - 1) / (16 * p.mf_down);
      const int rows = p.mf_down == 1 ? 64 : 128, ks_step = p.mf_down == 1 ? 128 : 64;
      const int64_t want = std::max<int64_t>(1, 768 / std::max<int64_t>(1, tiles * (H / rows)));
      for (int d = (int)std::min<int64_t>(want, DENSE_MAX_KSPLIT); d > 1; --d)
        if (I % d == 0 && (I / d) % ks_step == 0) {
          p.ksplit_down = d;
          break;
        }
    }
  }
  const int64_t pairs = T * K + T * S;
  p.max_tiles = pairs / p.bm + std::min<int64_t>(E, T * K) + S + 1;
  return p;
}

hipError_t launch_expert_ffn(const FfnPlan& p, const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                             int32_t* tile_prefix, const FfnWeights& w, int T, int H, int I, int E, int S,
                             float limit, float shared_limit, uint16_t* h_hi, uint16_t* h_lo, float* y,
                             bool tiles_ready, hipStream_t s, Tracer* tr) {
  hipError_t err = hipSuccess;
  if (p.tiles) {
    if (!tiles_ready) {
      launch(tr, tile_prefix_kernel, dim3(1), dim3(64), s, offsets, E + S, p.bm, tile_prefix, tile_info_offset(E));
      err = hipGetLastError();
      if (tr) tr->mark("expert_tiles", s);
      if (err != hipSuccess) return err;
    }
    return launch_expert_ffn_tiles(x, offsets, sorted_token, tile_prefix, p.max_tiles, w, T, H, I, E, S, limit,
                                   shared_limit, h_hi, h_lo, y, s, tr);
  }
  if (!tiles_ready) {
    launch(tr, tile_prefix_kernel, dim3(1), dim3(64), s, offsets, E + S, p.bm, tile_prefix, tile_info_offset(E));
    err = hipGetLastError();
    if (tr) tr->mark("expert_tiles", s);
  }
  if (err != hipSuccess) return err;

  FfnArgs gu{};
  gu.act = x; gu.sorted_token = sorted_token; gu.offsets = offsets; gu.tile_prefix = tile_prefix;
  gu.w0 = w.gate; gu.w1 = w.up; gu.s0 = w.gate_scale; gu.s1 = w.up_scale;
  gu.sw0 = w.sh_gate; gu.sw1 = w.sh_up; gu.out = h_hi; gu.out_lo = h_lo;
  gu.T = T; gu.E = E; gu.S = S; gu.K = H; gu.N = I;
  gu.limit = limit; gu.shared_limit = shared_limit;
  gu.ksplit = 1;

  FfnArgs dn = gu;
  dn.act = h_hi; dn.act_lo = h_lo; dn.sorted_token = nullptr; dn.out_lo = nullptr;
  dn.w0 = w.down; dn.w1 = nullptr; dn.s0 = w.down_scale; dn.s1 = nullptr;
  dn.sw0 = w.sh_down; dn.sw1 = nullptr; dn.out = y;
  dn.K = I; dn.N = H;

  gu.bm_list = dn.bm_list = p.bm;
  gu.group_major = dn.group_major = p.group_major ? 1 : 0;
  err = launch_mode<MODE_GATEUP>(p.mf_gate_up, gu, p.rbw_gate_up, w.fmt, p.max_tiles, s, tr);
  if (err != hipSuccess) return err;
  return launch_mode<MODE_DOWN>(p.mf_down, dn, p.rbw_down, w.fmt, p.max_tiles, s, tr);
}

hipError_t launch_dense_ffn_tiled(const FfnPlan& p, const uint16_t* x, const uint16_t* gate, const uint16_t* up,
                                  const uint16_t* down, int T, int H, int I, float limit, uint16_t* h_hi,
                                  uint16_t* h_lo, float* part, uint16_t* out, hipStream_t s) {
  if (p.tiles) return hipErrorInvalidValue;  // the 256-position tile kernel reads the dispatch arrays
  if (p.ksplit_down > 1 && !part) return hipErrorInvalidValue;
  FfnArgs gu{};
  gu.act = x; gu.w0 = gate; gu.w1 = up; gu.out = h_hi; gu.out_lo = h_lo;
  gu.T = T; gu.E = 1; gu.S = 0; gu.K = H; gu.N = I;
  gu.limit = limit;
  gu.bm_list = p.bm;
  gu.group_major = p.group_major ? 1 : 0;
  gu.dense = 1;
  gu.ksplit = 1;
  FfnArgs dn = gu;
  dn.act = h_hi; dn.act_lo = h_lo; dn.out_lo = nullptr; dn.w0 = down; dn.w1 = nullptr; dn.out = out;
  dn.K = I; dn.N = H;
  dn.ksplit = p.ksplit_down;
  dn.part = part;
  const int64_t ntiles = ((int64_t)T + p.bm - 1) / p.bm;
  hipError_t err = launch_mode<MODE_GATEUP>(p.mf_gate_up, gu, p.rbw_gate_up, FMT_BF16, ntiles, s, nullptr);
  if (err != hipSuccess) return err;
  err = launch_mode<MODE_DOWN>(p.mf_down, dn, p.rbw_down, FMT_BF16, ntiles, s, nullptr);
  if (err != hipSuccess || dn.ksplit == 1) return err;
  const int64_t n4 = (int64_t)T * H / 4;
  hipLaunchKernelGGL(ksplit_sum_kernel, dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, s, (const float*)part,
                     dn.ksplit, n4, out);
  return hipGetLastError();
}

}  // namespace moe
