// Expert FFNs of the BailingMoeV3 sparse MoE block as a grouped GEMM on bf16 MFMA.
//
// Each expert is a SwiGLU FFN of three matrices, gate and up (hidden -> intermediate) and
// down (intermediate -> hidden) (Ling-3.0-flash-VL routing walk-through page, lqnn.cn,
// section 二); activations may be clamped to +-limit (section 四, expert_swiglu_limit_list);
// routed-expert weights may be MXFP4 or MXFP8 (hybrid-attention page, lpnh.cn, table 模型一览:
// "FP8 + MXFP4").
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
//     the activation h is stored as one plane: fp16 (11 significand bits) for bf16 and MXFP8
//     weights, whose down GEMM converts (bf16) or decodes (MXFP8) its weights to fp16 and
//     runs on the fp16 MFMA, bf16 for MXFP4 weights; the down projection writes fp32 expert
//     outputs, or fp16 ones inside moe_forward;
//   * MXFP4 weights (KS = 128: one 16-byte load = 32 codes = one scale block per lane) and
//     MXFP8 weights (two 16-byte loads for the same 32 values) are decoded exactly to bf16 in
//     registers by gfx950's scaled fp4 / fp8 -> bf16 conversions;
//   * the work list (tiles per expert) lives on the device; consecutive work ids are placed
//     on the same XCD so the row blocks of one tile share its token rows in that XCD's L2.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int MODE_GATEUP = 0, MODE_DOWN = 1;

struct FfnArgs {
  const uint16_t* act;          // gate/up: x [T,K]; down: h hi plane [P,K]
  const int32_t* sorted_token;  // gate/up: token of each sorted position
  const int32_t* offsets;       // [E+2]
  const int32_t* tile_prefix;   // [E+2] tiles of all experts before e
  const void* w0;               // routed gate (gate/up) or down
  const void* w1;               // routed up (gate/up)
  const uint8_t* s0;            // MX (block-format) scales of w0
  const uint8_t* s1;            // MX scales of w1
  const void* sw0;              // shared expert gate or down
  const void* sw1;              // shared expert up
  void* out;                    // gate/up: h plane (fp16, or bf16 for MXFP4) [P,N]; down: y fp32 (fp16 with y16) [P,N]
  int T, E, S;
  int K;                        // reduction length
  int N;                        // output columns per expert
  int nrb;                      // row blocks per expert (N / rows per workgroup)
  int rbw;                      // row blocks one workgroup streams back to back
  int ngroups;                  // ceil(nrb / rbw): row-block groups per tile
  int bm_list;                  // positions per tile of the device tile list (a multiple of 16*MF)
  int group_major;              // 1: work id = group * tiles + tile (else tile * groups + group)
  int dense;                    // 1: one weight set and the identity permutation (a dense FFN, or the
                                // shared expert of a block-format layer): tiles follow from T, no
                                // dispatch arrays are read
  int out_bf16;                 // down writes bf16 out [T,N] (the dense FFN) instead of fp32 y
  int y16;                      // down writes y as fp16 [P,N] (saturated at +-65504) instead of fp32
  int ksplit;                   // workgroups splitting the reduction (down of a dense FFN; else 1)
  float* part;                  // ksplit > 1: fp32 partial sums [ksplit,T,N], added in order later
  float limit, shared_limit;
  // MXFP8 activations of the routed experts (the scaled-MFMA path): codes and e8m0 scales of
  // the token operand (gate/up: x [T,K] and [T,K/32]; down: h [P,K] and [P,K/32]) and, for
  // gate/up, of the h it writes ([P,N] and [P,N/32])
  const uint8_t* aq;
  const uint8_t* as;
  uint8_t* oq;
  uint8_t* os;
  // the launch covers the tiles of experts e_lo .. e_hi-1 only (e_hi = 0: all E + S experts)
  int e_lo, e_hi;
  // MXFP4 weights in the tiled order (codes in 1 KB blocks of 16 rows x 128 values, lane
  // (r, q) holding row r's values 32q .. 32q+31 at byte 16 * (16q + r); scales in 128-byte
  // blocks of 16 rows x 256 values, row r's eight block scales at byte 8r), else row-major
  int tiled;
};

typedef int i32x8 __attribute__((ext_vector_type(8)));

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

// 8 E4M3 codes (two words, low byte first) times a power of two -> 8 bf16 (exact: every E4M3
// value times 2^(s-127) within the e8m0 range is a bf16).  gfx950 converts two codes (one
// 16-bit half of a word) per instruction.
__device__ __forceinline__ u32x4 fp8x8_to_bf16x8(uint32_t v0, uint32_t v1, float scale) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v0, scale, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v0, scale, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v1, scale, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v1, scale, true));
  return o;
}

// The same 8 E4M3 codes times a power of two -> 8 fp16: exact while the products stay within
// fp16's range (2^-24 .. 65504 in magnitude, i.e. block scales from 2^-15 to 2^7 for every
// code; model weights sit far inside), smaller ones rounded to fp16's subnormal grid.
__device__ __forceinline__ u32x4 fp8x8_to_f16x8(uint32_t v0, uint32_t v1, float scale) {
  u32x4 o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v0, scale, false));
  o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v0, scale, true));
  o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v1, scale, false));
  o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(v1, scale, true));
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

// h passes from gate/up to down as one plane: fp16 (11 significant bits) for bf16 and MXFP8
// expert weights, held to max|err| <= 2e-2 RMS, whose down GEMM converts the bf16 weights to
// fp16 in registers (exact for model weights) or decodes the MXFP8 ones to fp16 and runs on
// the fp16 MFMA; bf16 for MXFP4 expert weights, held to 5e-2 RMS (the rounding of h to bf16
// alone measured at most 2.5e-2 RMS, on the tiny layouts with few, large expert sums).
template <int MODE, int WF> struct HPlanes {
  static constexpr int value = 1;
};
template <int WF> struct HFp16 {
  static constexpr bool value = WF != FMT_MXFP4;
};

// One work unit.  D = prefetch distance: the loads of step s + D (weights and the token
// tile) are issued while step s computes, all in one batch, so that waiting for the token
// tile of the next step (loads complete in issue order) never waits for younger weights.
template <int NW, int RF, int MF, int D, int MODE, int KS, int WF, bool PADDED>
__device__ __forceinline__ void ffn_tile(const FfnArgs& a, int e, int pos0, int nrows, int rb0, int nrb_here,
                                         int ksp, uint16_t* lds) {
  constexpr int NMAT = MODE == MODE_GATEUP ? 2 : 1;
  constexpr int NTP = HPlanes<MODE, WF>::value;  // token planes (one: x for gate/up, h for down)
  constexpr int BM = MF * 16;
  constexpr int SUB = KS / 32;       // MFMA sub-steps per step
  constexpr int LROW = KS + 16;      // LDS row stride (bf16); the 32-byte pad measured fewest bank conflicts
  constexpr int NTH = NW * 64;
  constexpr int CHUNKS = BM * KS / 8;  // 16-byte pieces of one token plane per step
  constexpr int CPT = (CHUNKS + NTH - 1) / NTH;
  constexpr int ROWS = NW * RF * 16;
  constexpr bool MX = WF != FMT_BF16;       // block-format weights (MXFP4 or MXFP8), KS = 128
  constexpr bool FP4 = WF == FMT_MXFP4;
  constexpr int WREGS = MX ? (FP4 ? 1 : 2) : SUB;  // 16-byte weight registers per (matrix, row block) and step
  static_assert(!MX || KS == 128, "MX weights take 128-value steps");
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
    }
    tvalid[i] = ok;
  }

  // weight rows of this lane.  bf16: sub-step s of a step reads k = 32s + 8q .. +7, so
  // one load instruction covers 64 contiguous bytes of each of the 16 rows.  MXFP4: lane
  // group q owns the 32-value block q of the step (16 bytes of codes, one scale byte) and
  // sub-step s uses its codes 8s .. 8s+7.  MXFP8: lane group q owns values 16q .. 16q+15 and
  // 64+16q .. 64+16q+15 of the step (the scaled MFMA's E4M3 operand layout, so that one tiled
  // order serves both kernels), sub-step s values 16q + 8(s&1) + 64(s>>1) .. +7, whose block
  // scale is byte (q>>1) + 2(s>>1) of the row's scale word of the step.
  const int nbase = rb0 * ROWS + wave * RF * 16;
  const uint16_t* wp[NMAT][RF];
  const uint8_t* wq[NMAT][RF];
  const uint8_t* wsc[NMAT][RF];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int f = 0; f < RF; ++f) {
      const size_t row = (size_t)(nbase + f * 16 + r16);
      if constexpr (MX) {
        constexpr int VPB = FP4 ? 2 : 1;  // values per byte
        const uint8_t* base = (const uint8_t*)(m == 0 ? a.w0 : a.w1) + (size_t)e * N * (K / VPB);
        const uint8_t* sbase = (m == 0 ? a.s0 : a.s1) + (size_t)e * N * (K / 32);
        if (a.tiled) {  // (no split reduction for block-format weights: k0 = 0)
          const size_t b16 = (size_t)(nbase + f * 16) / 16;
          wq[m][f] = base + b16 * (K / 128) * 1024 * WREGS + lane * 16;
          wsc[m][f] = sbase + b16 * (K / 256) * 128 + r16 * 8 + (FP4 ? q : 0);
        } else {
          wq[m][f] = base + row * (K / VPB) + k0 / VPB + q * 16;
          wsc[m][f] = sbase + row * (K / 32) + k0 / 32 + (FP4 ? q : 0);
        }
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
        if constexpr (MX) {
          constexpr int VPB = FP4 ? 2 : 1;
          // a row block is ROWS * K / VPB code bytes and ROWS * K / 32 scale bytes in both
          // layouts; a 128-value step is 128 / VPB code bytes of a row (row-major) or a block
          // of 1 KB per load (tiled), 4 scale bytes of a row or half of a row's 8 bytes in a
          // 128-byte block.  MXFP8 takes the row's whole scale word, MXFP4 the lane's byte.
          const bool tl = a.tiled;
          const uint8_t* src = wq[m][f] + (size_t)rbi * ROWS * (K / VPB) + (size_t)ks * (tl ? 1024 * WREGS : KS / VPB);
#pragma unroll
          for (int r = 0; r < WREGS; ++r) st.w[m][f][r] = *(const u32x4*)(src + (tl ? 1024 : 64) * r);
          const size_t so = (size_t)rbi * ROWS * (K / 32) +
                            (tl ? (size_t)(ks >> 1) * 128 + (ks & 1) * 4 : (size_t)ks * (KS / 32));
          if constexpr (FP4)
            st.sc[m][f] = wsc[m][f][so];
          else
            st.sc[m][f] = *(const uint32_t*)(wsc[m][f] + so);
        } else {
#pragma unroll
          for (int s = 0; s < WREGS; ++s)
            st.w[m][f][s] = *(const u32x4*)(wp[m][f] + (size_t)rbi * ROWS * K + (size_t)ks * KS + s * 32);
        }
      }
  };
  // the 8 weights of sub-step s as bf16 (MXFP4: codes 8s .. 8s+7 of the lane's block; MXFP8:
  // bytes 8(s&1) .. +7 of its load s>>1)
  auto decode_mx = [&](const WStage<NMAT, RF, WREGS>& st, int m, int f, int s) -> u32x4 {
    if constexpr (FP4) {
      return fp4x8_to_bf16x8(st.w[m][f][0][s], e8m0_to_f32(st.sc[m][f]));
    } else {
      const float sc = e8m0_to_f32((st.sc[m][f] >> (8 * ((q >> 1) + 2 * (s >> 1)))) & 0xFFu);
      if constexpr (MODE == MODE_DOWN && HFp16<WF>::value)
        return fp8x8_to_f16x8(st.w[m][f][s >> 1][(2 * s) & 3], st.w[m][f][s >> 1][(2 * s + 1) & 3], sc);
      else
        return fp8x8_to_bf16x8(st.w[m][f][s >> 1][(2 * s) & 3], st.w[m][f][s >> 1][(2 * s + 1) & 3], sc);
    }
  };
  // the MFMA of this GEMM: fp16 for the down GEMM of MXFP8 weights (fp16 h), else bf16
  auto mm = [](const u32x4& w, const u32x4& t, floatx4 c) -> floatx4 {
    if constexpr (MODE == MODE_DOWN && HFp16<WF>::value) return mfma16_f16(w, t, c);
    else return mfma16(w, t, c);
  };
  // the k offset, within a step, of the lane's sub-step s values (both operands)
  auto kcol = [&](int s) {
    if constexpr (!MX) return s * 32 + q * 8;
    else if constexpr (FP4) return q * 32 + s * 8;
    else return q * 16 + (s & 1) * 8 + (s >> 1) * 64;
  };
  auto compute_at_use = [&](const WStage<NMAT, RF, WREGS>& st, int buf) {
    const uint16_t* L = lds + buf * NTP * BM * LROW + r16 * LROW;
#pragma unroll
    for (int s = 0; s < SUB; ++s) {
      const int col = kcol(s);
      u32x4 wf[NMAT][RF];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if constexpr (MX) {
            wf[m][f] = decode_mx(st, m, f, s);
          } else if constexpr (MODE == MODE_DOWN && HFp16<WF>::value) {
            wf[m][f] = bf16x8_to_f16x8(st.w[m][f][s]);
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
            for (int f = 0; f < RF; ++f) acc[m][f][mf] = mm(wf[m][f], tf, acc[m][f][mf]);
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
      const int col = kcol(s);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int p = 0; p < NTP; ++p) t[p][mf] = *(const u32x4*)(L + p * BM * LROW + mf * 16 * LROW + col);
    };
    // MX weights: those of sub-step s + 1 are also decoded while sub-step s multiplies
    u32x4 wf[2][NMAT][RF];
    auto weights = [&](u32x4 (&w)[NMAT][RF], int s) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int f = 0; f < RF; ++f) {
          if constexpr (MX) {
            w[m][f] = decode_mx(st, m, f, s);
          } else if constexpr (MODE == MODE_DOWN && HFp16<WF>::value) {
            w[m][f] = bf16x8_to_f16x8(st.w[m][f][s]);
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
            for (int f = 0; f < RF; ++f) acc[m][f][mf] = mm(wf[s & 1][m][f], tf[s & 1][p][mf], acc[m][f][mf]);
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
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = acc[0][f][mf][r], u = acc[NMAT - 1][f][mf][r];
              float h = g / (1.0f + __expf(-g)) * u;
              if (limit > 0.f) h = fminf(fmaxf(h, -limit), limit);
              hv[r] = h;
            }
            // h rounded once: to fp16 (bf16 and MXFP8 weights) or to bf16 (MXFP4 weights)
            if constexpr (HFp16<WF>::value)
              *(u32x2*)((uint16_t*)a.out + obase + f * 16) =
                  u32x2{pack_f16x2_sat(hv[0], hv[1]), pack_f16x2_sat(hv[2], hv[3])};
            else
              *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_bf16x2(hv[0], hv[1]), pack_bf16x2(hv[2], hv[3])};
          } else if (a.ksplit > 1) {
            *(floatx4*)(a.part + ((size_t)ksp * a.T + pos0 + j) * N + ncol + f * 16) = acc[0][f][mf];
          } else if (a.out_bf16) {
            const floatx4 v = acc[0][f][mf];
            *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          } else if (a.y16) {
            const floatx4 v = acc[0][f][mf];
            *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_f16x2_sat(v[0], v[1]), pack_f16x2_sat(v[2], v[3])};
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

// One work unit with MXFP8 activations (routed experts with MXFP4 or MXFP8 weights).  The
// token operand -- x rows gathered for gate/up, h rows for down -- is E4M3 codes with one e8m0
// scale per 32 values, staged in double-buffered LDS with its scales; each 16x16x128 product
// is one scaled MFMA (v_mfma_scale_f32_16x16x128_f8f6f4), which applies both operands' block
// scales, so no decode instruction runs.  Operand layout of that instruction (measured on
// gfx950 with one-hot operands): lane (r16, q) gives the scale of row r16's 32-value block q
// (byte 0 of its scale register); an E2M1 operand holds that block's 32 values in the lane
// (low nibble first); an E4M3 operand holds k = 16q .. 16q+15 in its first 16 bytes and
// k = 64+16q .. 64+16q+15 in its last 16.  The gate/up epilogue rounds h to
// MXFP8 along the intermediate dimension: a block of 32 rows is two 16-row fragments of one
// wave, its maximum taken over the four lane groups; down then reads the 8-bit h.
// direct global -> LDS loads of 16 or 4 bytes per lane: lane l writes l_base + size*l
// (l_base wave-uniform), counted by vmcnt like any load
__device__ __forceinline__ void a8_dma16(const void* g, void* l_base) {
  __builtin_amdgcn_global_load_lds(g, l_base, 16, 0, 0);
}
__device__ __forceinline__ void a8_dma4(const void* g, void* l_base) {
  __builtin_amdgcn_global_load_lds(g, l_base, 4, 0, 0);
}

// vmcnt wait with a compile-time count (other counters left alone)
template <int N>
__device__ __forceinline__ void a8_wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// KS = 128 * KC values per step: the KC 128-value chunks of a step are loaded together, so each
// weight row is fetched in runs of 64 * KC (E2M1) or 128 * KC (E4M3) bytes; each chunk is one
// scaled MFMA per (row block, token fragment).
template <int NW, int RF, int MF, int D, int MODE, int WF, int KS>
__device__ __forceinline__ void ffn_tile_a8(const FfnArgs& a, int e, int pos0, int nrows, int rb0, int nrb_here,
                                            uint8_t* lds) {
  constexpr int NMAT = MODE == MODE_GATEUP ? 2 : 1;
  constexpr int BM = MF * 16;
  constexpr int KC = KS / 128;                     // 128-value chunks per step
  constexpr int NST = D + 1;                       // LDS token stages: D in flight + the one read
  constexpr int SROWS = (BM + 63) / 64 * 64;       // rows per scale plane (a dword load covers 64 rows)
  constexpr int STAGE = BM * KS + KC * SROWS * 4;  // codes, then one plane of scale words per chunk
  constexpr int ROWS = NW * RF * 16;
  constexpr bool FP4 = WF == FMT_MXFP4;
  constexpr int WREGS = FP4 ? 1 : 2;               // 16-byte weight loads per (row block, chunk)
  constexpr int VPB = FP4 ? 2 : 1;                 // weight values per byte
  constexpr int AFMT = FP4 ? 4 : 0;                // scaled-MFMA operand format: 4 = E2M1, 0 = E4M3
  // token loads per step: 1 KB of codes per wave instruction, 64 scale words (one chunk) per
  // dword instruction; every wave issues the same number (small tiles repeat an instruction in
  // a second wave, writing the same bytes), so that one wait count covers every wave
  constexpr int RPI = 1024 / KS;                   // code rows per instruction
  constexpr int CODE_INSTR = BM / RPI, SCALE_INSTR = KC * (SROWS / 64);
  constexpr int NCI = (CODE_INSTR + NW - 1) / NW, NSI = (SCALE_INSTR + NW - 1) / NW;
  constexpr int NLOAD = NCI + NSI + NMAT * RF * (KC * WREGS + 1);  // loads per wave per step
  constexpr int VM_WAIT = (D - 1) * NLOAD;
  static_assert(MODE == MODE_DOWN || RF % 2 == 0, "h is rounded in 32-row blocks: two fragments per wave");
  static_assert((KC == 1 || KC == 2) && BM % RPI == 0, "steps of 128 or 256 values");
  static_assert(VM_WAIT < 64, "vmcnt range");

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r16 = lane & 15, q = lane >> 4;
  const int K = a.K, N = a.N;
  const int nsteps = K / KS;
  const int total_steps = nsteps * nrb_here;

  // token row of tile row r (r < BM): its code row and scale row; rows past the tile, or
  // positions without a token, read tile row 0's (or token 0's) and are masked in the epilogue
  auto row_src = [&](int r, bool& ok) -> int64_t {
    const int pr = r < nrows ? r : 0;
    if (MODE == MODE_GATEUP) {
      const int tok = a.sorted_token[pos0 + pr];
      ok = r < nrows && (unsigned)tok < (unsigned)a.T;
      return (unsigned)tok < (unsigned)a.T ? tok : 0;
    }
    ok = r < nrows;
    return pos0 + pr;
  };
  // codes: a row is KS / 16 chunks of 16 bytes; within each 128-byte segment chunk c sits in
  // slot c ^ (row & 7) (so the fragment reads of 8 consecutive rows fall on distinct banks).
  // Instruction i covers rows RPI*i .. RPI*i + RPI-1; lane l writes row RPI*i + l / (KS/16),
  // slot l % (KS/16), and so loads the chunk that slot holds.
  const uint8_t* csrc[NCI];
  int cdst[NCI];
#pragma unroll
  for (int k = 0; k < NCI; ++k) {
    const int ci = (wave + k * NW) % CODE_INSTR;
    const int r = ci * RPI + lane / (KS / 16), slot = lane % (KS / 16);
    bool ok;
    const int64_t row = row_src(r, ok);
    csrc[k] = a.aq + row * K + (slot >> 3) * 128 + 16 * ((slot & 7) ^ (r & 7));
    cdst[k] = ci * 1024;
  }
  // scales: plane c holds, per row, the dword of the step's chunk c (its four block scales)
  const uint8_t* ssrc[NSI];
  int sdst[NSI];
#pragma unroll
  for (int k = 0; k < NSI; ++k) {
    const int si = (wave + k * NW) % SCALE_INSTR;
    const int c = si % KC, r = (si / KC) * 64 + lane;
    bool ok;
    const int64_t row = row_src(r < BM ? r : 0, ok);
    ssrc[k] = a.as + row * (K / 32) + 4 * c;
    sdst[k] = BM * KS + c * SROWS * 4 + (si / KC) * 256;
  }
  // the epilogue's row validity (gate/up: a position without a token gets h = 0)
  bool row_ok[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) row_src(mf * 16 + r16, row_ok[mf]);

  // weights: lane group q gives the scale of block q of a chunk; E2M1 codes: block q's 16
  // bytes; E4M3 codes: bytes 16q .. 16q+15 and 64+16q .. 64+16q+15 of the chunk (the
  // instruction's layout).  Buffer loads: one resource per matrix of this expert, the lane's
  // row in a VGPR offset and the step in an SGPR offset, so a step's loads need no address
  // arithmetic per lane.
  const int nbase = rb0 * ROWS + wave * RF * 16;
  __amdgpu_buffer_rsrc_t wres[NMAT], sres[NMAT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m) {
    const uint8_t* base = (const uint8_t*)(m == 0 ? a.w0 : a.w1) + (size_t)e * N * (K / VPB);
    const uint8_t* sbase = (m == 0 ? a.s0 : a.s1) + (size_t)e * N * (K / 32);
    wres[m] = __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, N * (K / VPB), 0x00020000);
    sres[m] = __builtin_amdgcn_make_buffer_rsrc((void*)sbase, (short)0, N * (K / 32), 0x00020000);
  }
  const bool tl = a.tiled;
  int woff[RF], soff[RF];
#pragma unroll
  for (int f = 0; f < RF; ++f) {
    const int row = nbase + f * 16 + r16, b16 = (nbase + f * 16) / 16;
    woff[f] = tl ? b16 * (K / 128) * 1024 * WREGS + lane * 16 : row * (K / VPB) + q * 16;
    soff[f] = tl ? b16 * (K / 256) * 128 + r16 * 8 : row * (K / 32);
  }
  // per 128-value chunk: 128 / VPB code bytes of a row (row-major) or 1 KB per load (tiled);
  // an E4M3 operand's second 16 bytes 64 bytes on in the row or one 1 KB load on
  const int wchunk = tl ? 1024 * WREGS : 128 / VPB, whi = tl ? 1024 : 64;

  // a weight stage holds the MFMA a operands themselves (an E2M1 operand's upper half stays
  // zero) and the rows' scale words of each chunk
  struct WSt {
    i32x8 w[NMAT][RF][KC];
    uint32_t sc[NMAT][RF][KC];
  };
  floatx4 acc[NMAT][RF][MF];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int f = 0; f < RF; ++f)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) acc[m][f][mf] = floatx4{0.f, 0.f, 0.f, 0.f};

  // the issue side's position (k-step and row block of the next step to load), advanced one
  // step per issue and held at the last step once the tile is done (loads past the end repeat
  // it, into a stage and a register slot nobody reads again); no division in the loop
  int i_ks = 0, i_rb = 0, i_step = 0;
  auto advance = [&]() {
    if (i_step + 1 < total_steps) {
      ++i_step;
      if (++i_ks == nsteps) {
        i_ks = 0;
        ++i_rb;
      }
    }
  };
  auto issue_t = [&](int step) {
    uint8_t* st = lds + (step % NST) * STAGE;
#pragma unroll
    for (int k = 0; k < NCI; ++k) a8_dma16(csrc[k] + i_ks * KS, st + cdst[k]);
#pragma unroll
    for (int k = 0; k < NSI; ++k) a8_dma4(ssrc[k] + i_ks * (KS / 32), st + sdst[k]);
  };
  auto issue_w = [&](WSt& w) {
    // a row block is ROWS * K / VPB code bytes and ROWS * K / 32 scale bytes in both layouts;
    // the step's scales are 4 * KC bytes of a row, at 8 bytes per row and 256 values (tiled)
    const int wso = i_rb * ROWS * (K / VPB) + i_ks * KC * wchunk;
    const int sso = i_rb * ROWS * (K / 32) + (tl ? (KC == 2 ? i_ks * 128 : (i_ks >> 1) * 128 + (i_ks & 1) * 4)
                                                 : i_ks * (KS / 32));
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int f = 0; f < RF; ++f) {
#pragma unroll
        for (int c = 0; c < KC; ++c) {
          const u32x4 lo = __builtin_bit_cast(
              u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres[m], woff[f] + c * wchunk, wso, 0));
          w.w[m][f][c][0] = (int)lo[0];
          w.w[m][f][c][1] = (int)lo[1];
          w.w[m][f][c][2] = (int)lo[2];
          w.w[m][f][c][3] = (int)lo[3];
          if constexpr (!FP4) {
            const u32x4 hi = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(wres[m], woff[f] + c * wchunk + whi, wso, 0));
            w.w[m][f][c][4] = (int)hi[0];
            w.w[m][f][c][5] = (int)hi[1];
            w.w[m][f][c][6] = (int)hi[2];
            w.w[m][f][c][7] = (int)hi[3];
          }
        }
        // the row's block scales of the step, one word per chunk (K / 32 is a multiple of 4 * KC
        // bytes); the lane's byte is shifted down where the MFMA uses it
        if constexpr (KC == 2) {
          const auto sw = __builtin_amdgcn_raw_buffer_load_b64(sres[m], soff[f], sso, 0);
          w.sc[m][f][0] = (uint32_t)sw[0];
          w.sc[m][f][KC - 1] = (uint32_t)sw[1];
        } else {
          w.sc[m][f][0] = __builtin_amdgcn_raw_buffer_load_b32(sres[m], soff[f], sso, 0);
        }
      }
  };
  // the token fragment of (mf, chunk c) in stage `st`: row r16's codes 16q .. 16q+15 and
  // 64+16q .. 64+16q+15 of the chunk, read through the slot swizzle, and block q's scale (the
  // instruction reads byte 0 of a scale register: the lane's byte is shifted down, the bytes
  // above it are ignored)
  auto bfrag = [&](const uint8_t* st, int mf, int c) {
    const int r = mf * 16 + r16;
    const uint8_t* L = st + r * KS + c * 128;
    const u32x4 lo = *(const u32x4*)(L + 16 * (q ^ (r & 7)));
    const u32x4 hi = *(const u32x4*)(L + 16 * ((4 + q) ^ (r & 7)));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  auto bscale = [&](const uint8_t* st, int mf, int c) {
    return (int)(((const uint32_t*)(st + BM * KS + c * SROWS * 4))[mf * 16 + r16] >> (8 * q));
  };
  auto compute = [&](const WSt& w, int step) {
    const uint8_t* st = lds + (step % NST) * STAGE;
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      i32x8 bf[2];
      int bs[2];
      bf[0] = bfrag(st, 0, c);
      bs[0] = bscale(st, 0, c);
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        if (mf + 1 < MF) {  // the next fragment's LDS reads overlap this one's MFMAs
          bf[(mf + 1) & 1] = bfrag(st, mf + 1, c);
          bs[(mf + 1) & 1] = bscale(st, mf + 1, c);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int f = 0; f < RF; ++f)
            acc[m][f][mf] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                w.w[m][f][c], bf[mf & 1], acc[m][f][mf], AFMT, 0, 0, (int)(w.sc[m][f][c] >> (8 * q)), 0,
                bs[mf & 1]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // lane holds token r16 of each fragment and rows 4q .. 4q+3 of each 16-row block
  auto epilogue = [&](int rbi) {
    const int ncol0 = nbase + rbi * ROWS;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const int j = mf * 16 + r16;
      const bool keep = j < nrows;
      if constexpr (MODE == MODE_GATEUP) {
#pragma unroll
        for (int fp = 0; fp < RF / 2; ++fp) {
          float h[8];
#pragma unroll
          for (int hf = 0; hf < 2; ++hf)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = acc[0][2 * fp + hf][mf][r], u = acc[1][2 * fp + hf][mf][r];
              float v = g / (1.0f + __expf(-g)) * u;
              if (a.limit > 0.f) v = fminf(fmaxf(v, -a.limit), a.limit);
              h[4 * hf + r] = row_ok[mf] ? v : 0.f;
            }
          float am = 0.f;
#pragma unroll
          for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(h[i]));
          am = fmaxf(am, __shfl_xor(am, 16, WAVE));
          am = fmaxf(am, __shfl_xor(am, 32, WAVE));
          const int sb = mx8_scale_byte(am), X = sb - 127;
          const uint32_t c0 = mx8_pack4(h[0], h[1], h[2], h[3], X);
          const uint32_t c1 = mx8_pack4(h[4], h[5], h[6], h[7], X);
          if (keep) {
            uint8_t* dst = a.oq + (size_t)(pos0 + j) * N + ncol0 + 32 * fp + 4 * q;
            *(uint32_t*)dst = c0;
            *(uint32_t*)(dst + 16) = c1;
            if (q == 0) a.os[(size_t)(pos0 + j) * (N / 32) + (ncol0 + 32 * fp) / 32] = (uint8_t)sb;
          }
        }
      } else {
        if (keep) {
#pragma unroll
          for (int f = 0; f < RF; ++f) {
            const size_t o = (size_t)(pos0 + j) * N + ncol0 + f * 16 + 4 * q;
            const floatx4 v = acc[0][f][mf];
            if (a.y16)
              *(u32x2*)((uint16_t*)a.out + o) = u32x2{pack_f16x2_sat(v[0], v[1]), pack_f16x2_sat(v[2], v[3])};
            else
              *(floatx4*)((float*)a.out + o) = v;
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

  // prologue: steps 0 .. D-1 (tokens into stages 0 .. D-1, weights into slots 0 .. D-1)
  WSt ws[D];
#pragma unroll
  for (int j = 0; j < D; ++j)
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int f = 0; f < RF; ++f)
#pragma unroll
        for (int c = 0; c < KC; ++c) ws[j].w[m][f][c] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int j = 0; j < D; ++j) {
    issue_t(j);
    issue_w(ws[j]);
    advance();
  }
  // Step g: wait until at most VM_WAIT loads are outstanding (those of the D-1 later steps:
  // loads complete in order, so step g's tokens and weights have landed); barrier (every
  // wave's token loads of step g are in LDS, and every wave has finished reading the stage
  // that step g+D overwrites); issue step g+D's tokens; compute; issue step g+D's weights
  // into the slot compute(g) has just read; store a finished row block.  Every step issues
  // the same loads, so the count is exact; the loop is unrolled by D so slots are static.
  // A down GEMM whose reduction is exactly NST steps (intermediate 768 at 256-value steps)
  // keeps its whole h tile in the ring: the tokens are loaded during the first row block only
  // and read again for the others, whose steps issue weight loads only (the wait then counts
  // those) and need no barrier (LDS no longer changes).
  const bool resident = D == 2 && MODE == MODE_DOWN && nsteps == NST;
  constexpr int VM_WAIT_W = (D - 1) * NMAT * RF * (KC * WREGS + 1);
  const int padded_steps = (total_steps + D - 1) / D * D;
  int c_ks = 0, c_rb = 0;  // the compute side's k-step and row block
  for (int g0 = 0; g0 < padded_steps; g0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int g = g0 + j;
      const bool real = g < total_steps;
      if (resident && g + 1 >= nsteps)
        a8_wait_vmcnt<VM_WAIT_W>();  // step g+1 (the D-1 = 1 later step) loaded weights only
      else
        a8_wait_vmcnt<VM_WAIT>();
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
      if (!resident || g < nsteps) __builtin_amdgcn_s_barrier();
      if (!resident || g + D < nsteps) issue_t(g + D);
      if (real) compute(ws[j], g);
      issue_w(ws[j]);
      advance();
      if (real && ++c_ks == nsteps) {
        epilogue(c_rb);
        c_ks = 0;
        ++c_rb;
      }
    }
  }
  a8_wait_vmcnt<0>();  // no direct-to-LDS load may outlive the work unit's LDS
  __builtin_amdgcn_s_barrier();
}

// x [rows, cols] bf16 -> MXFP8 codes [rows, cols] and e8m0 scales [rows, cols/32]: one 32-value
// block per thread (64 bytes read, 33 written)
__global__ __launch_bounds__(256) void mx8_quant_kernel(const uint16_t* __restrict__ x, int64_t nblocks,
                                                        uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= nblocks) return;
  const u32x4* src = (const u32x4*)(x + i * 32);
  float v[32];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const u32x4 w = src[j];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * j + 2 * k] = __uint_as_float(w[k] << 16);
      v[8 * j + 2 * k + 1] = __uint_as_float(w[k] & 0xFFFF0000u);
    }
  }
  float am = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) am = fmaxf(am, fabsf(v[j]));
  const int sb = mx8_scale_byte(am), X = sb - 127;
  u32x4 c[2];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j >> 2][j & 3] = mx8_pack4(v[4 * j], v[4 * j + 1], v[4 * j + 2], v[4 * j + 3], X);
  ((u32x4*)(codes + i * 32))[0] = c[0];
  ((u32x4*)(codes + i * 32))[1] = c[1];
  scales[i] = (uint8_t)sb;
}

// A tile of block-format experts runs as ceil(nrows / 16) fragments of 16 positions: the
// fragments past its last token issue no loads, LDS reads or MFMAs, so an expert with n tokens
// costs ceil(n / 16) fragments rather than whole tiles (at 4096 tokens, 64-position tiles are
// 65 % occupied by tokens, their 16-position fragments 90 %).  Bf16 activations take the
// decoding kernel, MXFP8 activations the scaled MFMA.
// row-major MXFP4 codes [mats, N, Kd/2] -> tiled order: 16-byte chunk i is lane l = 16q + r of
// block (mb, s), mb = mat * N/16 + b, and takes row 16 mb + r's bytes 64s + 16q .. +15
__global__ __launch_bounds__(256) void pack_mxfp4_codes_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                               int64_t n16, int Kd) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const int l = (int)(i & 63), ns = Kd / 128;
  const int64_t blk = i >> 6, mb = blk / ns;
  const int st = (int)(blk - mb * ns);
  dst[i] = src[(mb * 16 + (l & 15)) * (Kd / 32) + st * 4 + (l >> 4)];
}

// row-major MXFP8 codes [mats, N, Kd] -> tiled order: 16-byte chunk i is lane l = 16q + r of
// half p of block (mb, s) and takes row 16 mb + r's bytes 128s + 64p + 16q .. +15
__global__ __launch_bounds__(256) void pack_mxfp8_codes_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                               int64_t n16, int Kd) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n16) return;
  const int l = (int)(i & 63), half = (int)((i >> 6) & 1), ns = Kd / 128;
  const int64_t blk = i >> 7, mb = blk / ns;
  const int st = (int)(blk - mb * ns);
  dst[i] = src[(mb * 16 + (l & 15)) * (Kd / 16) + st * 8 + half * 4 + (l >> 4)];
}

// row-major scales [mats, N, Kd/32] -> tiled order: 8-byte word i is row r = i mod 16 of block
// (mb, t) and takes row 16 mb + r's scale bytes 8t .. 8t+7
__global__ __launch_bounds__(256) void pack_mxfp4_scales_kernel(const uint64_t* __restrict__ src,
                                                                uint64_t* __restrict__ dst, int64_t n8, int Kd) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const int r = (int)(i & 15), nt = Kd / 256;
  const int64_t blk = i >> 4, mb = blk / nt;
  const int t = (int)(blk - mb * nt);
  dst[i] = src[(mb * 16 + r) * nt + t];
}

template <int NW, int RF, int MF, int D, int MODE, int FMT, int KS, int ACT, bool PADDED>
__device__ __forceinline__ void ffn_tile_mx(const FfnArgs& a, int e, int pos0, int nrows, int rb0, int nrb_here,
                                            int ksp, uint16_t* lds) {
  if constexpr (MF > 1) {
    if (nrows <= (MF - 1) * 16) {
      ffn_tile_mx<NW, RF, MF - 1, D, MODE, FMT, KS, ACT, PADDED>(a, e, pos0, nrows, rb0, nrb_here, ksp, lds);
      return;
    }
  }
  if constexpr (ACT == ACT_MXFP8)
    ffn_tile_a8<NW, RF, MF, D, MODE, FMT, KS>(a, e, pos0, nrows, rb0, nrb_here, (uint8_t*)lds);
  else
    ffn_tile<NW, RF, MF, D, MODE, KS, FMT, PADDED>(a, e, pos0, nrows, rb0, nrb_here, ksp, lds);
}

// Waves per SIMD the compiler must leave room for.  A 256-thread workgroup lets it take all 512
// registers of a lane (one wave per SIMD); the MXFP4-weight, MXFP8-activation gate/up kernel
// then held 197 VGPRs and 64 AGPRs, and at two waves per SIMD (215 VGPRs, no spill) it is 4 %
// faster at 4096 tokens.  Its MXFP8-weight twin would spill there, so it keeps the default.
template <int NW, int MODE, int FMT, int ACT>
struct FfnMinWaves {
  static constexpr int value = (ACT == ACT_MXFP8 && FMT == FMT_MXFP4 && MODE == MODE_GATEUP) ? 2 : 1;
};

template <int NW, int RF, int MF, int D, int MODE, int FMT, int KS, int ACT>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(FfnMinWaves<NW, MODE, FMT, ACT>::value)))
void ffn_kernel(FfnArgs a) {
  constexpr bool PADDED = FMT != FMT_BF16 || MF >= 4;
  constexpr int BM = MF * 16;
  constexpr int NTP = HPlanes<MODE, FMT>::value;
  // bf16 token planes (double-buffered, rows padded by 32 bytes), or for MXFP8 activations a
  // ring of D + 1 stages of codes and scale words
  constexpr int LDS_BYTES = ACT == ACT_MXFP8 ? (D + 1) * (BM * KS + (KS / 128) * ((BM + 63) / 64 * 64) * 4)
                                             : 2 * NTP * BM * (KS + 16) * 2;
  __shared__ __align__(16) uint8_t lds_raw[LDS_BYTES];
  uint16_t* lds = (uint16_t*)lds_raw;

  // device work list: work id -> (tile, sub-tile, row-block group); consecutive work ids
  // run on the same XCD.  A tile of the list holds bm_list positions and splits into
  // bm_list / BM sub-tiles of this kernel's size (empty sub-tiles exit at once).  Tile-major
  // order puts the row-block groups of a tile side by side (they share its token rows in
  // L2); group-major order, for a single weight set, the tiles of a row-block group (they
  // share its weight rows).
  const int subs = a.bm_list / BM;
  const int t_lo = a.dense || a.e_hi == 0 ? 0 : a.tile_prefix[a.e_lo];
  const int t_hi = a.dense ? (a.T + a.bm_list - 1) / a.bm_list : a.tile_prefix[a.e_hi == 0 ? a.E + a.S : a.e_hi];
  const int ntsub = (t_hi - t_lo) * subs;
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
  const int tile = t_lo + tsub / subs, sub = tsub - (tsub / subs) * subs;
  const int rb0 = grp * a.rbw, nrb_here = min(a.rbw, a.nrb - rb0);
  const int4 info = a.dense ? int4{0, tile * a.bm_list, min(a.bm_list, a.T - tile * a.bm_list), 0}
                            : ((const int4*)(a.tile_prefix + tile_info_offset(a.E)))[tile];
  const int e = info.x, m0 = sub * BM;
  if (m0 >= info.z) return;
  const int nrows = min(BM, info.z - m0);
  if constexpr (FMT != FMT_BF16) {
    // routed experts in the block format only (the bf16 shared expert runs in launches of its
    // own, so these kernels carry no bf16-weight registers)
    if (e < a.E) ffn_tile_mx<NW, RF, MF, D, MODE, FMT, KS, ACT, PADDED>(a, e, info.y + m0, nrows, rb0, nrb_here, ksp, lds);
    return;
  }
  ffn_tile<NW, RF, MF, D, MODE, KS, FMT_BF16, PADDED>(a, e, info.y + m0, nrows, rb0, nrb_here, ksp, lds);
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
// values of k per step, D steps of loads in flight.  Otherwise the down GEMM keeps two weight
// blocks per wave to halve its LDS reads per MFMA (measured when it read two h planes per
// token fragment).  16-token bf16 tiles (decode) take 256-value steps, two in flight, in 64-row
// workgroups: each weight row then goes out in 512-byte runs (measured: decode gate/up 311 ->
// 297 us, down 161 -> 159 us against 64-value steps); so does the gate/up of 32-token tiles
// (T = 1024: 683 -> 655 us; their down GEMM measured slower that way).  The down GEMM of
// 16-token tiles takes 384-value steps, so that a 768-long reduction is two steps, both in
// flight from the start (decode down 155.4 -> 153.9 us).  Where K is not a multiple of the
// step they fall back to 256-value steps (KS_MID), then to 128-value steps, four in flight
// (KS_ALT, D_ALT).
// MXFP8 activations (ACT_MXFP8): 4 waves of two 16-row blocks each (gate/up rounds h in
// blocks of 32 rows of one wave), 128-value steps.
template <int MF, int FMT, int MODE, int ACT = ACT_BF16> struct FfnCfg {
  static constexpr bool FP4 = FMT != FMT_BF16;  // MX weights (MXFP4 or MXFP8): 128-value steps
  static constexpr bool A8 = ACT == ACT_MXFP8;
  static constexpr bool DOWN = MODE == MODE_DOWN;
  static constexpr bool WIDE = !FP4 && (MF == 1 || (MF == 2 && !DOWN));
  static constexpr int NW = (MF <= 2 || DOWN || A8) ? 4 : 8;
  static constexpr int RF = WIDE ? 1 : (MF <= 2 || DOWN || A8) ? 2 : 1;
  static constexpr int KS = A8 ? 256 : FP4 ? 128 : WIDE ? ((MF == 1 && DOWN) ? 384 : 256) : 64;
  // MXFP8 activations: 256-value steps where K allows (128 otherwise), tokens in an LDS ring
  // (no registers), weights D steps ahead in registers
  static constexpr int D = A8 ? 2
                         : WIDE ? 2
                         : MF <= 2 ? (FP4 ? 3 : 4)
                         : MF == 4 ? (FP4 ? 2 : 4)
                         : MF == 8 ? (FP4 ? 2 : (DOWN ? 3 : 4))
                                   : 2;
  static constexpr int KS_MID = WIDE ? 256 : KS;  // where K is not a multiple of KS
  static constexpr int KS_ALT = (WIDE || A8) ? 128 : KS, D_ALT = WIDE ? 4 : D;
};

template <int MF, int MODE, int FMT, int ACT = ACT_BF16>
hipError_t launch_one(FfnArgs a, int rbw, int64_t max_tiles, hipStream_t s, Tracer* tr, const char* name = nullptr) {
  using C = FfnCfg<MF, FMT, MODE, ACT>;
  if (ACT == ACT_MXFP8 && (a.ksplit != 1 || a.dense)) return hipErrorInvalidValue;
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
    launch(tr, ffn_kernel<C::NW, C::RF, MF, C::D, MODE, FMT, C::KS, ACT>, dim3((unsigned)grid), dim3(C::NW * 64), s,
           a);
  else if (ACT == ACT_BF16 && C::KS_MID != C::KS && kspan % C::KS_MID == 0)
    launch(tr, ffn_kernel<C::NW, C::RF, MF, C::D, MODE, FMT, C::KS_MID, ACT>, dim3((unsigned)grid),
           dim3(C::NW * 64), s, a);
  else if (C::KS_ALT != C::KS && kspan % C::KS_ALT == 0)
    launch(tr, ffn_kernel<C::NW, C::RF, MF, C::D_ALT, MODE, FMT, C::KS_ALT, ACT>, dim3((unsigned)grid),
           dim3(C::NW * 64), s, a);
  else
    return hipErrorInvalidValue;
  hipError_t err = hipGetLastError();
  if (tr) tr->mark(name ? name : MODE == MODE_GATEUP ? "expert_gate_up" : "expert_down", s);
  return err;
}

template <int MODE>
hipError_t launch_mode(int mf, const FfnArgs& a, int rbw, int fmt, int64_t max_tiles, hipStream_t s, Tracer* tr,
                       int act = ACT_BF16, const char* name = nullptr) {
  if (act == ACT_MXFP8) {
#define MOE_A8(F)                                                                    \
  switch (mf) {                                                                      \
    case 1: return launch_one<1, MODE, F, ACT_MXFP8>(a, rbw, max_tiles, s, tr, name);     \
    case 2: return launch_one<2, MODE, F, ACT_MXFP8>(a, rbw, max_tiles, s, tr, name);     \
    case 4: return launch_one<4, MODE, F, ACT_MXFP8>(a, rbw, max_tiles, s, tr, name);     \
    case 8: return launch_one<8, MODE, F, ACT_MXFP8>(a, rbw, max_tiles, s, tr, name);     \
    default: return hipErrorInvalidValue;                                            \
  }
    if (fmt == FMT_MXFP4) MOE_A8(FMT_MXFP4)
    if (fmt == FMT_MXFP8) MOE_A8(FMT_MXFP8)
#undef MOE_A8
    return hipErrorInvalidValue;  // MXFP8 activations need block-format weights
  }
  if (fmt == FMT_MXFP4) {
    switch (mf) {
      case 1: return launch_one<1, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      case 2: return launch_one<2, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      case 4: return launch_one<4, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      case 8: return launch_one<8, MODE, FMT_MXFP4>(a, rbw, max_tiles, s, tr);
      default: return hipErrorInvalidValue;  // the plan never picks 16 for MX weights
    }
  }
  if (fmt == FMT_MXFP8) {
    switch (mf) {
      case 1: return launch_one<1, MODE, FMT_MXFP8>(a, rbw, max_tiles, s, tr);
      case 2: return launch_one<2, MODE, FMT_MXFP8>(a, rbw, max_tiles, s, tr);
      case 4: return launch_one<4, MODE, FMT_MXFP8>(a, rbw, max_tiles, s, tr);
      case 8: return launch_one<8, MODE, FMT_MXFP8>(a, rbw, max_tiles, s, tr);
      default: return hipErrorInvalidValue;
    }
  }
  switch (mf) {
    case 1: return launch_one<1, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr, name);
    case 2: return launch_one<2, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr, name);
    case 4: return launch_one<4, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr, name);
    case 8: return launch_one<8, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr, name);
    default: return launch_one<16, MODE, FMT_BF16>(a, rbw, max_tiles, s, tr, name);
  }
}

}  // namespace

// The shared expert of a block-format layer runs as a dense FFN over all T tokens (one bf16
// weight set): tiles of 16 * mf tokens growing with T, the tiles of a row block side by side
// up to 512 tokens (measured at 4096 tokens, hidden 2560, intermediate 768: 128-token tiles
// take 0.067 ms for gate/up, 64-token tiles 0.101 ms)
SharedPlan shared_plan(int64_t T) {
  SharedPlan sp;
  sp.mf = T <= 32 ? 1 : T <= 128 ? 2 : T <= 512 ? 4 : 8;
  sp.mf_down = std::min(sp.mf, 4);
  sp.group_major = T <= 512 ? 1 : 0;
  sp.tiles = (T + 16 * sp.mf - 1) / (16 * sp.mf);
  return sp;
}

FfnPlan ffn_plan(int64_t T, int K, int E, int S, int fmt, int H, int I) {
  FfnPlan p;
  p.topk = K;
  const double avg = (double)T * K / E;  // routed tokens per expert on average
  // tile list of 16*mf positions; gate/up runs whole tiles, down runs sub-tiles of 16*mf_down
  // (measured when the down GEMM read two h planes: it is fastest with 64-token tiles at
  // two waves per SIMD; gate/up with 128, or 256 when experts average well above 128 tokens;
  // MXFP4 experts with up to 96 tokens on average take 64-token tiles: at 64 per expert,
  // gate/up 0.694 -> 0.731 ms but down 0.606 -> 0.548 ms)
  const bool mx = fmt != FMT_BF16;  // MXFP8 weights take the MXFP4 tile sizes
  p.mf = avg <= 12 ? 1 : avg <= 24 ? 2 : (avg <= 48 || (mx && avg <= 96)) ? 4
       : (avg <= 192 || mx) ? 8 : 16;
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
  // (block-format experts at 4096 tokens: 2 and 4, measured against 3 and 5: gate/up 0.518 ->
  // 0.499 ms with bf16 activations, 0.381 -> 0.364 with MXFP8 ones; down 0.251 -> 0.242 with MXFP8)
  p.rbw_gate_up = p.mf >= 4 ? (mx ? 2 : 3) : 1;
  p.rbw_down = p.mf >= 4 ? (mx ? 4 : 5) : 1;  // decode: one row block per workgroup (measured)
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
                             float limit, float shared_limit, uint16_t* h, float* y,
                             bool tiles_ready, hipStream_t s, Tracer* tr, const ActBufs* ab, bool own_shared,
                             hipStream_t shared_s, bool y16) {
  hipError_t err = hipSuccess;
  const bool a8 = ab && ab->act == ACT_MXFP8;
  if (a8 && (p.tiles || w.fmt == FMT_BF16 || !ab->xq || !ab->xs || !ab->hq || !ab->hs)) return hipErrorInvalidValue;
  if (p.tiles) {
    if (!tiles_ready) {
      launch(tr, tile_prefix_kernel, dim3(1), dim3(64), s, offsets, E + S, p.bm, tile_prefix, tile_info_offset(E));
      err = hipGetLastError();
      if (tr) tr->mark("expert_tiles", s);
      if (err != hipSuccess) return err;
    }
    return launch_expert_ffn_tiles(x, offsets, sorted_token, tile_prefix, p.max_tiles, w, T, H, I, E, S, limit,
                                   shared_limit, h, y, s, tr, y16);
  }
  if (!tiles_ready) {
    launch(tr, tile_prefix_kernel, dim3(1), dim3(64), s, offsets, E + S, p.bm, tile_prefix, tile_info_offset(E));
    err = hipGetLastError();
    if (tr) tr->mark("expert_tiles", s);
  }
  if (err != hipSuccess) return err;
  if (a8) {
    // x rounded to MXFP8 once for all routed experts (the shared expert reads x as bf16)
    const int64_t nblocks = (int64_t)T * H / 32;
    launch(tr, mx8_quant_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), s, x, nblocks, ab->xq, ab->xs);
    err = hipGetLastError();
    if (tr) tr->mark("act_quant", s);
    if (err != hipSuccess) return err;
  }

  FfnArgs gu{};
  gu.act = x; gu.sorted_token = sorted_token; gu.offsets = offsets; gu.tile_prefix = tile_prefix;
  gu.w0 = w.gate; gu.w1 = w.up; gu.s0 = w.gate_scale; gu.s1 = w.up_scale;
  gu.sw0 = w.sh_gate; gu.sw1 = w.sh_up; gu.out = h;
  gu.T = T; gu.E = E; gu.S = S; gu.K = H; gu.N = I;
  gu.limit = limit; gu.shared_limit = shared_limit;
  gu.ksplit = 1;
  gu.y16 = 0;

  FfnArgs dn = gu;
  dn.act = h; dn.sorted_token = nullptr;
  dn.w0 = w.down; dn.w1 = nullptr; dn.s0 = w.down_scale; dn.s1 = nullptr;
  dn.sw0 = w.sh_down; dn.sw1 = nullptr; dn.out = y;
  dn.K = I; dn.N = H;
  dn.y16 = y16 ? 1 : 0;

  gu.bm_list = dn.bm_list = p.bm;
  gu.group_major = dn.group_major = p.group_major ? 1 : 0;
  if (w.fmt == FMT_BF16) {  // bf16 weights: the shared expert is one more expert of the same launches
    err = launch_mode<MODE_GATEUP>(p.mf_gate_up, gu, p.rbw_gate_up, w.fmt, p.max_tiles, s, tr);
    if (err != hipSuccess) return err;
    return launch_mode<MODE_DOWN>(p.mf_down, dn, p.rbw_down, w.fmt, p.max_tiles, s, tr);
  }
  // block-format weights: the routed experts on the MX kernels (with MXFP8 activations, the
  // scaled-MFMA ones), restricted to their tiles, so that they carry no bf16-weight registers;
  // the shared expert (bf16 weights and activations) on the bf16 kernels as a dense FFN over
  // all T tokens, whose block of sorted positions is the identity at T*K (so its tile size
  // follows from T, not from the routed experts' tokens).  It reads x only, so the caller may
  // give it a stream of its own (own_shared, shared_s) that runs beside the routing and the
  // routed experts; the launches keep their order in the tracer's count either way.
  const hipStream_t ss = own_shared ? shared_s : s;
  const int act = a8 ? ACT_MXFP8 : ACT_BF16;
  FfnArgs gu_s = gu, dn_s = dn;
  if (a8) {
    gu.aq = ab->xq; gu.as = ab->xs; gu.oq = ab->hq; gu.os = ab->hs;
    dn.aq = ab->hq; dn.as = ab->hs;
  }
  gu.e_lo = dn.e_lo = 0;
  gu.e_hi = dn.e_hi = E;
  gu.tiled = dn.tiled = w.tiled;
  const int64_t sh_tiles = S ? ((int64_t)T + p.bm - 1) / p.bm : 0;
  err = launch_mode<MODE_GATEUP>(p.mf_gate_up, gu, p.rbw_gate_up, w.fmt, p.max_tiles - sh_tiles, s, tr, act);
  if (err != hipSuccess) return err;
  const SharedPlan sp = shared_plan(T);
  const size_t pos = (size_t)T * (size_t)p.topk;  // the shared expert's first sorted position
  if (S) {
    gu_s.act = x; gu_s.sorted_token = nullptr; gu_s.offsets = nullptr; gu_s.tile_prefix = nullptr;
    gu_s.w0 = w.sh_gate; gu_s.w1 = w.sh_up; gu_s.s0 = gu_s.s1 = nullptr;
    gu_s.out = h + pos * I;
    gu_s.E = 1; gu_s.S = 0; gu_s.limit = shared_limit;
    gu_s.dense = 1; gu_s.bm_list = 16 * sp.mf; gu_s.group_major = sp.group_major;
    err = launch_mode<MODE_GATEUP>(sp.mf, gu_s, 1, FMT_BF16, sp.tiles, ss, tr, ACT_BF16, "expert_gate_up_shared");
    if (err != hipSuccess) return err;
  }
  // (MXFP4 weights with bf16 activations read one h plane, so their down GEMM keeps the
  // plan's tiles: measured at 4096 tokens, 0.270 ms with 64-token tiles against 0.304 with
  // 32-token ones, and 0.312 with 32-token tiles of four 16-row blocks per wave, the shape that
  // was fastest with two planes)
  err = launch_mode<MODE_DOWN>(p.mf_down, dn, p.rbw_down, w.fmt, p.max_tiles - sh_tiles, s, tr, act);
  if (err != hipSuccess || !S) return err;
  dn_s.act = h + pos * I;
  dn_s.w0 = w.sh_down; dn_s.s0 = nullptr;
  dn_s.out = y16 ? (void*)((uint16_t*)y + pos * H) : (void*)(y + pos * H);
  dn_s.E = 1; dn_s.S = 0; dn_s.limit = shared_limit;
  dn_s.dense = 1; dn_s.out_bf16 = 0; dn_s.bm_list = 16 * sp.mf; dn_s.group_major = sp.group_major;
  return launch_mode<MODE_DOWN>(sp.mf_down, dn_s, 1, FMT_BF16, sp.tiles, ss, tr, ACT_BF16, "expert_down_shared");
}

hipError_t launch_pack_mx(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t mats, int N, int Kd,
                          uint8_t* codes_out, uint8_t* scales_out, hipStream_t s) {
  if ((fmt != FMT_MXFP4 && fmt != FMT_MXFP8) || mats < 0 || N <= 0 || N % 16 || Kd <= 0 || Kd % 256)
    return hipErrorInvalidValue;
  const int vpb = fmt == FMT_MXFP4 ? 2 : 1;
  const int64_t n16 = mats * N * (int64_t)(Kd / vpb / 16), n8 = mats * N * (int64_t)(Kd / 256);
  if (n16 == 0) return hipSuccess;
  if (fmt == FMT_MXFP4)
    hipLaunchKernelGGL(pack_mxfp4_codes_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       (const u32x4*)codes, (u32x4*)codes_out, n16, Kd);
  else
    hipLaunchKernelGGL(pack_mxfp8_codes_kernel, dim3((unsigned)((n16 + 255) / 256)), dim3(256), 0, s,
                       (const u32x4*)codes, (u32x4*)codes_out, n16, Kd);
  hipLaunchKernelGGL(pack_mxfp4_scales_kernel, dim3((unsigned)((n8 + 255) / 256)), dim3(256), 0, s,
                     (const uint64_t*)scales, (uint64_t*)scales_out, n8, Kd);
  return hipGetLastError();
}

hipError_t launch_mx8_quant(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales, hipStream_t s) {
  if (cols % 32 || rows < 0) return hipErrorInvalidValue;
  const int64_t nblocks = rows * cols / 32;
  if (nblocks == 0) return hipSuccess;
  hipLaunchKernelGGL(mx8_quant_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s, x, nblocks, codes,
                     scales);
  return hipGetLastError();
}

hipError_t launch_dense_ffn_tiled(const FfnPlan& p, const uint16_t* x, const uint16_t* gate, const uint16_t* up,
                                  const uint16_t* down, int T, int H, int I, float limit, uint16_t* h,
                                  float* part, uint16_t* out, hipStream_t s) {
  if (p.tiles) return hipErrorInvalidValue;  // the 256-position tile kernel reads the dispatch arrays
  if (p.ksplit_down > 1 && !part) return hipErrorInvalidValue;
  FfnArgs gu{};
  gu.act = x; gu.w0 = gate; gu.w1 = up; gu.out = h;
  gu.T = T; gu.E = 1; gu.S = 0; gu.K = H; gu.N = I;
  gu.limit = limit;
  gu.bm_list = p.bm;
  gu.group_major = p.group_major ? 1 : 0;
  gu.dense = 1;
  gu.ksplit = 1;
  FfnArgs dn = gu;
  dn.act = h; dn.w0 = down; dn.w1 = nullptr; dn.out = out;
  dn.K = I; dn.N = H;
  dn.out_bf16 = 1;
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
