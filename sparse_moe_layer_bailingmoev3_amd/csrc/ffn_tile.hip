// Expert FFNs for many tokens per expert (prefill): grouped GEMM with 128/256-token tiles.
//
// Same mathematics as ffn.hip (the SwiGLU experts of the routing walk-through page, lqnn.cn,
// section 二, clamp of section 四); a different decomposition for the regime where each
// expert serves ~100-300 tokens and the kernel must keep a deep HBM weight stream in flight
// beside the MFMA work:
//   * a workgroup (8 waves) owns a tile of up to BM = 16*TPW*8 sorted positions of one
//     expert; wave w owns 16*TPW of them and all rows of the current row block
//     (128 gate + 128 up rows, or 256 down rows), so each weight byte is read from HBM once
//     per workgroup;
//   * weights, which every wave uses, move through an NSTAGE-deep ring in LDS with direct
//     global->LDS loads; a wave's token values, used by that wave only, go straight into
//     registers in MFMA operand layout, into a ring of NSTAGE-1 register slots.  Step s
//     issues both for step s+NSTAGE-1, so NSTAGE-1 steps of weights are always in flight
//     while LDS holds weights only;
//   * every step issues the same loads (past the end they repeat a valid address into a
//     slot that is not read again), so one exact vmcnt wait covers step s's weights and
//     tokens: vector memory loads complete in issue order;
//   * LDS rows are 128 bytes with the 16-byte chunks XOR-swizzled by (row >> 1) & 7, which
//     keeps the MFMA fragment reads free of bank conflicts;
//   * MFMA sub-step u takes k = 32u + 8q .. +7 for lane group q in both operands;
//   * the SwiGLU activation h passes from gate/up to down as one fp16 plane (11 significant
//     bits, as in the few-token kernels with bf16 weights): the down GEMM converts each
//     LDS stage of bf16 weights to fp16 in place once it has landed (each chunk by one lane,
//     then a second barrier; exact for these weights) and multiplies on the fp16 MFMA, at
//     the bf16 rate, so h costs half the bytes and half the MFMAs.
#include "moe_common.h"
#include "moe_internal.h"

namespace moe {

namespace {

constexpr int TM_GATEUP = 0, TM_DOWN = 1;
constexpr int T_NW = 8;            // waves per workgroup
constexpr int T_KS = 64;           // k per step
constexpr int T_ROWB = T_KS * 2;   // bytes of one row (weight or token) per stage
constexpr int T_LIST_BM = 256;     // positions per tile of the device tile list

struct TileArgs {
  const uint16_t* act;          // gate/up: x [T,K] bf16; down: h [P,K] fp16
  const int32_t* sorted_token;  // gate/up: token of each sorted position
  const int32_t* offsets;       // [E+2]
  const int32_t* tile_prefix;   // [E+2] tiles of 256 positions before expert e
  const uint16_t* w0;           // routed gate (gate/up) or down, bf16
  const uint16_t* w1;           // routed up (gate/up)
  const uint16_t* sw0;          // shared expert gate or down
  const uint16_t* sw1;          // shared expert up
  void* out;                    // gate/up: h fp16 [P,N]; down: y fp32 (fp16 with y16) [P,N]
  int T, E, S;
  int K, N;                     // reduction length, output columns per expert
  int nrb;                      // row blocks per expert (N / rows of one block)
  int rbw;                      // row blocks per workgroup
  int ngroups;                  // ceil(nrb / rbw)
  int interleave;               // 1: sub-tile t on XCD t mod 8; 0: contiguous item ranges per XCD
  int y16;                      // down: y as fp16 [P,N] (saturated at +-65504) instead of fp32
  float limit, shared_limit;
};

__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0), vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
}

// 16 bytes per lane, global -> LDS: lane l writes l_base + 16*l (l_base wave-uniform).  Kept in
// a device function: called straight from the kernel's lambdas, the builtin made the host pass
// drop the kernel's launch stub without any diagnostic.
__device__ __forceinline__ void lds_dma16(const void* g, void* l_base) {
  __builtin_amdgcn_global_load_lds(g, l_base, 16, 0, 0);
}

__device__ __forceinline__ int swz(int row) { return (row >> 1) & 7; }

// two fp32 -> two fp16, round to nearest even, low half first
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) | ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}


// vmcnt wait with a compile-time count (other counters left alone)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Loads through the scalar data cache (uniform addresses of data the kernel never writes):
// they are counted by lgkmcnt, so fetching the next work item never waits on the vector
// memory pipeline that streams the weights.
typedef const __attribute__((address_space(4))) int32_t* sptr;

template <int MODE, int RFR, int TPW, int NSTAGE>
__global__ __launch_bounds__(T_NW * 64) void ffn_tile_kernel(TileArgs a) {
  constexpr int NMAT = MODE == TM_GATEUP ? 2 : 1;
  constexpr int NTP = 1;  // token planes: x (gate/up) or the fp16 h (down)
  constexpr int BM = T_NW * TPW * 16;              // positions per work item
  constexpr int WROWS = NMAT * RFR * 16;           // weight rows per stage
  constexpr int W_BYTES = WROWS * T_ROWB;
  constexpr int W_DMA = W_BYTES / (T_NW * 1024);   // 1 KB per wave instruction
  static_assert(W_DMA * T_NW * 1024 == W_BYTES, "weight stage must split evenly over waves");
  static_assert((W_DMA * 8) % (RFR * 16) == 0 || (RFR * 16) % (W_DMA * 8) == 0, "a wave's rows in one matrix");
  constexpr int D = NSTAGE - 1;                    // prefetch distance in steps
  constexpr int NLOAD = W_DMA + NTP * TPW * 2;     // loads per wave per step
  constexpr int VM_WAIT = (D - 1) * NLOAD;         // loads issued after step g's tokens
  static_assert(VM_WAIT < 64, "vmcnt range");
  constexpr int SUBS = T_LIST_BM / BM;
  __shared__ __align__(16) uint8_t lds[NSTAGE * W_BYTES];

  const sptr tile_prefix = (sptr)a.tile_prefix;
  const sptr offsets = (sptr)a.offsets;
  const sptr sorted_token = (sptr)a.sorted_token;

  // ---- this workgroup's work items: sub-tile t belongs to XCD t mod 8 (blockIdx mod 8), so
  // every XCD gets an even share of the experts, the shared expert's tiles included; an
  // XCD's workgroups take its (sub-tile, row-block group) items round-robin, so the groups of
  // one sub-tile run side by side in that XCD's L2
  const int ntsub = tile_prefix[a.E + a.S] * SUBS;
  const int xcd = blockIdx.x & 7;
  const int slots = gridDim.x >> 3;
  const int per_xcd = (ntsub * a.ngroups + 7) >> 3;
  int wi = blockIdx.x >> 3;  // item index within this XCD's list

  const int K = a.K, N = a.N;
  const int nsteps = K / T_KS;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r16 = lane & 15, q = lane >> 4;

  struct Item { int e, pos0, nrows, rb0, steps; };
  // the next work item at or after wi that holds positions (empty sub-tiles are skipped)
  auto next_item = [&](Item& it) -> bool {
    for (;; wi += slots) {
      int tsub, grp;
      if (a.interleave) {
        const int tl = wi / a.ngroups;
        grp = wi - tl * a.ngroups;
        tsub = tl * 8 + xcd;
        if (tsub >= ntsub) return false;
      } else {
        if (wi >= per_xcd) return false;
        const int id = xcd * per_xcd + wi;
        tsub = id / a.ngroups;
        grp = id - tsub * a.ngroups;
        if (tsub >= ntsub) return false;
      }
      const int tile = tsub / SUBS, sub = tsub - tile * SUBS;
      int lo = 0, hi = a.E + a.S;
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (tile_prefix[mid] <= tile) lo = mid; else hi = mid;
      }
      const int m0 = (tile - tile_prefix[lo]) * T_LIST_BM + sub * BM;
      const int p0 = offsets[lo], cnt = offsets[lo + 1] - p0;
      if (m0 < cnt) {
        it.e = lo;
        it.pos0 = p0 + m0;
        it.nrows = min(BM, cnt - m0);
        it.rb0 = grp * a.rbw;
        it.steps = min(a.rbw, a.nrb - it.rb0) * nsteps;
        return true;
      }
    }
  };

  // ---- issue side: the item whose loads are being issued, D steps ahead of the compute side
  Item iss;
  if (!next_item(iss)) return;
  int isn = 0;              // step of `iss` issued next
  bool iss_live = true;     // false once this workgroup has no further item (then the last
                            // step's loads are repeated, into stages nobody reads)
  // weight sources: lane l of an instruction covering rows R0..R0+7 writes row R0 + l/8,
  // slot l%8, which holds chunk (l%8) ^ swz(row) of that row
  const uint16_t* wsrc[W_DMA];
  int wdst[W_DMA];
  // token sources: lane (r16, q) of fragment tf reads position j = its row, values
  // k0 + 32u + 8q .. +7 (sub-step u).  Rows past the tile's end, or positions that hold no
  // token, read the tile's first row; gate/up stores h = 0 for positions without a token.
  const uint16_t* tsrc[NTP][TPW];
  bool tok_new[TPW];        // per-position validity of the item just taken by the issue side
  auto set_sources = [&](const Item& it) {
    const bool sh = it.e == a.E;
#pragma unroll
    for (int i = 0; i < W_DMA; ++i) {
      const int R0 = (wave * W_DMA + i) * 8;
      const int r = R0 + (lane >> 3);
      const int m = R0 / (RFR * 16), rr = r - m * (RFR * 16);  // m is uniform
      const uint16_t* b = sh ? (m == 0 ? a.sw0 : a.sw1) : (m == 0 ? a.w0 : a.w1) + (size_t)it.e * N * K;
      wsrc[i] = b + (size_t)(it.rb0 * RFR * 16 + rr) * K + ((lane & 7) ^ swz(r)) * 8;
      wdst[i] = R0 * T_ROWB;
    }
#pragma unroll
    for (int tf = 0; tf < TPW; ++tf) {
      const int j0 = wave * TPW * 16 + tf * 16;
      const int j = j0 + r16;
      if (MODE == TM_GATEUP) {
        int tok = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int t = sorted_token[it.pos0 + min(j0 + i, it.nrows - 1)];
          tok = r16 == i ? t : tok;
        }
        const bool ok = j < it.nrows && (unsigned)tok < (unsigned)a.T;
        tok_new[tf] = ok;
        tsrc[0][tf] = a.act + (size_t)(ok ? tok : 0) * K + q * 8;
      } else {
        tok_new[tf] = true;
        tsrc[0][tf] = a.act + (size_t)(it.pos0 + (j < it.nrows ? j : 0)) * K + q * 8;
      }
    }
  };
  set_sources(iss);

  // ---- compute side
  Item cmp = iss, nxt = iss;
  bool tok_ok[TPW], tok_nxt[TPW];
#pragma unroll
  for (int tf = 0; tf < TPW; ++tf) tok_ok[tf] = tok_nxt[tf] = tok_new[tf];
  bool nxt_valid = false;
  int csn = 0;              // step of `cmp` computed next
  bool cmp_live = true;

  u32x4 tk[D][NTP][TPW][2];  // token ring: slot j holds the steps g with g mod D == j

  // loads of global step g (weights into stage g mod NSTAGE) for (iss, isn)
  auto issue_w = [&](int g) {
    const int rbi = isn / nsteps, ks = isn - rbi * nsteps;
    uint8_t* st = lds + (g % NSTAGE) * W_BYTES;
#pragma unroll
    for (int i = 0; i < W_DMA; ++i)
      lds_dma16(wsrc[i] + (size_t)rbi * RFR * 16 * K + ks * T_KS, st + wdst[i]);
  };
  auto issue_t = [&](u32x4 (&dst)[NTP][TPW][2]) {
    const int ks = isn % nsteps;
#pragma unroll
    for (int p = 0; p < NTP; ++p)
#pragma unroll
      for (int tf = 0; tf < TPW; ++tf)
#pragma unroll
        for (int u = 0; u < 2; ++u) dst[p][tf][u] = *(const u32x4*)(tsrc[p][tf] + ks * T_KS + u * 32);
  };
  // at a chunk boundary: when the issue side has finished its item, move it to the next one
  // (item lengths are multiples of D, so items start and end on chunk boundaries)
  // (called after the compute side has taken any pending item, so `nxt` is free here)
  auto switch_issue = [&]() {
    if (!iss_live || isn < iss.steps) return;
    wi += slots;
    Item it;
    if (next_item(it)) {
      iss = it;
      isn = 0;
      set_sources(iss);
      nxt = it;
      nxt_valid = true;
#pragma unroll
      for (int tf = 0; tf < TPW; ++tf) tok_nxt[tf] = tok_new[tf];
    } else {
      iss_live = false;
      isn = iss.steps - 1;
    }
  };

  floatx4 acc[NMAT][RFR][TPW];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int f = 0; f < RFR; ++f)
#pragma unroll
      for (int tf = 0; tf < TPW; ++tf) acc[m][f][tf] = floatx4{0.f, 0.f, 0.f, 0.f};

  // One step's MFMAs.  The 2*NMAT*RFR weight fragments (sub-step u, matrix m, row block f)
  // are read from LDS FPF fragments ahead of their MFMAs; the scheduling barriers keep the
  // compiler from sinking those reads next to their use, so the LDS latency overlaps the
  // MFMAs of the fragments before.
  constexpr int NF = NMAT * RFR;
  constexpr int FPF = 8;  // ~256 MFMA cycles between a read and its use
  auto compute = [&](int g, const u32x4 (&tv)[NTP][TPW][2]) {
    const uint8_t* st = lds + (g % NSTAGE) * W_BYTES;
    auto frag = [&](int idx) {
      const int u = idx / NF, fi = idx - u * NF;
      const int r = fi * 16 + r16;
      return *(const u32x4*)(st + r * T_ROWB + (((4 * u + q) ^ swz(r)) << 4));
    };
    u32x4 wf[FPF + 1];
#pragma unroll
    for (int i = 0; i < FPF; ++i) wf[i] = frag(i);
#pragma unroll
    for (int idx = 0; idx < 2 * NF; ++idx) {
      if (idx + FPF < 2 * NF) wf[(idx + FPF) % (FPF + 1)] = frag(idx + FPF);
      __builtin_amdgcn_sched_barrier(0);
      const int u = idx / NF, fi = idx - u * NF;
      const int m = fi / RFR, f = fi - m * RFR;
      if constexpr (MODE == TM_GATEUP) {
#pragma unroll
        for (int tf = 0; tf < TPW; ++tf) acc[m][f][tf] = mfma16(wf[idx % (FPF + 1)], tv[0][tf][u], acc[m][f][tf]);
      } else {
        // down: the weights, already converted to fp16 in the stage, against the fp16 h
#pragma unroll
        for (int tf = 0; tf < TPW; ++tf) acc[m][f][tf] = mfma16_f16(wf[idx % (FPF + 1)], tv[0][tf][u], acc[m][f][tf]);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // down: stage g's bf16 weights -> fp16 in place (exact from 2^-17 up to 65504, which holds
  // bf16 model weights); the chunks of a stage are spread over all lanes of the workgroup
  auto convert_stage = [&](int g) {
    constexpr int CH = W_BYTES / 16 / (T_NW * 64);  // 16-byte chunks per lane
    static_assert(CH * 16 * T_NW * 64 == W_BYTES, "a stage must split evenly over the lanes");
    uint8_t* st = lds + (g % NSTAGE) * W_BYTES;
    u32x4 v[CH];
#pragma unroll
    for (int c = 0; c < CH; ++c) v[c] = *(const u32x4*)(st + (c * T_NW * 64 + threadIdx.x) * 16);
#pragma unroll
    for (int c = 0; c < CH; ++c) *(u32x4*)(st + (c * T_NW * 64 + threadIdx.x) * 16) = bf16x8_to_f16x8(v[c]);
  };

  auto epilogue = [&](int rbi) {
    const float limit = cmp.e == a.E ? a.shared_limit : a.limit;
    const int ncol = (cmp.rb0 + rbi) * RFR * 16 + 4 * q;
#pragma unroll
    for (int tf = 0; tf < TPW; ++tf) {
      const int j = wave * TPW * 16 + tf * 16 + r16;
      if (j < cmp.nrows) {
        const size_t obase = (size_t)(cmp.pos0 + j) * N + ncol;
#pragma unroll
        for (int f = 0; f < RFR; ++f) {
          if (MODE == TM_GATEUP) {
            // h in fp16, one plane: 11 significant bits (bf16 keeps 8); saturated at the fp16
            // maximum, which the clamp of the deep layers and these activations stay far below
            float hv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const float g = acc[0][f][tf][r], uu = acc[NMAT - 1][f][tf][r];
              float h = g / (1.0f + __expf(-g)) * uu;
              if (limit > 0.f) h = fminf(fmaxf(h, -limit), limit);
              if (!tok_ok[tf]) h = 0.f;
              hv[r] = fminf(fmaxf(h, -65504.f), 65504.f);
            }
            *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_f16x2(hv[0], hv[1]), pack_f16x2(hv[2], hv[3])};
          } else if (a.y16) {
            // y in fp16 (11 significant bits), saturated like h
            float yv[4];
#pragma unroll
            for (int r = 0; r < 4; ++r) yv[r] = fminf(fmaxf(acc[0][f][tf][r], -65504.f), 65504.f);
            *(u32x2*)((uint16_t*)a.out + obase + f * 16) = u32x2{pack_f16x2(yv[0], yv[1]), pack_f16x2(yv[2], yv[3])};
          } else {
            *(floatx4*)((float*)a.out + obase + f * 16) = acc[0][f][tf];
          }
        }
      }
    }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int f = 0; f < RFR; ++f)
#pragma unroll
        for (int tf = 0; tf < TPW; ++tf) acc[m][f][tf] = floatx4{0.f, 0.f, 0.f, 0.f};
  };

  // ---- prologue: global steps 0 .. D-1 into token slots 0 .. D-1
#pragma unroll
  for (int j = 0; j < D; ++j) {
    issue_w(j);
    issue_t(tk[j]);
    if (iss_live) ++isn;
  }
  switch_issue();

  // ---- main loop over this workgroup's steps (all its items back to back) in chunks of D
  // steps, unrolled so that the token slot of every step is static and every step issues its
  // loads unconditionally (the compiler's own wait counting then agrees with the waits
  // below).  Step g: wait until at most VM_WAIT loads are outstanding (those of the D-1
  // later steps), which means step g's weights and tokens have landed (loads complete in
  // order; output stores, which may complete out of order, only ever make the wait
  // stricter); barrier (every wave's weight loads for g are in, and every wave has finished
  // reading the stage that step g+D overwrites); issue step g+D's weights; compute; issue
  // step g+D's tokens into the slot compute(g) has just read; after the last step of a row
  // block, store it.  Items switch between chunks.
  for (int g0 = 0; cmp_live; g0 += D) {
    const bool active = wave * TPW * 16 < cmp.nrows;  // wave-uniform
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int g = g0 + j;
      wait_vmcnt<VM_WAIT>();
      lds_barrier();
      issue_w(g + D);
      if constexpr (MODE == TM_DOWN) {
        // the stage's bf16 weights become fp16 in place, each 16-byte chunk converted once by
        // one lane (not by every wave that reads it), before any wave reads them
        convert_stage(g);
        lds_barrier();
      }
      if (active) compute(g, tk[j]);
      issue_t(tk[j]);
      if (iss_live) ++isn;
      if ((csn + 1) % nsteps == 0 && active) epilogue(csn / nsteps);
      ++csn;
    }
    // the compute side takes the pending item before the issue side may replace it: the
    // issue side runs exactly one chunk ahead, so an item it took at the end of the previous
    // chunk is the one compute starts now, and an item of D steps makes the issue side take
    // the next one at this same chunk boundary (one pending item is then always enough)
    if (csn == cmp.steps) {
      if (nxt_valid) {
        cmp = nxt;
#pragma unroll
        for (int tf = 0; tf < TPW; ++tf) tok_ok[tf] = tok_nxt[tf];
        nxt_valid = false;
        csn = 0;
      } else {
        cmp_live = false;
      }
    }
    switch_issue();
  }
  wait_vmcnt<0>();  // no direct-to-LDS load may outlive the workgroup
}

}  // namespace

// Kernel shapes: gate/up 128 gate + 128 up rows per row block; down 256 rows per row block;
// both with 256-position workgroups.
constexpr int GU_RFR = 8, GU_TPW = 2, GU_NST = 3, GU_RBW = 2;
constexpr int DN_RFR = 16, DN_TPW = 2, DN_NST = 3, DN_RBW = 2;
constexpr int GU_INTERLEAVE = 1, DN_INTERLEAVE = 1;

// compute units of the current device (queried once per device)
static int cu_count() {
  static int cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64 && cache[dev] > 0) return cache[dev];
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < 64) cache[dev] = n;
  return n;
}

// every work item's step count (row blocks of the item x k-steps per row block) must be a
// multiple of the prefetch distance: items then start and end on chunk boundaries
static bool items_fit(int n_rows, int rows_per_block, int rbw, int k, int dist) {
  if (n_rows % rows_per_block) return false;
  const int nrb = n_rows / rows_per_block, nsteps = k / T_KS, w = std::min(nrb, rbw);
  return (w * nsteps) % dist == 0 && ((nrb % w) * nsteps) % dist == 0;
}

// shapes the tile kernels take
bool ffn_tiles_supported(int H, int I) {
  return items_fit(I, GU_RFR * 16, GU_RBW, H, GU_NST - 1) && items_fit(H, DN_RFR * 16, DN_RBW, I, DN_NST - 1);
}

// Launch gate/up and down with the 256-position tile list in tile_prefix.
hipError_t launch_expert_ffn_tiles(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                                   const int32_t* tile_prefix, int64_t max_tiles, const FfnWeights& w, int T, int H,
                                   int I, int E, int S, float limit, float shared_limit, uint16_t* h, void* y,
                                   hipStream_t s, Tracer* tr, bool y16) {
  if (!ffn_tiles_supported(H, I)) return hipErrorInvalidValue;
  TileArgs gu{};
  gu.act = x; gu.sorted_token = sorted_token; gu.offsets = offsets; gu.tile_prefix = tile_prefix;
  gu.w0 = (const uint16_t*)w.gate; gu.w1 = (const uint16_t*)w.up;
  gu.sw0 = (const uint16_t*)w.sh_gate; gu.sw1 = (const uint16_t*)w.sh_up;
  gu.out = h;  // h as one fp16 plane
  gu.T = T; gu.E = E; gu.S = S; gu.K = H; gu.N = I;
  // one weight set (a dense FFN): one row block per item, for twice the items (a single
  // expert has few token tiles to spread over the CUs)
  const bool single = E == 1 && S == 0 && items_fit(I, GU_RFR * 16, 1, H, GU_NST - 1) &&
                      items_fit(H, DN_RFR * 16, 1, I, DN_NST - 1);
  gu.nrb = I / (GU_RFR * 16); gu.rbw = std::min(gu.nrb, single ? 1 : GU_RBW);
  gu.ngroups = (gu.nrb + gu.rbw - 1) / gu.rbw;
  gu.limit = limit; gu.shared_limit = shared_limit;
  gu.interleave = GU_INTERLEAVE;
  gu.y16 = 0;

  TileArgs dn = gu;
  dn.act = h; dn.sorted_token = nullptr;
  dn.w0 = (const uint16_t*)w.down; dn.w1 = nullptr; dn.sw0 = (const uint16_t*)w.sh_down; dn.sw1 = nullptr;
  dn.out = y;
  dn.K = I; dn.N = H;
  dn.interleave = DN_INTERLEAVE;
  dn.y16 = y16 ? 1 : 0;
  dn.nrb = H / (DN_RFR * 16); dn.rbw = std::min(dn.nrb, single ? 1 : DN_RBW);
  dn.ngroups = (dn.nrb + dn.rbw - 1) / dn.rbw;

  // workgroups that each take several work items: four per CU (one is resident at a time, as
  // each holds 96 KB of LDS), so a CU whose items ran fast picks up the next workgroup;
  // measured against one per CU and one per item, on uniform and skewed routing
  const int cus = cu_count();
  if (cus <= 0) return hipErrorInvalidDevice;
  const int64_t grid_max = std::max<int64_t>(8, cus / 8 * 32);
  constexpr int GU_SUBS = T_LIST_BM / (T_NW * GU_TPW * 16), DN_SUBS = T_LIST_BM / (T_NW * DN_TPW * 16);
  int64_t g = std::min(grid_max, (max_tiles * GU_SUBS * gu.ngroups + 7) / 8 * 8);
  if (g > 0) {
    launch(tr, ffn_tile_kernel<TM_GATEUP, GU_RFR, GU_TPW, GU_NST>, dim3((unsigned)g), dim3(T_NW * 64), s, gu);
    hipError_t err = hipGetLastError();
    if (tr) tr->mark("expert_gate_up", s);
    if (err != hipSuccess) return err;
  }
  g = std::min(grid_max, (max_tiles * DN_SUBS * dn.ngroups + 7) / 8 * 8);
  if (g > 0) {
    launch(tr, ffn_tile_kernel<TM_DOWN, DN_RFR, DN_TPW, DN_NST>, dim3((unsigned)g), dim3(T_NW * 64), s, dn);
    hipError_t err = hipGetLastError();
    if (tr) tr->mark("expert_down", s);
    if (err != hipSuccess) return err;
  }
  return hipSuccess;
}

}  // namespace moe
