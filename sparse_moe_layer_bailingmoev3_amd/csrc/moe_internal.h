// Internal launch interface between the C-ABI host layer and the kernels.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// routed-expert weight formats (moe_weight_format_t values)
enum { FMT_BF16 = 0, FMT_MXFP4 = 1, FMT_MXFP8 = 2 };
// activations of the routed experts' products (moe_act_format_t values)
enum { ACT_BF16 = 0, ACT_MXFP8 = 1 };

// The FFN tile list: tile_prefix[0 .. E+1] (tiles of the experts before e), then, from this
// offset (in int32, 16-byte aligned), one record per tile: {expert, its first sorted
// position, its rows, 0}, so that a workgroup finds its tile with one load instead of a
// binary search.  Whoever writes the prefix writes the records too.
constexpr int tile_info_offset(int E) { return (E + 2 + 3) / 4 * 4; }

// Optional per-kernel event trace: events[0] is recorded before the first launch,
// events[i+1] right after the i-th kernel (a NULL slot records nothing); names[i] names that
// kernel.  Independently, kernel `tindex` can be timed by events bound to its own dispatch
// (tstart, tstop: no extra queue packets, so the step runs as it does untraced).
struct Tracer {
  hipEvent_t* events = nullptr;
  const char** names = nullptr;
  int cap = 0;  // number of events available
  int n = 0;    // kernels launched so far
  int tindex = -1;
  hipEvent_t tstart = nullptr, tstop = nullptr;
  bool timed = false;  // the timed kernel was launched
  void mark(const char* name, hipStream_t s) {
    if (events && n + 1 < cap) {
      if (events[n + 1]) (void)hipEventRecord(events[n + 1], s);
      names[n] = name;
    }
    ++n;
  }
};

// Every kernel of the library is launched through here: the kernel of step `tr->n` gets the
// timing events bound to its dispatch when the tracer asks for them (the first launch of a
// step that launches several).  Errors are read by the caller with hipGetLastError.
template <typename... KArgs, typename... Args>
void launch(Tracer* tr, void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t s, Args... args) {
  if (tr && tr->tstart && !tr->timed && tr->tindex == tr->n) {
    hipExtLaunchKernelGGL(kernel, grid, block, 0, s, tr->tstart, tr->tstop, 0, args...);
    tr->timed = true;
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, s, args...);
  }
}

// ---- router ------------------------------------------------------------------
struct RouterPlan {
  int mf;       // 16-token fragments per workgroup (1, 2, 4 or 8)
  int rf;       // 16-expert blocks per wave (1 or 2)
  int nsplit;   // split of the hidden dimension (partial logits summed in order)
  int m_tiles, n_tiles;
  bool kwaves;  // few tokens: 16 experts per workgroup, its 4 waves split the k range
};
RouterPlan router_plan(int64_t T, int H, int E);
size_t router_partial_bytes(int64_t T, int H, int E);
// `clear` (optional): words zeroed by the logits kernel (the fused forward's dispatch bitmap
// and counters, which the top-k kernel then fills)
hipError_t launch_router_logits(const RouterPlan& p, const uint16_t* x, const float* w, int T, int H,
                                int E, float* partial, uint32_t* clear, int64_t clear_words, hipStream_t s,
                                Tracer* tr = nullptr);
// Dispatch finished inside the top-k kernel (few tokens): the last workgroup to finish, found
// with a counter (`done`, zero before the launch), writes the offsets, the sorted tokens,
// inv_perm, the expert counts and the FFN tile prefix from the complete topk_idx (bitmap and
// histogram rebuilt in its LDS; the top-k workgroups then make no dispatch atomics).
struct FusedDispatch {
  int32_t* done = nullptr;  // null: no fused dispatch
  int32_t* counts_out = nullptr;
  int32_t* offsets = nullptr;
  int32_t* sorted_token = nullptr;
  int32_t* inv_perm = nullptr;
  int32_t* tile_prefix = nullptr;  // optional
  int S = 0, bm = 1;
};
constexpr int FUSED_DISPATCH_MAX_T = 256;
constexpr int FUSED_DISPATCH_MAX_PAIRS = 4096;  // tokens x slots
constexpr int FUSED_DISPATCH_MAX_E = 1024;
hipError_t launch_router_topk(const float* partial, int nsplit, int T, int E, const float* bias, int G,
                              int TG, int K, int norm, float scale, int32_t* topk_idx, float* topk_w,
                              uint32_t* bitmap, const FusedDispatch& fd, hipStream_t s, Tracer* tr = nullptr);

// expert-bias update from the routed counts (one workgroup; E <= 1024)
hipError_t launch_expert_bias_update(const int32_t* counts, int E, float gamma, float* bias, hipStream_t s);

// ---- dispatch ----------------------------------------------------------------
size_t dispatch_bitmap_words(int64_t T, int E);
// marked: the bitmap was already filled by the router's top-k kernel (and cleared by its
// logits kernel), which lists an expert at most once per token, so the histogram is the
// popcount of each bitmap row.  tile_prefix (optional): tiles of bm positions per expert.
// counts: the histogram (filled here); counts_out receives a copy plus the shared expert's
// entry (may equal counts)
hipError_t launch_dispatch(const int32_t* topk_idx, int T, int K, int E, int S, uint32_t* bitmap,
                           int32_t* counts, int32_t* counts_out, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm,
                           bool marked, int32_t* tile_prefix, int bm, hipStream_t s, Tracer* tr = nullptr);

// dense FFN as a one-expert layer: offsets {0, T, T}, identity permutation, slot weight 1
hipError_t launch_dense_dispatch(int T, int32_t* offsets, int32_t* sorted_token, int32_t* inv_perm, float* topk_w,
                                 hipStream_t s);

// ---- expert FFN --------------------------------------------------------------
struct FfnWeights {
  const void* gate; const void* up; const void* down;
  const uint8_t* gate_scale; const uint8_t* up_scale; const uint8_t* down_scale;
  const void* sh_gate; const void* sh_up; const void* sh_down;
  int fmt;
  int tiled;  // MXFP4 / MXFP8 in the tiled order (moe_pack_mxfp4 / moe_pack_mxfp8)
};
struct FfnPlan {
  int mf;      // 16-token fragments per tile of the tile list (1, 2, 4, 8; 16 for bf16 weights)
  int mf_gate_up, mf_down;  // fragments per workgroup of each GEMM (divide mf)
  int bm;      // tokens per tile = 16 * mf
  int rbw_gate_up, rbw_down;  // 128-row weight blocks per workgroup
  bool tiles;  // use the 256-token tile kernel (bm = 256)
  bool group_major;  // work order: the tiles of one row-block group consecutive (one weight set)
  int ksplit_down;   // workgroups splitting the down reduction (a dense FFN with few tokens; else 1)
  int64_t max_tiles;
  int topk;          // routed slots per token (the shared expert's positions start at T * topk)
};
FfnPlan ffn_plan(int64_t T, int K, int E, int S, int fmt, int H, int I);
// the shared expert's own launches in block-format layers (a dense FFN over the T tokens)
struct SharedPlan {
  int mf, mf_down;   // 16-token fragments per tile of gate/up and of down
  int group_major;   // work order: the tiles of one row block consecutive
  int64_t tiles;     // ceil(T / (16 * mf))
};
SharedPlan shared_plan(int64_t T);
// MXFP8 activations of the routed experts (act == ACT_MXFP8): x rounded to MXFP8 (codes [T,H],
// scales [T,H/32]) by a first kernel, h written by gate/up as MXFP8 (codes [P,I], scales
// [P,I/32]); the shared expert keeps bf16 x and its fp16 h plane
struct ActBufs {
  int act = ACT_BF16;
  uint8_t* xq = nullptr;
  uint8_t* xs = nullptr;
  uint8_t* hq = nullptr;
  uint8_t* hs = nullptr;
};
hipError_t launch_expert_ffn(const FfnPlan& p, const uint16_t* x, const int32_t* offsets,
                             const int32_t* sorted_token, int32_t* tile_prefix, const FfnWeights& w,
                             int T, int H, int I, int E, int S, float limit, float shared_limit,
                             uint16_t* h, float* y, bool tiles_ready, hipStream_t s,
                             Tracer* tr = nullptr, const ActBufs* ab = nullptr, bool own_shared = false,
                             hipStream_t shared_s = nullptr, bool y16 = false);
// (y16: y written as fp16 [P,H], saturated at +-65504, instead of fp32)
// bf16 [rows, cols] -> MXFP8 codes [rows, cols] and e8m0 scales [rows, cols/32] (cols % 32 == 0)
// row-major MXFP4 (fmt FMT_MXFP4) or MXFP8 arrays of `mats` matrices [N, Kd] -> the tiled order
// of moe_pack_mxfp4 / moe_pack_mxfp8
hipError_t launch_pack_mx(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t mats, int N, int Kd,
                          uint8_t* codes_out, uint8_t* scales_out, hipStream_t s);
hipError_t launch_mx8_quant(const uint16_t* x, int64_t rows, int cols, uint8_t* codes, uint8_t* scales,
                            hipStream_t s);

// a dense FFN (one weight set, every token, weight 1) on the expert FFN kernels without the
// dispatch and combine: tiles follow from T, down writes the bf16 output [T,H] (plan from
// ffn_plan(T, 1, 1, 0, FMT_BF16, H, I) without the 256-position tile kernel)
// part: fp32 [p.ksplit_down, T, H] when p.ksplit_down > 1 (the partial sums of the split down
// reduction, added in order by a last kernel)
constexpr int DENSE_MAX_KSPLIT = 16;
constexpr int64_t DENSE_KSPLIT_MAX_T = 512;
hipError_t launch_dense_ffn_tiled(const FfnPlan& p, const uint16_t* x, const uint16_t* gate, const uint16_t* up,
                                  const uint16_t* down, int T, int H, int I, float limit, uint16_t* h,
                                  float* part, uint16_t* out, hipStream_t s);

// 256-position tiles, bf16 weights (ffn_tile.hip); tile_prefix holds the 256-position tiles.
// y16: y written as fp16 [P,H] (saturated at +-65504) instead of fp32
bool ffn_tiles_supported(int H, int I);
hipError_t launch_expert_ffn_tiles(const uint16_t* x, const int32_t* offsets, const int32_t* sorted_token,
                                   const int32_t* tile_prefix, int64_t max_tiles, const FfnWeights& w, int T, int H,
                                   int I, int E, int S, float limit, float shared_limit, uint16_t* h,
                                   void* y, hipStream_t s, Tracer* tr, bool y16 = false);

// ---- dense FFN for few tokens (dense_ffn.hip) -----------------------------------
// gate/up then down, each workgroup's waves splitting the reduction; h planes [T,I] in the
// caller's workspace, the bf16 output written by the down kernel (no dispatch, no combine)
constexpr int DENSE_SMALL_MAX_T = 10;  // measured crossover with the expert kernels (T = 8: 35.6 against 38.5 us, 16: 45.4 against 40.2)
bool dense_ffn_small_supported(int64_t T, int H, int I);
hipError_t launch_dense_ffn_small(const uint16_t* x, const uint16_t* gate, const uint16_t* up, const uint16_t* down,
                                  int T, int H, int I, float limit, uint16_t* h_hi, uint16_t* h_lo, uint16_t* out,
                                  hipStream_t s);

// ---- combine -----------------------------------------------------------------
// y16: y_sorted holds fp16 values (the tile kernels' y16 output) instead of fp32
hipError_t launch_combine(const void* y_sorted, const int32_t* inv_perm, const float* topk_w, int T,
                          int K, int H, int S, uint16_t* out, hipStream_t s, Tracer* tr = nullptr,
                          bool y16 = false);

}  // namespace moe
