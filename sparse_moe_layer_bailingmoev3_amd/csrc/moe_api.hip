// C-ABI host layer of libmoe: argument validation (pure host code, before any HIP call),
// workspace layout and launch sequencing on the caller's stream.  The declarations and the
// contract of every entry point are in include/moe.h.
#include <stdarg.h>
#include <stdio.h>

#include <cmath>
#include <mutex>
#include <string>

#include "moe.h"
#include "moe_internal.h"

namespace {

thread_local std::string g_last_error;

// Device scratch of moe_forward_noalloc: one copy per GPU the library runs on, held until the
// process ends.  In host code `scratch` only names the symbol; its device address comes from
// hipGetSymbolAddress, once per device (g_scratch_ptr).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)64 << 20;
static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES];

moe_status_t fail(moe_status_t st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

moe_status_t hip_fail(hipError_t e, const char* what) {
  return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

#define MOE_CHECK_PTR(p, name)                                                            \
  do {                                                                                    \
    if (!(p)) return fail(MOE_ERR_INVALID_ARG, "%s must not be NULL", name);              \
    if (!aligned16(p)) return fail(MOE_ERR_ALIGNMENT, "%s is not 16-byte aligned", name); \
  } while (0)

#define MOE_CHECK_OPT_PTR(p, name)                                                               \
  do {                                                                                           \
    if ((p) && !aligned16(p)) return fail(MOE_ERR_ALIGNMENT, "%s is not 16-byte aligned", name); \
  } while (0)

moe_status_t validate_config(const moe_config_t* c, int64_t T) {
  if (!c) return fail(MOE_ERR_INVALID_ARG, "cfg must not be NULL");
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld must be >= 0", (long long)T);
  if (c->hidden_size <= 0) return fail(MOE_ERR_INVALID_ARG, "hidden_size must be > 0");
  if (c->hidden_size % 128) return fail(MOE_ERR_UNSUPPORTED, "hidden_size %d is not a multiple of 128", c->hidden_size);
  const int E = c->num_experts;
  if (E <= 0) return fail(MOE_ERR_INVALID_ARG, "num_experts must be > 0");
  if (E % 64 || E > 1024 || ((E / 64) & (E / 64 - 1)))
    return fail(MOE_ERR_UNSUPPORTED, "num_experts %d must be 64 * 2^k and at most 1024", E);
  const int G = c->n_group;
  if (G <= 0 || E % G) return fail(MOE_ERR_INVALID_ARG, "n_group %d must divide num_experts %d", G, E);
  if (64 % G) return fail(MOE_ERR_UNSUPPORTED, "n_group %d must divide 64", G);
  if (c->topk_group < 1 || c->topk_group > G)
    return fail(MOE_ERR_INVALID_ARG, "topk_group %d must be in [1, n_group=%d]", c->topk_group, G);
  const int K = c->num_experts_per_tok;
  if (K < 1 || K > c->topk_group * (E / G))
    return fail(MOE_ERR_INVALID_ARG, "num_experts_per_tok %d must be in [1, topk_group*E/n_group=%d]", K,
                c->topk_group * (E / G));
  if (K > 16) return fail(MOE_ERR_UNSUPPORTED, "num_experts_per_tok %d is above 16", K);
  if (c->moe_intermediate_size <= 0) return fail(MOE_ERR_INVALID_ARG, "moe_intermediate_size must be > 0");
  if (c->moe_intermediate_size % 128)
    return fail(MOE_ERR_UNSUPPORTED, "moe_intermediate_size %d is not a multiple of 128", c->moe_intermediate_size);
  if (c->num_shared_experts < 0 || c->num_shared_experts > 1)
    return fail(MOE_ERR_INVALID_ARG, "num_shared_experts %d must be 0 or 1", c->num_shared_experts);
  if (c->num_shared_experts && c->shared_intermediate_size != c->moe_intermediate_size)
    return fail(MOE_ERR_UNSUPPORTED, "shared_intermediate_size %d must equal moe_intermediate_size %d",
                c->shared_intermediate_size, c->moe_intermediate_size);
  if (c->expert_weight_format != MOE_WEIGHTS_BF16 && c->expert_weight_format != MOE_WEIGHTS_MXFP4 &&
      c->expert_weight_format != MOE_WEIGHTS_MXFP8 && c->expert_weight_format != MOE_WEIGHTS_MXFP4_TILED &&
      c->expert_weight_format != MOE_WEIGHTS_MXFP8_TILED)
    return fail(MOE_ERR_INVALID_ARG, "expert_weight_format %d is unknown", c->expert_weight_format);
  const bool tiled = c->expert_weight_format == MOE_WEIGHTS_MXFP4_TILED ||
                     c->expert_weight_format == MOE_WEIGHTS_MXFP8_TILED;
  if (tiled && (c->hidden_size % 256 || c->moe_intermediate_size % 256))
    return fail(MOE_ERR_UNSUPPORTED, "tiled block-format weights need hidden_size (%d) and moe_intermediate_size "
                "(%d) multiples of 256", c->hidden_size, c->moe_intermediate_size);
  if (c->expert_act_format != MOE_ACT_BF16 && c->expert_act_format != MOE_ACT_MXFP8)
    return fail(MOE_ERR_INVALID_ARG, "expert_act_format %d is unknown", c->expert_act_format);
  if (c->expert_act_format == MOE_ACT_MXFP8 && c->expert_weight_format == MOE_WEIGHTS_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "MXFP8 activations need MXFP4 or MXFP8 expert weights");
  if (!std::isfinite(c->routed_scaling_factor)) return fail(MOE_ERR_INVALID_ARG, "routed_scaling_factor is not finite");
  if (std::isnan(c->swiglu_limit) || std::isnan(c->shared_swiglu_limit))
    return fail(MOE_ERR_INVALID_ARG, "swiglu limits must not be NaN");
  if (T > (int64_t)((1u << 31) - 1) / (K + 1))
    return fail(MOE_ERR_UNSUPPORTED, "T = %lld is too large for 32-bit positions", (long long)T);
  return MOE_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// the kernels' weight-format code (the row-major and tiled orders of a format share the
// kernels; the tiled one sets FfnWeights::tiled)
int wfmt(const moe_config_t* c) {
  const int f = c->expert_weight_format;
  return f == MOE_WEIGHTS_MXFP4 || f == MOE_WEIGHTS_MXFP4_TILED   ? moe::FMT_MXFP4
         : f == MOE_WEIGHTS_MXFP8 || f == MOE_WEIGHTS_MXFP8_TILED ? moe::FMT_MXFP8
                                                                    : moe::FMT_BF16;
}

struct Layout {
  size_t partial, bitmap, counts, counts_out, offsets, tile_prefix, topk_idx, topk_w, sorted_token, inv_perm, h_hi, h_lo, y,
      xq, xs, hq, hs, total;
};

// y_bytes: bytes per value of the expert outputs y in the workspace (2: moe_forward writes them
// in fp16; 4: the dense FFN's one-expert path and its split partial sums)
Layout layout(const moe_config_t* c, int64_t T, int y_bytes = 2) {
  const int64_t E = c->num_experts, K = c->num_experts_per_tok, H = c->hidden_size, I = c->moe_intermediate_size;
  const int64_t S = c->num_shared_experts;
  const int64_t P = T * K + T * S;
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.partial = take(moe::router_partial_bytes(T, (int)H, (int)E));
  L.bitmap = take(moe::dispatch_bitmap_words(T, (int)E) * 4);
  L.counts = take((E + 1) * 4);
  L.counts_out = take((E + 1) * 4);
  L.offsets = take((E + 2) * 4);
  // the FFN tile prefix and, after it, one 16-byte record per tile of the plan
  L.tile_prefix = take(((size_t)moe::tile_info_offset((int)E) +
                        4 * (size_t)moe::ffn_plan(T, (int)K, (int)E, (int)S,
                                                  wfmt(c),
                                                  (int)H, (int)I).max_tiles) * 4);
  L.topk_idx = take(T * K * 4);
  L.topk_w = take(T * K * 4);
  L.sorted_token = take(P * 4);
  L.inv_perm = take(T * K * 4);
  L.h_hi = take(P * I * 2);
  // h's second (lo) bf16 plane: only the dense FFN's few-token kernels still write one; every
  // expert FFN kernel passes h as one plane
  L.h_lo = take(T <= moe::DENSE_SMALL_MAX_T ? P * I * 2 : 0);
  L.y = take(P * H * y_bytes);
  // MXFP8 activations: x and h as E4M3 codes and e8m0 scales (empty otherwise)
  const bool a8 = c->expert_act_format == MOE_ACT_MXFP8;
  L.xq = take(a8 ? T * H : 0);
  L.xs = take(a8 ? T * H / 32 : 0);
  L.hq = take(a8 ? P * I : 0);
  L.hs = take(a8 ? P * I / 32 : 0);
  L.total = off;
  return L;
}

moe_status_t check_ws(const moe_config_t* c, int64_t T, const void* ws, size_t ws_bytes, Layout* out,
                      int y_bytes = 2) {
  Layout L = layout(c, T, y_bytes);
  if (!ws) return fail(MOE_ERR_WORKSPACE, "workspace must not be NULL");
  if (((uintptr_t)ws & 255u) != 0) return fail(MOE_ERR_ALIGNMENT, "workspace is not 256-byte aligned");
  if (ws_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T=%lld", ws_bytes, L.total, (long long)T);
  *out = L;
  return MOE_OK;
}

moe_status_t check_weights(const moe_config_t* c, const moe_expert_weights_t* w) {
  if (!w) return fail(MOE_ERR_INVALID_ARG, "weights must not be NULL");
  MOE_CHECK_PTR(w->gate, "weights->gate");
  MOE_CHECK_PTR(w->up, "weights->up");
  MOE_CHECK_PTR(w->down, "weights->down");
  if (c->expert_weight_format != MOE_WEIGHTS_BF16) {
    if (!w->gate_scale || !w->up_scale || !w->down_scale)
      return fail(MOE_ERR_INVALID_ARG, "MXFP4 and MXFP8 weights need gate_scale, up_scale and down_scale");
    MOE_CHECK_PTR(w->gate_scale, "weights->gate_scale");
    MOE_CHECK_PTR(w->up_scale, "weights->up_scale");
    MOE_CHECK_PTR(w->down_scale, "weights->down_scale");
  }
  if (c->num_shared_experts) {
    MOE_CHECK_PTR(w->shared_gate, "weights->shared_gate");
    MOE_CHECK_PTR(w->shared_up, "weights->shared_up");
    MOE_CHECK_PTR(w->shared_down, "weights->shared_down");
  }
  return MOE_OK;
}

moe::FfnWeights ffn_weights(const moe_config_t* c, const moe_expert_weights_t* w) {
  moe::FfnWeights f{};
  f.gate = w->gate; f.up = w->up; f.down = w->down;
  f.gate_scale = w->gate_scale; f.up_scale = w->up_scale; f.down_scale = w->down_scale;
  f.sh_gate = w->shared_gate; f.sh_up = w->shared_up; f.sh_down = w->shared_down;
  f.fmt = wfmt(c);
  f.tiled = c->expert_weight_format == MOE_WEIGHTS_MXFP4_TILED || c->expert_weight_format == MOE_WEIGHTS_MXFP8_TILED;
  return f;
}

char* at(void* ws, size_t off) { return (char*)ws + off; }

// mark: also clear (logits kernel) the dispatch bitmap and histogram in the workspace and fill
// the bitmap (top-k kernel), so moe_dispatch's clear and mark kernels are not needed (the
// dispatch counts the histogram from the bitmap)
// fd (optional, with mark): finish the dispatch inside the top-k kernel; its counter is the
// histogram's spare last entry
moe_status_t do_route(const moe_config_t* c, int64_t T, const void* x, const float* rw, const float* bias,
                      int32_t* idx, float* wts, const Layout& L, void* ws, hipStream_t s,
                      moe::Tracer* tr = nullptr, bool mark = false, moe::FusedDispatch* fd = nullptr) {
  moe::RouterPlan p = moe::router_plan(T, c->hidden_size, c->num_experts);
  float* partial = (float*)at(ws, L.partial);
  uint32_t* bitmap = mark ? (uint32_t*)at(ws, L.bitmap) : nullptr;
  int32_t* counts = mark ? (int32_t*)at(ws, L.counts) : nullptr;
  moe::FusedDispatch none;
  if (fd) fd->done = counts + c->num_experts;
  // the bitmap and the counts (with the fused dispatch's counter after them) are adjacent in
  // the layout: one range to clear
  const int64_t clear_words = (int64_t)(L.counts - L.bitmap) / 4 + c->num_experts + 1;
  hipError_t e = moe::launch_router_logits(p, (const uint16_t*)x, rw, (int)T, c->hidden_size, c->num_experts,
                                           partial, bitmap, clear_words, s, tr);
  if (e != hipSuccess) return hip_fail(e, "router logits launch");
  e = moe::launch_router_topk(partial, p.nsplit, (int)T, c->num_experts, bias, c->n_group, c->topk_group,
                              c->num_experts_per_tok, c->norm_topk_prob, c->routed_scaling_factor, idx, wts, bitmap,
                              fd ? *fd : none, s, tr);
  if (e != hipSuccess) return hip_fail(e, "router top-k launch");
  return MOE_OK;
}

// marked: the router already filled the bitmap; the workspace histogram is counted from it
// and copied to `counts` by the finish kernel.  with_tiles: also write the FFN tile prefix.
moe_status_t do_dispatch(const moe_config_t* c, int64_t T, const int32_t* idx, int32_t* counts, int32_t* offsets,
                         int32_t* sorted_token, int32_t* inv_perm, const Layout& L, void* ws, hipStream_t s,
                         moe::Tracer* tr = nullptr, bool marked = false, bool with_tiles = false) {
  moe::FfnPlan fp = moe::ffn_plan(T, c->num_experts_per_tok, c->num_experts, c->num_shared_experts,
                                   wfmt(c),
                                   c->hidden_size, c->moe_intermediate_size);
  int32_t* hist = marked ? (int32_t*)at(ws, L.counts) : counts;
  hipError_t e = moe::launch_dispatch(idx, (int)T, c->num_experts_per_tok, c->num_experts, c->num_shared_experts,
                                      (uint32_t*)at(ws, L.bitmap), hist, counts, offsets, sorted_token, inv_perm,
                                      marked, with_tiles ? (int32_t*)at(ws, L.tile_prefix) : nullptr, fp.bm, s, tr);
  if (e != hipSuccess) return hip_fail(e, "dispatch launch");
  return MOE_OK;
}

moe_status_t do_ffn(const moe_config_t* c, int64_t T, const void* x, const int32_t* offsets,
                    const int32_t* sorted_token, const moe_expert_weights_t* w, void* y, const Layout& L, void* ws,
                    hipStream_t s, moe::Tracer* tr = nullptr, bool tiles_ready = false, bool own_shared = false,
                    hipStream_t shared_s = nullptr, bool y16 = false) {
  moe::FfnPlan p = moe::ffn_plan(T, c->num_experts_per_tok, c->num_experts, c->num_shared_experts,
                                  wfmt(c),
                                  c->hidden_size, c->moe_intermediate_size);
  const float lim = c->swiglu_limit > 0 ? c->swiglu_limit : 0.f;
  const float slim = c->shared_swiglu_limit > 0 ? c->shared_swiglu_limit : 0.f;
  moe::ActBufs ab;
  if (c->expert_act_format == MOE_ACT_MXFP8) {
    ab.act = moe::ACT_MXFP8;
    ab.xq = (uint8_t*)at(ws, L.xq);
    ab.xs = (uint8_t*)at(ws, L.xs);
    ab.hq = (uint8_t*)at(ws, L.hq);
    ab.hs = (uint8_t*)at(ws, L.hs);
  }
  hipError_t e = moe::launch_expert_ffn(p, (const uint16_t*)x, offsets, sorted_token, (int32_t*)at(ws, L.tile_prefix),
                                        ffn_weights(c, w), (int)T, c->hidden_size, c->moe_intermediate_size,
                                        c->num_experts, c->num_shared_experts, lim, slim, (uint16_t*)at(ws, L.h_hi),
                                        (float*)y, tiles_ready, s, tr, &ab, own_shared,
                                        shared_s, y16);
  if (e != hipSuccess) return hip_fail(e, "expert FFN launch");
  return MOE_OK;
}

moe_status_t do_combine(const moe_config_t* c, int64_t T, const void* y, const int32_t* inv, const float* wts,
                        void* out, hipStream_t s, moe::Tracer* tr = nullptr, bool y16 = false) {
  hipError_t e = moe::launch_combine(y, inv, wts, (int)T, c->num_experts_per_tok, c->hidden_size,
                                     c->num_shared_experts, (uint16_t*)out, s, tr, y16);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return MOE_OK;
}

}  // namespace

extern "C" {

const char* moe_status_string(moe_status_t st) {
  switch (st) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_ALIGNMENT: return "MOE_ERR_ALIGNMENT";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "unknown moe_status_t";
}

const char* moe_last_error(void) { return g_last_error.c_str(); }

moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes must not be NULL");
  *bytes = layout(cfg, T).total;
  return MOE_OK;
}

moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                       const float* expert_bias, int32_t* topk_idx, float* topk_w, void* ws, size_t ws_bytes,
                       void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  MOE_CHECK_PTR(router_w, "router_w");
  MOE_CHECK_OPT_PTR(expert_bias, "expert_bias");
  MOE_CHECK_PTR(topk_idx, "topk_idx");
  MOE_CHECK_PTR(topk_w, "topk_w");
  Layout L;
  if ((st = check_ws(cfg, T, ws, ws_bytes, &L)) != MOE_OK) return st;
  return do_route(cfg, T, x, router_w, expert_bias, topk_idx, topk_w, L, ws, (hipStream_t)stream);
}

moe_status_t moe_dispatch(const moe_config_t* cfg, int64_t T, const int32_t* topk_idx, int32_t* expert_counts,
                          int32_t* expert_offsets, int32_t* sorted_token, int32_t* inv_perm, void* ws, size_t ws_bytes,
                          void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_PTR(topk_idx, "topk_idx");
  MOE_CHECK_PTR(expert_counts, "expert_counts");
  MOE_CHECK_PTR(expert_offsets, "expert_offsets");
  MOE_CHECK_PTR(sorted_token, "sorted_token");
  MOE_CHECK_PTR(inv_perm, "inv_perm");
  Layout L;
  if ((st = check_ws(cfg, T, ws, ws_bytes, &L)) != MOE_OK) return st;
  return do_dispatch(cfg, T, topk_idx, expert_counts, expert_offsets, sorted_token, inv_perm, L, ws,
                     (hipStream_t)stream);
}

moe_status_t moe_expert_ffn(const moe_config_t* cfg, int64_t T, const void* x, const int32_t* expert_offsets,
                            const int32_t* sorted_token, const moe_expert_weights_t* weights, void* y_sorted, void* ws,
                            size_t ws_bytes, void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  MOE_CHECK_PTR(expert_offsets, "expert_offsets");
  MOE_CHECK_PTR(sorted_token, "sorted_token");
  MOE_CHECK_PTR(y_sorted, "y_sorted");
  if ((st = check_weights(cfg, weights)) != MOE_OK) return st;
  Layout L;
  if ((st = check_ws(cfg, T, ws, ws_bytes, &L)) != MOE_OK) return st;
  return do_ffn(cfg, T, x, expert_offsets, sorted_token, weights, y_sorted, L, ws, (hipStream_t)stream);
}

}  // extern "C"

namespace {

// A dense SwiGLU FFN is the layer with one routed expert that every token picks with weight 1
// and no shared expert: the same FFN kernels and the same combine (which then only rounds y).
moe_config_t dense_config(int32_t H, int32_t I, float limit) {
  moe_config_t c{};
  c.hidden_size = H;
  c.num_experts = 1;
  c.num_experts_per_tok = 1;
  c.n_group = 1;
  c.topk_group = 1;
  c.moe_intermediate_size = I;
  c.num_shared_experts = 0;
  c.shared_intermediate_size = 0;
  c.norm_topk_prob = 0;
  c.routed_scaling_factor = 1.0f;
  c.swiglu_limit = limit;
  c.shared_swiglu_limit = 0.0f;
  c.expert_weight_format = MOE_WEIGHTS_BF16;
  return c;
}

// the layer's workspace; with a split down reduction its partial sums start at the y region
// (the last one) and may run past it
size_t dense_ws_bytes(const moe_config_t* dc, int64_t T) {
  const Layout L = layout(dc, T, 4);
  const moe::FfnPlan p = moe::ffn_plan(T, 1, 1, 0, moe::FMT_BF16, dc->hidden_size, dc->moe_intermediate_size);
  if (p.ksplit_down <= 1) return L.total;
  return std::max(L.total, L.y + align256((size_t)p.ksplit_down * T * dc->hidden_size * 4));
}

moe_status_t validate_dense(int32_t H, int32_t I, float limit, int64_t T) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T = %lld must be >= 0", (long long)T);
  if (T > (int64_t)((1u << 31) - 1) / 2) return fail(MOE_ERR_UNSUPPORTED, "T = %lld is too large", (long long)T);
  if (H <= 0 || I <= 0) return fail(MOE_ERR_INVALID_ARG, "hidden_size and intermediate_size must be > 0");
  if (H % 128) return fail(MOE_ERR_UNSUPPORTED, "hidden_size %d is not a multiple of 128", H);
  if (I % 128) return fail(MOE_ERR_UNSUPPORTED, "intermediate_size %d is not a multiple of 128", I);
  if (!std::isfinite(limit)) return fail(MOE_ERR_INVALID_ARG, "swiglu_limit must be finite");
  return MOE_OK;
}

}  // namespace

extern "C" {

moe_status_t moe_dense_ffn_workspace_size(int32_t hidden_size, int32_t intermediate_size, int64_t T, size_t* bytes) {
  g_last_error.clear();
  moe_status_t st = validate_dense(hidden_size, intermediate_size, 0.0f, T);
  if (st != MOE_OK) return st;
  if (!bytes) return fail(MOE_ERR_INVALID_ARG, "bytes must not be NULL");
  const moe_config_t dc = dense_config(hidden_size, intermediate_size, 0.0f);
  *bytes = dense_ws_bytes(&dc, T);
  return MOE_OK;
}

moe_status_t moe_dense_ffn(int32_t hidden_size, int32_t intermediate_size, float swiglu_limit, int64_t T,
                           const void* x, const void* gate, const void* up, const void* down, void* out, void* ws,
                           size_t ws_bytes, void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_dense(hidden_size, intermediate_size, swiglu_limit, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  MOE_CHECK_PTR(out, "out");
  const moe_config_t dc = dense_config(hidden_size, intermediate_size, swiglu_limit > 0 ? swiglu_limit : 0.0f);
  moe_expert_weights_t w{};
  w.gate = gate;
  w.up = up;
  w.down = down;
  if ((st = check_weights(&dc, &w)) != MOE_OK) return st;
  Layout L;
  if ((st = check_ws(&dc, T, ws, ws_bytes, &L, 4)) != MOE_OK) return st;
  if (ws_bytes < dense_ws_bytes(&dc, T))
    return fail(MOE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed for T=%lld", ws_bytes, dense_ws_bytes(&dc, T),
                (long long)T);
  hipStream_t s = (hipStream_t)stream;
  if (moe::dense_ffn_small_supported(T, hidden_size, intermediate_size)) {
    hipError_t e = moe::launch_dense_ffn_small((const uint16_t*)x, (const uint16_t*)gate, (const uint16_t*)up,
                                               (const uint16_t*)down, (int)T, hidden_size, intermediate_size,
                                               dc.swiglu_limit, (uint16_t*)at(ws, L.h_hi), (uint16_t*)at(ws, L.h_lo),
                                               (uint16_t*)out, s);
    if (e != hipSuccess) return hip_fail(e, "dense FFN launch");
    return MOE_OK;
  }
  const moe::FfnPlan plan = moe::ffn_plan(T, 1, 1, 0, moe::FMT_BF16, hidden_size, intermediate_size);
  if (!plan.tiles) {
    // the expert FFN kernels with the tiles computed from T (no dispatch, no combine)
    hipError_t e = moe::launch_dense_ffn_tiled(plan, (const uint16_t*)x, (const uint16_t*)gate, (const uint16_t*)up,
                                               (const uint16_t*)down, (int)T, hidden_size, intermediate_size,
                                               dc.swiglu_limit, (uint16_t*)at(ws, L.h_hi),
                                               (float*)at(ws, L.y), (uint16_t*)out, s);
    if (e != hipSuccess) return hip_fail(e, "dense FFN launch");
    return MOE_OK;
  }
  int32_t* offsets = (int32_t*)at(ws, L.offsets);
  int32_t* sorted_token = (int32_t*)at(ws, L.sorted_token);
  int32_t* inv = (int32_t*)at(ws, L.inv_perm);
  float* wts = (float*)at(ws, L.topk_w);
  hipError_t e = moe::launch_dense_dispatch((int)T, offsets, sorted_token, inv, wts, s);
  if (e != hipSuccess) return hip_fail(e, "dense dispatch launch");
  void* y = at(ws, L.y);
  if ((st = do_ffn(&dc, T, x, offsets, sorted_token, &w, y, L, ws, s)) != MOE_OK) return st;
  return do_combine(&dc, T, y, inv, wts, out, s);
}

moe_status_t moe_quantise_mxfp8(const void* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                                void* stream) {
  g_last_error.clear();
  if (rows < 0) return fail(MOE_ERR_INVALID_ARG, "rows = %lld must be >= 0", (long long)rows);
  if (cols <= 0 || cols % 32) return fail(MOE_ERR_INVALID_ARG, "cols = %d must be a positive multiple of 32", cols);
  if (rows == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  MOE_CHECK_PTR(codes, "codes");
  if (!scales) return fail(MOE_ERR_INVALID_ARG, "scales must not be NULL");
  hipError_t e = moe::launch_mx8_quant((const uint16_t*)x, rows, cols, codes, scales, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "MXFP8 quantise launch");
  return MOE_OK;
}

static moe_status_t pack_mx(int fmt, const uint8_t* codes, const uint8_t* scales, int64_t mats, int32_t N,
                            int32_t Kd, uint8_t* codes_out, uint8_t* scales_out, void* stream) {
  g_last_error.clear();
  if (mats < 0) return fail(MOE_ERR_INVALID_ARG, "mats = %lld must be >= 0", (long long)mats);
  if (N <= 0 || N % 16) return fail(MOE_ERR_INVALID_ARG, "N = %d must be a positive multiple of 16", N);
  if (Kd <= 0 || Kd % 256) return fail(MOE_ERR_INVALID_ARG, "Kd = %d must be a positive multiple of 256", Kd);
  if (mats == 0) return MOE_OK;
  MOE_CHECK_PTR(codes, "codes");
  MOE_CHECK_PTR(codes_out, "codes_out");
  if (!scales || !scales_out) return fail(MOE_ERR_INVALID_ARG, "scales and scales_out must not be NULL");
  if (((uintptr_t)scales & 7u) || ((uintptr_t)scales_out & 7u))
    return fail(MOE_ERR_ALIGNMENT, "scales and scales_out must be 8-byte aligned");
  const uintptr_t cb = (uintptr_t)mats * (uintptr_t)N * (uintptr_t)(fmt == moe::FMT_MXFP4 ? Kd / 2 : Kd);
  const uintptr_t sb = (uintptr_t)mats * (uintptr_t)N * (uintptr_t)(Kd / 32);
  auto overlap = [](const void* a, uintptr_t na, const void* b, uintptr_t nb) {
    return (uintptr_t)a < (uintptr_t)b + nb && (uintptr_t)b < (uintptr_t)a + na;
  };
  if (overlap(codes_out, cb, codes, cb) || overlap(codes_out, cb, scales, sb) || overlap(codes_out, cb, scales_out, sb) ||
      overlap(scales_out, sb, codes, cb) || overlap(scales_out, sb, scales, sb))
    return fail(MOE_ERR_INVALID_ARG, "the output arrays must not overlap each other or the inputs");
  hipError_t e = moe::launch_pack_mx(fmt, codes, scales, mats, N, Kd, codes_out, scales_out, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "block-format pack launch");
  return MOE_OK;
}

moe_status_t moe_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t mats, int32_t N, int32_t Kd,
                            uint8_t* codes_out, uint8_t* scales_out, void* stream) {
  return pack_mx(moe::FMT_MXFP4, codes, scales, mats, N, Kd, codes_out, scales_out, stream);
}

moe_status_t moe_pack_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t mats, int32_t N, int32_t Kd,
                            uint8_t* codes_out, uint8_t* scales_out, void* stream) {
  return pack_mx(moe::FMT_MXFP8, codes, scales, mats, N, Kd, codes_out, scales_out, stream);
}

moe_status_t moe_update_expert_bias(const moe_config_t* cfg, const int32_t* expert_counts, float* expert_bias,
                                    float gamma, void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, 0);
  if (st != MOE_OK) return st;
  MOE_CHECK_PTR(expert_counts, "expert_counts");
  MOE_CHECK_PTR(expert_bias, "expert_bias");
  if (!std::isfinite(gamma)) return fail(MOE_ERR_INVALID_ARG, "gamma must be finite");
  hipError_t e = moe::launch_expert_bias_update(expert_counts, cfg->num_experts, gamma, expert_bias,
                                                (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "expert bias update launch");
  return MOE_OK;
}

moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const void* y_sorted, const int32_t* inv_perm,
                         const float* topk_w, void* out, void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_PTR(y_sorted, "y_sorted");
  MOE_CHECK_PTR(inv_perm, "inv_perm");
  MOE_CHECK_PTR(topk_w, "topk_w");
  MOE_CHECK_PTR(out, "out");
  return do_combine(cfg, T, y_sorted, inv_perm, topk_w, out, (hipStream_t)stream);
}

namespace {

// The shared expert of a block-format layer runs on bf16 kernels of its own and reads x only,
// so moe_forward gives it a second stream of the library's, forked from the caller's stream
// at the start of the step and joined before the combine: it then runs beside the router, the
// dispatch and the routed experts (all of which wait on their memory pipelines) instead of
// after them.  One stream and two events per device, created on the device's first such
// forward; the mutex is held from the fork to the join, so concurrent callers never reuse an
// event before its wait is enqueued.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
std::mutex g_side_mu;
SideStream g_side[MAX_DEVICES];

// with g_side_mu held
moe_status_t side_stream(SideStream** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MOE_ERR_UNSUPPORTED, "device %d is beyond %d", dev, MAX_DEVICES);
  SideStream& d = g_side[dev];
  if (!d.s) {
    SideStream n;
    e = hipStreamCreateWithFlags(&n.s, hipStreamNonBlocking);  // default priority
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.fork, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&n.join, hipEventDisableTiming);
    if (e != hipSuccess) {
      if (n.join) (void)hipEventDestroy(n.join);
      if (n.fork) (void)hipEventDestroy(n.fork);
      if (n.s) (void)hipStreamDestroy(n.s);
      return hip_fail(e, "creating the shared expert's stream");
    }
    d = n;
  }
  *out = &d;
  return MOE_OK;
}

moe_status_t route_dispatch_ffn(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                                const float* expert_bias, const moe_expert_weights_t* weights, int32_t* idx,
                                float* wts, int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv,
                                void* y, const Layout& L, void* ws, hipStream_t s, moe::Tracer* tr,
                                hipStream_t shared_s, bool y16);

moe_status_t forward_impl(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                          const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                          int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out, void* ws,
                          size_t ws_bytes, void* stream, moe::Tracer* tr, bool may_fork = true) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  MOE_CHECK_PTR(x, "x");
  MOE_CHECK_PTR(router_w, "router_w");
  MOE_CHECK_OPT_PTR(expert_bias, "expert_bias");
  MOE_CHECK_PTR(out, "out");
  MOE_CHECK_OPT_PTR(topk_idx_out, "topk_idx_out");
  MOE_CHECK_OPT_PTR(topk_w_out, "topk_w_out");
  MOE_CHECK_OPT_PTR(expert_counts_out, "expert_counts_out");
  if ((st = check_weights(cfg, weights)) != MOE_OK) return st;
  Layout L;
  if ((st = check_ws(cfg, T, ws, ws_bytes, &L)) != MOE_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  int32_t* idx = topk_idx_out ? topk_idx_out : (int32_t*)at(ws, L.topk_idx);
  float* wts = topk_w_out ? topk_w_out : (float*)at(ws, L.topk_w);
  int32_t* counts = expert_counts_out ? expert_counts_out : (int32_t*)at(ws, L.counts_out);
  int32_t* offsets = (int32_t*)at(ws, L.offsets);
  int32_t* sorted_token = (int32_t*)at(ws, L.sorted_token);
  int32_t* inv = (int32_t*)at(ws, L.inv_perm);
  void* y = at(ws, L.y);
  if (tr && tr->events && tr->cap > 0 && tr->events[0]) (void)hipEventRecord(tr->events[0], s);
  // the shared expert of a block-format layer on the second stream (not when every kernel is
  // followed by an event on the caller's stream: the trace times the kernels one by one)
  // (bf16 layers keep the shared expert inside the routed launches: measured as launches of
  // its own on the second stream, the 256-position tile kernels' prefill went 2.03 -> 2.05 ms
  // and the skewed workload 2.64 -> 2.71 ms)
  const bool fork = may_fork && cfg->num_shared_experts && wfmt(cfg) != moe::FMT_BF16 && !(tr && tr->events);
  std::unique_lock<std::mutex> side_lock;
  SideStream* side = nullptr;
  if (fork) {
    side_lock = std::unique_lock<std::mutex>(g_side_mu);
    if ((st = side_stream(&side)) != MOE_OK) return st;
    hipError_t e = hipEventRecord(side->fork, s);
    if (e == hipSuccess) e = hipStreamWaitEvent(side->s, side->fork, 0);
    if (e != hipSuccess) return hip_fail(e, "forking the shared expert's stream");
  }
  // expert outputs y in fp16: half the down GEMM's writes and the combine's reads; the staged
  // calls (moe_expert_ffn, moe_combine) keep their fp32 y_sorted
  const bool y16 = true;
  st = route_dispatch_ffn(cfg, T, x, router_w, expert_bias, weights, idx, wts, counts, offsets, sorted_token, inv, y,
                          L, ws, s, tr, fork ? side->s : s, y16);
  if (fork) {
    // joined whatever happened above, so that no work of this step on the second stream can
    // run after what the caller enqueues next
    hipError_t e = hipEventRecord(side->join, side->s);
    if (e == hipSuccess) e = hipStreamWaitEvent(s, side->join, 0);
    side_lock.unlock();
    if (st == MOE_OK && e != hipSuccess) return hip_fail(e, "joining the shared expert's stream");
  }
  if (st != MOE_OK) return st;
  return do_combine(cfg, T, y, inv, wts, out, s, tr, y16);
}

// router, dispatch and expert FFNs of one forward; the shared expert, where it has launches
// of its own, goes to shared_s (the second stream or the caller's)
moe_status_t route_dispatch_ffn(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                                const float* expert_bias, const moe_expert_weights_t* weights, int32_t* idx,
                                float* wts, int32_t* counts, int32_t* offsets, int32_t* sorted_token, int32_t* inv,
                                void* y, const Layout& L, void* ws, hipStream_t s, moe::Tracer* tr,
                                hipStream_t shared_s, bool y16) {
  moe_status_t st;
  if (T <= moe::FUSED_DISPATCH_MAX_T && T * cfg->num_experts_per_tok <= moe::FUSED_DISPATCH_MAX_PAIRS &&
      cfg->num_experts <= moe::FUSED_DISPATCH_MAX_E) {
    // few tokens: the top-k kernel's last workgroup finishes the dispatch (one launch fewer)
    moe::FusedDispatch fd;
    fd.counts_out = counts;
    fd.offsets = offsets;
    fd.sorted_token = sorted_token;
    fd.inv_perm = inv;
    fd.tile_prefix = (int32_t*)at(ws, L.tile_prefix);
    fd.S = cfg->num_shared_experts;
    fd.bm = moe::ffn_plan(T, cfg->num_experts_per_tok, cfg->num_experts, cfg->num_shared_experts,
                          wfmt(cfg),
                          cfg->hidden_size, cfg->moe_intermediate_size).bm;
    if ((st = do_route(cfg, T, x, router_w, expert_bias, idx, wts, L, ws, s, tr, true, &fd)) != MOE_OK) return st;
  } else {
    if ((st = do_route(cfg, T, x, router_w, expert_bias, idx, wts, L, ws, s, tr, true)) != MOE_OK) return st;
    if ((st = do_dispatch(cfg, T, idx, counts, offsets, sorted_token, inv, L, ws, s, tr, true, true)) != MOE_OK)
      return st;
  }
  return do_ffn(cfg, T, x, offsets, sorted_token, weights, y, L, ws, s, tr, true, true, shared_s, y16);
}

}  // namespace

moe_status_t moe_forward(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                         const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                         int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out, void* ws,
                         size_t ws_bytes, void* stream) {
  return forward_impl(cfg, T, x, router_w, expert_bias, weights, out, topk_idx_out, topk_w_out, expert_counts_out,
                      ws, ws_bytes, stream, nullptr);
}

moe_status_t moe_forward_traced(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                                const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                                void* ws, size_t ws_bytes, void* stream, void* const* events, int32_t max_events,
                                const char** kernel_names, int32_t* n_kernels) {
  if (!events || max_events < 1 || !kernel_names || !n_kernels)
    return fail(MOE_ERR_INVALID_ARG, "events, kernel_names and n_kernels are required, max_events >= 1");
  moe::Tracer tr;
  tr.events = (hipEvent_t*)events;
  tr.names = kernel_names;
  tr.cap = max_events;
  moe_status_t st = forward_impl(cfg, T, x, router_w, expert_bias, weights, out, nullptr, nullptr, nullptr, ws,
                                 ws_bytes, stream, &tr);
  *n_kernels = tr.n;
  if (st == MOE_OK && tr.n + 1 > max_events)
    return fail(MOE_ERR_INVALID_ARG, "%d kernels launched but only %d events given", tr.n, max_events);
  return st;
}

moe_status_t moe_forward_timed(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                               const float* expert_bias, const moe_expert_weights_t* weights, void* out, void* ws,
                               size_t ws_bytes, void* stream, int32_t kernel_index, void* start_event,
                               void* stop_event) {
  if (!start_event || !stop_event || kernel_index < 0)
    return fail(MOE_ERR_INVALID_ARG, "start_event and stop_event are required, kernel_index >= 0");
  moe::Tracer tr;
  tr.tindex = kernel_index;
  tr.tstart = (hipEvent_t)start_event;
  tr.tstop = (hipEvent_t)stop_event;
  moe_status_t st = forward_impl(cfg, T, x, router_w, expert_bias, weights, out, nullptr, nullptr, nullptr, ws,
                                 ws_bytes, stream, &tr);
  if (st == MOE_OK && !tr.timed)
    return fail(MOE_ERR_INVALID_ARG, "kernel_index %d: the forward launched %d kernels", kernel_index, tr.n);
  return st;
}


moe_status_t moe_forward_noalloc(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                                 const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                                 int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out,
                                 void* stream) {
  g_last_error.clear();
  moe_status_t st = validate_config(cfg, T);
  if (st != MOE_OK) return st;
  if (T == 0) return MOE_OK;
  const size_t need = layout(cfg, T).total;
  if (need > NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "moe_forward_noalloc: T=%lld needs %zu bytes of scratch, the static scratch holds %zu; "
                "use moe_forward with a caller workspace", (long long)T, need, NOALLOC_SCRATCH_BYTES);
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= MAX_DEVICES) return fail(MOE_ERR_UNSUPPORTED, "device %d is beyond %d", dev, MAX_DEVICES);
  void* ws = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
      // first call on this device (it is current): the device address of its copy
      void* p = nullptr;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
      if (!p || ((uintptr_t)p & 255u)) return fail(MOE_ERR_HIP, "scratch has no 256-byte aligned device address");
      g_scratch_ptr[dev] = p;
    }
    ws = g_scratch_ptr[dev];
  }
  // no second stream here: its first creation would allocate
  return forward_impl(cfg, T, x, router_w, expert_bias, weights, out, topk_idx_out, topk_w_out, expert_counts_out,
                      ws, NOALLOC_SCRATCH_BYTES, stream, nullptr, false);
}

}  // extern "C"
