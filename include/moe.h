/*
 * moe.h -- C ABI of libmoe: the forward pass of one BailingMoeV3 sparse MoE layer
 * (Ling-3.0-flash / Ling-3.0-flash-VL) on one AMD Instinct MI355X (gfx950).
 *
 * What the layer computes (Ling-3.0-flash-VL routing walk-through page, lqnn.cn,
 * "MoE 稀疏路由机制"):
 *   section 三.1  router: one raw score per routed expert from the hidden state, then
 *                 an element-wise sigmoid (score_function "sigmoid");
 *   section 三.3  a per-expert bias is added to the score used for selection
 *                 (moe_router_enable_expert_bias);
 *   section 三.2  the experts form n_group equal groups; keep the topk_group groups
 *                 with the largest in-group maximum, then the num_experts_per_tok best
 *                 experts inside the kept groups;
 *   section 四    router in fp32 (router_dtype), weights renormalised to sum to 1
 *                 (norm_topk_prob) and multiplied by routed_scaling_factor; SwiGLU
 *                 activations optionally clamped (expert_swiglu_limit_list);
 *   section 二    each expert is a SwiGLU FFN (gate, up: hidden -> intermediate;
 *                 down: intermediate -> hidden) and one shared expert sees every token.
 * Routed-expert weights may be MXFP4 (hybrid-attention page, lpnh.cn, table 模型一览).
 * The block is BailingMoeV3SparseMoeBlock (Ling-3.0-flash page, wmrh.cn, section
 * 稀疏MoE设计).
 *
 * Conventions for every entry point
 *   - Pointers marked "device" are HIP device pointers the caller owns; the library
 *     keeps no pointer and no state after a call returns and allocates no device memory
 *     (moe_forward's second stream, below, is the one object it keeps).
 *     Every device pointer must be 16-byte aligned.  Outputs must not alias inputs.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).  Calls
 *     only enqueue work: they return before the GPU finishes, and a fault inside a
 *     kernel surfaces at the caller's next synchronisation as a HIP error.
 *   - Argument errors are found on the host before anything is enqueued and return a
 *     negative status; moe_last_error() then describes the failure (thread-local).
 *   - T (tokens) may be 0: the call returns MOE_OK and enqueues nothing.
 *   - Matrices are row-major.  bf16 tensors are passed as raw 16-bit patterns.
 *   - Results are bitwise reproducible run to run: no reduction uses atomics.
 *
 * Shapes (T tokens; symbols used below)
 *   H = hidden_size, E = num_experts, K = num_experts_per_tok, I = moe_intermediate_size,
 *   S = num_shared_experts (0 or 1), P = T*K + T*S sorted positions.
 */
#ifndef MOE_H_
#define MOE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1, /* a size, flag or pointer is out of range or NULL */
  MOE_ERR_UNSUPPORTED = -2, /* a valid configuration these kernels do not implement */
  MOE_ERR_ALIGNMENT = -3,   /* a device pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = -4,   /* workspace NULL or smaller than moe_workspace_size() */
  MOE_ERR_HIP = -5          /* a HIP launch failed; moe_last_error() has the HIP text */
} moe_status_t;

typedef enum {
  MOE_WEIGHTS_BF16 = 0,
  MOE_WEIGHTS_MXFP4 = 1,
  MOE_WEIGHTS_MXFP8 = 2,
  MOE_WEIGHTS_MXFP4_TILED = 3, /* MXFP4 in the kernels' tiled order (moe_pack_mxfp4) */
  MOE_WEIGHTS_MXFP8_TILED = 4  /* MXFP8 in the kernels' tiled order (moe_pack_mxfp8) */
} moe_weight_format_t;

/* Activations of the routed experts' two matrix products.  MOE_ACT_BF16: x as given (bf16)
 * and h kept as one fp16 plane (11 significant bits; one bf16 plane for MXFP4 weights).  MOE_ACT_MXFP8 (MXFP4 or MXFP8
 * weights only): x and h rounded to MXFP8 -- E4M3 values with one e8m0 scale per 32
 * consecutive values along the reduction (OCP MX v1.0: scale = 2^(floor(log2 amax) - 8),
 * round to nearest even, saturate at 448) -- and multiplied by gfx950's scaled MFMA; the
 * shared expert keeps bf16 activations.  The hybrid-attention page (table 模型一览) lists the
 * quantised model as "FP8 + MXFP4". */
typedef enum { MOE_ACT_BF16 = 0, MOE_ACT_MXFP8 = 1 } moe_act_format_t;

/* Layer configuration.  Field names follow the model's config.json text_config as the
 * routing walk-through page quotes them (sections 二, 三.2 and 四). */
typedef struct {
  int32_t hidden_size;              /* H; multiple of 128 */
  int32_t num_experts;              /* E routed experts; multiple of 64, at most 1024 */
  int32_t num_experts_per_tok;      /* K, 1..16 and at most topk_group*E/n_group */
  int32_t n_group;                  /* groups; divides 64 and E */
  int32_t topk_group;               /* kept groups, 1..n_group */
  int32_t moe_intermediate_size;    /* I; multiple of 128 */
  int32_t num_shared_experts;       /* S: 0 or 1 */
  int32_t shared_intermediate_size; /* must equal I when S == 1 */
  int32_t norm_topk_prob;           /* nonzero: renormalise the K weights to sum to 1 */
  float routed_scaling_factor;      /* multiplies the routed weights (2.5) */
  float swiglu_limit;               /* > 0: clamp routed activations to [-limit, limit] */
  float shared_swiglu_limit;        /* > 0: clamp shared-expert activations */
  int32_t expert_weight_format;     /* moe_weight_format_t of the routed experts */
  int32_t expert_act_format;        /* moe_act_format_t of the routed experts (0: bf16) */
} moe_config_t;

/* Expert weights, all device pointers, PyTorch [out_features, in_features] layout.
 *   MOE_WEIGHTS_BF16:  gate [E,I,H], up [E,I,H], down [E,H,I] bf16; *_scale NULL.
 *   MOE_WEIGHTS_MXFP4: gate [E,I,H/2], up [E,I,H/2], down [E,H,I/2] uint8, two e2m1
 *                      codes per byte (low nibble = even k, nibble = sign<<3 | code),
 *                      gate_scale/up_scale [E,I,H/32], down_scale [E,H,I/32] e8m0
 *                      bytes (value = e2m1 * 2^(scale-127), one scale per 32 k).
 *   MOE_WEIGHTS_MXFP8: gate [E,I,H], up [E,I,H], down [E,H,I] uint8 E4M3 codes (OCP FP8:
 *                      sign<<7 | exponent (bias 7)<<3 | mantissa; 0x7f/0xff NaN, never
 *                      given), scales as for MXFP4 (value = e4m3 * 2^(scale-127)).
 *   MOE_WEIGHTS_MXFP4_TILED: the MXFP4 arrays (same values, same sizes) in the order the
 *                      expert kernels read them, written by moe_pack_mxfp4; needs H and I
 *                      multiples of 256.  Each matrix [N, Kd] (gate, up: N = I, Kd = H;
 *                      down: N = H, Kd = I) is stored in blocks of 16 rows:
 *                      codes: 1 KB per 16 rows x 128 values, block (b, s) at byte
 *                        (b*(Kd/128) + s)*1024; in it, the 16 bytes at 16*(16*q + r) hold
 *                        row 16b + r's values k = 128s + 32q .. +31 (two per byte, low
 *                        nibble first), q = 0..3, r = 0..15;
 *                      scales: 128 bytes per 16 rows x 256 values, block (b, t) at byte
 *                        (b*(Kd/256) + t)*128; in it, byte 8*r + i is the scale of row
 *                        16b + r's 32-value block 8t + i.
 *                      A 16-lane x 4 load then reads 1 KB of contiguous codes per step (the
 *                      row-major layout spreads it over 16 rows' half cache lines).
 *   MOE_WEIGHTS_MXFP8_TILED: the MXFP8 arrays in the same manner (moe_pack_mxfp8; H and I
 *                      multiples of 256): codes 2 KB per 16 rows x 128 values, block (b, s) at
 *                      byte (b*(Kd/128) + s)*2048; in it, the 16 bytes at 1024*p + 16*(16*q + r)
 *                      hold row 16b + r's values k = 128s + 64p + 16q .. +15 (p = 0, 1: the
 *                      scaled MFMA's E4M3 operand halves); scales as for MOE_WEIGHTS_MXFP4_TILED.
 *   Shared expert (bf16, required when S == 1, else ignored):
 *                      shared_gate [I,H], shared_up [I,H], shared_down [H,I]. */
typedef struct {
  const void* gate;
  const void* up;
  const void* down;
  const uint8_t* gate_scale;
  const uint8_t* up_scale;
  const uint8_t* down_scale;
  const void* shared_gate;
  const void* shared_up;
  const void* shared_down;
} moe_expert_weights_t;

/* Bytes of device workspace that any entry point needs for T tokens (host call). */
moe_status_t moe_workspace_size(const moe_config_t* cfg, int64_t T, size_t* bytes);

/* Router (sections 三.1-三.3 and 四 of the routing walk-through page).
 *   x           device bf16 [T,H]   hidden states
 *   router_w    device fp32 [E,H]   router weight
 *   expert_bias device fp32 [E]     selection bias; NULL means no bias
 *   topk_idx    device int32 [T,K]  chosen experts of each token, ascending id
 *   topk_w      device fp32 [T,K]   their mixing weights, same order
 *   ws          device workspace of at least moe_workspace_size() bytes
 * Logits are computed in fp32 (bf16 x times fp32 W_r, fp32 accumulation); sigmoid,
 * bias, group scores and the selection are fp32.  Exact ties go to the lower group or
 * expert index.  The weight of a chosen expert is its unbiased sigmoid score. */
moe_status_t moe_route(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                       const float* expert_bias, int32_t* topk_idx, float* topk_w, void* ws,
                       size_t ws_bytes, void* stream);

/* Dispatch: group the T*K (token, slot) pairs by expert.
 *   topk_idx       device int32 [T,K] (each token's K ids distinct and in [0,E);
 *                  out-of-range ids are ignored: their slot gets inv_perm = -1 and they
 *                  are in no count)
 *   expert_counts  device int32 [E+1] tokens per expert; entry E = shared expert (T*S)
 *   expert_offsets device int32 [E+2] offsets[e] = sum of counts[0..e-1] for e < E;
 *                  offsets[E] = T*K and offsets[E+1] = T*K + T*S always
 *   sorted_token   device int32 [P]   positions offsets[e]..offsets[e]+counts[e]-1 hold the
 *                  tokens of expert e in ascending order; the shared expert's block
 *                  (from T*K) holds 0..T-1; positions no token fills (those of ignored
 *                  pairs, at the end of the last routed expert's range) hold -1
 *   inv_perm       device int32 [T,K] sorted position of each (token, slot) */
moe_status_t moe_dispatch(const moe_config_t* cfg, int64_t T, const int32_t* topk_idx,
                          int32_t* expert_counts, int32_t* expert_offsets, int32_t* sorted_token,
                          int32_t* inv_perm, void* ws, size_t ws_bytes, void* stream);

/* Expert FFNs (section 二 and 四): for every sorted position p of expert e and token
 * t = sorted_token[p],  y_sorted[p] = down_e( clamp( silu(gate_e x_t) * up_e x_t ) ).
 *   x              device bf16 [T,H]
 *   expert_offsets device int32 [E+2], sorted_token device int32 [P] (from moe_dispatch)
 *   weights        host pointer to the device weight table above
 *   y_sorted       device fp32 [P,H]  (rows of the shared expert at T*K + t)
 * gate/up runs on bf16 MFMA with fp32 accumulation.  The activation between the two
 * products is kept as one fp16 plane (11 significant bits) for bf16 and MXFP8 expert
 * weights, whose down product then runs on fp16 MFMA with the weights converted (bf16) or
 * decoded (MXFP8) exactly to fp16; as one bf16 plane for MXFP4 weights with bf16
 * activations; as MXFP8 with MXFP8 activations.  Block-format gate/up weights are decoded
 * exactly to bf16 in registers. */
moe_status_t moe_expert_ffn(const moe_config_t* cfg, int64_t T, const void* x,
                            const int32_t* expert_offsets, const int32_t* sorted_token,
                            const moe_expert_weights_t* weights, void* y_sorted, void* ws,
                            size_t ws_bytes, void* stream);

/* Combine: out[t] = sum_k topk_w[t,k] * y_sorted[inv_perm[t,k]]  (k ascending, fp32)
 *                   + y_sorted[T*K + t] when S == 1,   rounded once to bf16.
 *   y_sorted device fp32 [P,H], inv_perm device int32 [T,K], topk_w device fp32 [T,K],
 *   out device bf16 [T,H].  Slots with inv_perm < 0 contribute nothing. */
moe_status_t moe_combine(const moe_config_t* cfg, int64_t T, const void* y_sorted,
                         const int32_t* inv_perm, const float* topk_w, void* out, void* stream);

/* The whole layer: route, dispatch, expert FFNs, combine.
 *   out                device bf16 [T,H]
 *   topk_idx_out, topk_w_out, expert_counts_out: optional device copies of the
 *   routing ([T,K] int32, [T,K] fp32, [E+1] int32); NULL to skip.
 * Equivalent to the four calls above in order, with the same results bit for bit.
 * With block-format experts and a shared expert, the shared expert's kernels (which read x
 * only) run on a second stream of the library's, created once per device on its first such
 * call (default priority), forked from `stream` before the router and joined back into
 * `stream` before the combine: everything the call enqueues is still ordered after the
 * work already on `stream` and before the work enqueued on it afterwards. */
moe_status_t moe_forward(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                         const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                         int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out,
                         void* ws, size_t ws_bytes, void* stream);

/* Dense SwiGLU FFN, the layers before the MoE stack (routing walk-through page, section 二:
 * first_k_dense_replace = 2, the first two of the 42 layers use an ordinary dense FFN; the
 * page gives no intermediate size, so it is a parameter, and the FFN is read as the experts'
 * own SwiGLU form):  out[t] = ( silu(x[t] gate^T) * (x[t] up^T) ) down^T, the activation
 * clamped to +-swiglu_limit when it is > 0, fp32 accumulation, one rounding to bf16.
 * Up to 10 tokens it runs on two kernels of its own (gate/up, then down writing out); up to
 * 4096, on the kernels of moe_expert_ffn with tiles computed from T and the output written by
 * the down GEMM (or, up to 512 tokens, by a last kernel adding the down GEMM's split
 * reduction in order); above, as a layer with a single routed expert that every token takes with
 * weight 1, on the kernels of moe_expert_ffn and moe_combine.  Up to 10 tokens h is kept as
 * two bf16 planes (about 16 significand bits), above as one fp16 plane (11); every path sums
 * in a fixed order.
 *   x device bf16 [T,H]; gate, up device bf16 [I,H]; down device bf16 [H,I]; out device
 *   bf16 [T,H]; ws device, 256-byte aligned, moe_dense_ffn_workspace_size bytes.
 *   H and I multiples of 128 (MOE_ERR_UNSUPPORTED otherwise); T = 0 is a no-op.
 * Results are deterministic. */
moe_status_t moe_dense_ffn_workspace_size(int32_t hidden_size, int32_t intermediate_size, int64_t T,
                                          size_t* bytes);
moe_status_t moe_dense_ffn(int32_t hidden_size, int32_t intermediate_size, float swiglu_limit, int64_t T,
                           const void* x, const void* gate, const void* up, const void* down, void* out,
                           void* ws, size_t ws_bytes, void* stream);

/* MXFP8 rounding of bf16 activations, the step the MOE_ACT_MXFP8 path applies to x before
 * the routed experts' gate/up products (the same device code rounds h in the gate/up
 * epilogue): for each block of 32 consecutive values of a row, scale = 2^X with
 * X = floor(log2 max|v|) - 8 clamped to [-127, 127] (-127 for an all-zero block), and each
 * v / 2^X rounded to the nearest E4M3 value, ties to even, saturated at 448 (OCP MX v1.0).
 *   x       device bf16 [rows, cols]; cols a positive multiple of 32
 *   codes   device uint8 [rows, cols]     E4M3 codes (16-byte aligned)
 *   scales  device uint8 [rows, cols/32]  e8m0 bytes X + 127
 * Enqueued on `stream`; rows = 0 is a no-op. */
moe_status_t moe_quantise_mxfp8(const void* x, int64_t rows, int32_t cols, uint8_t* codes, uint8_t* scales,
                                void* stream);

/* MXFP4 weights from the row-major MOE_WEIGHTS_MXFP4 arrays into MOE_WEIGHTS_MXFP4_TILED
 * order (the layout above), for `mats` consecutive matrices of N x Kd values each; weights
 * are static, so this runs once when they are loaded (the hybrid-attention page, table
 * 模型一览, gives the routed experts in MXFP4; their memory order is not fixed there).
 *   codes      device uint8 [mats, N, Kd/2]   row-major E2M1 codes (16-byte aligned)
 *   scales     device uint8 [mats, N, Kd/32]  row-major e8m0 scales (8-byte aligned)
 *   codes_out  device uint8, mats * N * Kd/2 bytes (16-byte aligned; must not overlap codes)
 *   scales_out device uint8, mats * N * Kd/32 bytes (8-byte aligned; must not overlap scales)
 *   N          multiple of 16; Kd multiple of 256
 * MOE_ERR_INVALID_ARG for a NULL pointer, bad sizes or overlapping buffers, MOE_ERR_ALIGNMENT
 * for a misaligned pointer; mats = 0 is a no-op.  Enqueued on `stream`. */
moe_status_t moe_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t mats, int32_t N, int32_t Kd,
                            uint8_t* codes_out, uint8_t* scales_out, void* stream);

/* The same for MXFP8 weights (MOE_WEIGHTS_MXFP8 -> MOE_WEIGHTS_MXFP8_TILED): codes [mats, N, Kd]
 * (one E4M3 code per byte) and scales [mats, N, Kd/32], outputs of the same sizes; the same
 * requirements and errors as moe_pack_mxfp4. */
moe_status_t moe_pack_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t mats, int32_t N, int32_t Kd,
                            uint8_t* codes_out, uint8_t* scales_out, void* stream);

/* Expert-bias update, the step after the layer in training (routing walk-through page,
 * section 三.3: every routed expert's selection bias is lowered when it is busy and raised
 * when it is idle, balancing the load without an auxiliary loss).  The page gives neither the
 * rule nor the rate; this library takes the sign rule with a caller-chosen step gamma:
 *   bias[e] += gamma   if counts[e] * E < sum(counts)   (below the mean count)
 *   bias[e] -= gamma   if counts[e] * E > sum(counts)   (above it; unchanged at the mean)
 * computed as bias[e] + gamma * (+1 | -1 | 0) in fp32, the decision taken in integers.
 *   expert_counts  device int32 [E]: the routed counts of a step (the first E entries of the
 *                  expert_counts of moe_dispatch or moe_forward; the shared expert's is not read)
 *   expert_bias    device fp32 [E], updated in place (the array moe_route/moe_forward read)
 *   gamma          the step; any finite value (MOE_ERR_INVALID_ARG otherwise)
 * Enqueued on `stream`; it reads the counts when it runs, so it may follow the forward that
 * writes them on the same stream without a host synchronisation. */
moe_status_t moe_update_expert_bias(const moe_config_t* cfg, const int32_t* expert_counts,
                                    float* expert_bias, float gamma, void* stream);

/* moe_forward with a timing trace, for profiling (same results).  events[0] is recorded on
 * `stream` before the first kernel and events[i+1] right after the i-th kernel launch; the
 * caller creates the events (hipEvent_t, passed as void*) and later reads the elapsed times;
 * a NULL entry records nothing (each recorded event costs a few microseconds of queue time,
 * so a caller timing one kernel passes only the two events around it).
 * kernel_names (host array of max_events - 1 pointers) receives static kernel names and
 * *n_kernels the number of kernels launched.  Returns MOE_ERR_INVALID_ARG (after running
 * the layer) if max_events is smaller than n_kernels + 1. */
moe_status_t moe_forward_traced(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                                const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                                void* ws, size_t ws_bytes, void* stream, void* const* events,
                                int32_t max_events, const char** kernel_names, int32_t* n_kernels);

/* moe_forward with one kernel timed by events bound to its own dispatch (the AMD launch
 * extension hipExtLaunchKernel): start_event and stop_event (hipEvent_t created by the caller,
 * passed as void*) take that kernel's start and end times, and no other queue packets are
 * added, so the step runs as fast as moe_forward (same results).  kernel_index counts the
 * kernels in the order moe_forward_traced names them (0 = the first); a step that launches
 * several kernels under one name is timed by its first.  Returns MOE_ERR_INVALID_ARG (after
 * running the layer) if the forward launched no kernel with that index. */
moe_status_t moe_forward_timed(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                               const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                               void* ws, size_t ws_bytes, void* stream, int32_t kernel_index,
                               void* start_event, void* stop_event);

/* moe_forward without a caller workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments and results as moe_forward (bit for bit), minus ws/ws_bytes: the workspace
 * is a static device array inside the library, 64 MiB on each GPU the library runs on, held
 * until the process ends (its device address is looked up on the first call on a device,
 * which must be current).  The call allocates nothing.  T whose workspace
 * (moe_workspace_size) exceeds 64 MiB is rejected with MOE_ERR_WORKSPACE before anything is
 * enqueued: for the full-size layer (hidden 2560, 512 experts, intermediate 768) that is T
 * above about 970 tokens.  Every call on one GPU uses the same array and leaves its contents
 * behind (each call rewrites what it reads), so calls that overlap on one GPU -- on
 * different streams, or from different threads without ordering -- race. */
moe_status_t moe_forward_noalloc(const moe_config_t* cfg, int64_t T, const void* x, const float* router_w,
                                 const float* expert_bias, const moe_expert_weights_t* weights, void* out,
                                 int32_t* topk_idx_out, float* topk_w_out, int32_t* expert_counts_out,
                                 void* stream);

/* Static text for a status code. */
const char* moe_status_string(moe_status_t status);

/* Description of the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H_ */
