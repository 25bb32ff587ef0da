"""CPU oracle for the forward pass of one BailingMoeV3 sparse MoE layer.

TEST INFRASTRUCTURE ONLY.  This is the plain, slow, float64 definition of what the
layer computes, used to check the HIP library.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import it; the library never calls it and
shares no code with it.

Sources (the Ling-3.0-flash(-VL) web pages; no code was published with them):
  [R]  routing walk-through page (lqnn.cn, "Ling-3.0-flash-VL ... MoE 稀疏路由机制"):
       section 二 (512 routed experts + 1 always-on shared expert; gate/up/down,
       hidden 2560, moe_intermediate_size 768), section 三.1 (router logits through an
       element-wise sigmoid, score_function "sigmoid"), 三.2 (n_group 8 groups of 64,
       keep topk_group 4 groups by in-group maximum, then num_experts_per_tok 8 out of
       the 256 candidates), 三.3 (per-expert bias, moe_router_enable_expert_bias),
       四 (router_dtype fp32, routed_scaling_factor 2.5, norm_topk_prob, SwiGLU limit
       list: +-4 routed, +-5/+-7 shared, on the last layers).
  [Q]  hybrid-attention page (lpnh.cn, "Ling-3.0-flash-VL ... 5:1 混合"), table
       "模型一览": routed-expert weights in 4-bit MXFP4.
  [F]  Ling-3.0-flash architecture page (wmrh.cn, "5.1B激活参数的AI革命"), section
       "稀疏MoE设计": BailingMoeV3SparseMoeBlock, 512 routed + 1 shared, 8 active.

Readings of points the pages leave open (each one is a parameter or a documented
choice below): group score = max of the biased scores in the group; groups and
experts are chosen on the biased score c = sigmoid(l) + b, the mixing weight uses
the unbiased sigmoid score; experts outside the kept groups can never be chosen;
exact ties go to the lower index; renormalise, then scale; the SwiGLU limit clamps
the activation a = silu(g) * u symmetrically; the chosen experts of a token are
listed in ascending expert id and summed in that order, shared expert last.

Routing decisions are taken in fp32, the precision the pages fix for the router
([R] section 四): each stage's exact value is rounded to fp32 (logit, sigmoid score,
biased score) before any comparison.  Everything else is float64.
"""
from __future__ import annotations

import dataclasses
from typing import Callable, Optional

import numpy as np


# ----------------------------------------------------------------------------------
# input formats
# ----------------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit pattern -> exact float64 value (bf16 is the top half of an fp32)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# e2m1 code -> magnitude: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
# code 0 is zero, code 1 the subnormal 0.5, codes 2..7 are (1 + m/2) * 2^(e-1).
def _e2m1_magnitude(code: np.ndarray) -> np.ndarray:
    e = (code >> 1) & 3
    m = code & 1
    normal = (1.0 + 0.5 * m) * np.exp2(e - 1.0)
    sub = 0.5 * m
    return np.where(e == 0, sub, normal)


def mxfp4_dequant(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 weight -> float64 [N, K] ([Q] table 模型一览; block format: one e8m0 scale
    per 32 consecutive K values, value = e2m1 * 2^(scale - 127); low nibble = even k)."""
    packed = np.asarray(packed, dtype=np.uint8)
    N, Kh = packed.shape
    nib = np.empty((N, Kh * 2), dtype=np.uint8)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    mag = _e2m1_magnitude(nib.astype(np.int64))
    val = np.where(nib & 8, -mag, mag)
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)          # [N, K/32]
    return val * np.repeat(sc, 32, axis=1)


# FP8 E4M3 (OCP 8-bit floating point, as used by the OCP MX v1.0 MXFP8 format): sign bit 7,
# exponent bits 6..3 (bias 7), mantissa bits 2..0; exponent 0 is subnormal (m/8 * 2^-6); the
# all-ones exponent with all-ones mantissa is NaN and there are no infinities, so the largest
# finite magnitude is 1.75 * 2^8 = 448.
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest normal value


def e4m3_value(code: np.ndarray) -> np.ndarray:
    """E4M3 code (uint8) -> float64 value (NaN for 0x7F / 0xFF)."""
    c = np.asarray(code, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def mxfp8_dequant(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 (E4M3 elements, one e8m0 scale per 32 consecutive values of the last axis) ->
    float64: value = e4m3 * 2^(scale - 127)."""
    v = e4m3_value(codes)
    sc = np.exp2(np.asarray(scales, dtype=np.float64) - 127.0)
    return v * np.repeat(sc, 32, axis=-1)


# the 127 non-negative finite E4M3 values, indexed by their code (ascending)
_E4M3_GRID = e4m3_value(np.arange(127))


def mxfp8_quantise(a: np.ndarray):
    """float64 [..., K] -> (E4M3 codes uint8 [..., K], e8m0 scales uint8 [..., K/32]).

    The OCP MX v1.0 conversion for E4M3 elements, per block of 32 consecutive values of the
    last axis: shared exponent X = floor(log2(max |v|)) - 8 (8 = the exponent of E4M3's
    largest normal value), clamped to the e8m0 range [-127, 127] (-127 for an all-zero
    block); each v / 2^X rounded to the nearest E4M3 value, ties to the even code, and
    magnitudes beyond 448 saturated to 448."""
    a = np.asarray(a, dtype=np.float64)
    K = a.shape[-1]
    assert K % 32 == 0
    blk = a.reshape(a.shape[:-1] + (K // 32, 32))
    amax = np.abs(blk).max(axis=-1)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - E4M3_EMAX, -127)
    X = np.clip(X, -127, 127).astype(np.int64)
    mag = np.abs(blk) / np.exp2(X.astype(np.float64))[..., None]
    # nearest grid value: i = number of grid values <= mag, so mag lies in [grid[i-1], grid[i])
    i = np.searchsorted(_E4M3_GRID, mag, side="right")
    lo = np.clip(i - 1, 0, 126)
    hi = np.clip(i, 0, 126)
    dlo, dhi = mag - _E4M3_GRID[lo], _E4M3_GRID[hi] - mag
    code = np.where(dhi < dlo, hi, np.where(dlo < dhi, lo, np.where(lo % 2 == 0, lo, hi)))
    code = np.where(mag >= E4M3_MAX, 126, code)          # saturate (126 is 448)
    neg = (blk < 0) & (code != 0)
    codes = (code | (neg.astype(np.int64) << 7)).astype(np.uint8).reshape(a.shape)
    return codes, (X + 127).astype(np.uint8)


def act_mxfp8(a: np.ndarray) -> np.ndarray:
    """The values an MXFP8 matrix product sees for the activations a (last axis = the
    reduction axis): a quantised to MXFP8 and decoded again."""
    return mxfp8_dequant(*mxfp8_quantise(a))


# ----------------------------------------------------------------------------------
# routing ([R] sections 三.1-三.3, 四)
# ----------------------------------------------------------------------------------
@dataclasses.dataclass
class Routing:
    topk_idx: np.ndarray     # [T, K] int64, ascending expert id per token
    topk_w: np.ndarray       # [T, K] float64 mixing weights
    counts: np.ndarray       # [E] tokens per routed expert
    scores: np.ndarray       # [T, E] sigmoid score s (as compared, fp32-rounded in fp32 mode)
    choice: np.ndarray       # [T, E] biased score c = s + b (as compared)
    kept_groups: np.ndarray  # [T, TG] kept group ids, best first
    gap_group: np.ndarray    # [T] score gap between the last kept and the first dropped group
    gap_expert: np.ndarray   # [T] gap between the K-th and (K+1)-th candidate
    near_tie: np.ndarray     # [T] bool, min gap < tie_eps


def router_logits(x: np.ndarray, router_w: np.ndarray) -> np.ndarray:
    """l = x W_r^T, [T,H] x [E,H] -> [T,E], float64 ([R] 三.1: one raw score per expert
    from the hidden state; 四: router in fp32, and fp32/bf16 inputs are exact in fp64)."""
    return np.asarray(x, np.float64) @ np.asarray(router_w, np.float64).T


def _f32(a):
    return np.asarray(a, np.float64).astype(np.float32).astype(np.float64)


def route(logits: np.ndarray, bias: Optional[np.ndarray], n_group: int, topk_group: int,
          top_k: int, routed_scaling_factor: float = 2.5, norm_topk_prob: bool = True,
          decision: str = "fp32", tie_eps: float = 1e-6) -> Routing:
    """Grouped top-k routing of every token.

    Steps, in the order the routing page gives them:
      1. s = sigmoid(l), one independent score per expert ([R] 三.1);
      2. c = s + b with the per-expert selection bias ([R] 三.3);
      3. split the E experts into n_group equal groups; score each group by the
         maximum c inside it and keep the topk_group best groups ([R] 三.2 step 1);
      4. among the experts of the kept groups pick the top_k largest c ([R] 三.2
         step 2); experts of dropped groups are never eligible;
      5. mixing weight = the unbiased s of each chosen expert, renormalised to sum
         to 1 if norm_topk_prob, then multiplied by routed_scaling_factor ([R] 四).
    Ties go to the lower group / expert index.  decision="fp32" rounds l, s and c
    to fp32 before they are compared (router_dtype fp32, [R] 四); "fp64" keeps them
    exact."""
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    assert E % n_group == 0 and 1 <= topk_group <= n_group
    per = E // n_group
    assert 1 <= top_k <= topk_group * per
    b = np.zeros(E) if bias is None else np.asarray(bias, np.float64)
    if decision == "fp32":
        l = _f32(l)
        s = _f32(1.0 / (1.0 + np.exp(-l)))
        c = (s.astype(np.float32) + _f32(b).astype(np.float32)).astype(np.float64)
    elif decision == "fp64":
        s = 1.0 / (1.0 + np.exp(-l))
        c = s + b
    else:
        raise ValueError(decision)

    # group scores and kept groups (stable sort: equal scores keep ascending index)
    gscore = c.reshape(T, n_group, per).max(axis=2)
    gorder = np.argsort(-gscore, axis=1, kind="stable")
    kept = gorder[:, :topk_group]
    keep_mask = np.zeros((T, n_group), dtype=bool)
    np.put_along_axis(keep_mask, kept, True, axis=1)
    eligible = np.repeat(keep_mask, per, axis=1)

    cand = np.where(eligible, c, -np.inf)
    eorder = np.argsort(-cand, axis=1, kind="stable")
    chosen = np.sort(eorder[:, :top_k], axis=1)          # ascending expert id

    s_sel = np.take_along_axis(s, chosen, axis=1)
    w = s_sel / s_sel.sum(axis=1, keepdims=True) if norm_topk_prob else s_sel.copy()
    w = w * routed_scaling_factor

    gs = np.take_along_axis(gscore, gorder, axis=1)
    gap_g = gs[:, topk_group - 1] - gs[:, topk_group] if topk_group < n_group else np.full(T, np.inf)
    n_cand = topk_group * per
    cs = np.take_along_axis(cand, eorder, axis=1)
    gap_e = cs[:, top_k - 1] - cs[:, top_k] if top_k < n_cand else np.full(T, np.inf)
    counts = np.bincount(chosen.ravel(), minlength=E)
    return Routing(chosen, w, counts, s, c, kept, gap_g, gap_e, np.minimum(gap_g, gap_e) < tie_eps)


# ----------------------------------------------------------------------------------
# dispatch: plain definitions of histogram, exclusive scan and stable permutation
# ----------------------------------------------------------------------------------
@dataclasses.dataclass
class Dispatch:
    counts: np.ndarray        # [E+1] tokens per expert; entry E = shared expert (T or 0)
    offsets: np.ndarray       # [E+2] exclusive prefix sum of counts
    sorted_token: np.ndarray  # [T*K + T*S] token of each sorted position
    inv_perm: np.ndarray      # [T, K] sorted position of (token, slot)


def dispatch(topk_idx: np.ndarray, num_experts: int, num_shared: int = 1) -> Dispatch:
    """Group the (token, slot) pairs by expert: positions [offsets[e], offsets[e] + counts[e])
    hold expert e's tokens in ascending token order; the shared expert is expert E, owns every
    token in order and always starts at position T*K.

    A pair whose id lies outside [0, E) is ignored (the pages never produce one; this is the
    library's stated contract for such input): it is in no expert's count, its inv_perm is -1,
    and the positions it would have taken, counts[:E].sum() .. T*K-1, hold no token (-1) and
    belong to the last routed expert's range offsets[E-1] .. offsets[E]."""
    T, K = topk_idx.shape
    flat = np.asarray(topk_idx, np.int64).ravel()
    valid = (flat >= 0) & (flat < num_experts)
    counts = np.zeros(num_experts + 1, dtype=np.int64)
    counts[:num_experts] = np.bincount(flat[valid], minlength=num_experts)
    counts[num_experts] = T if num_shared else 0
    offsets = np.zeros(num_experts + 2, dtype=np.int64)
    offsets[1:num_experts + 1] = np.cumsum(counts[:num_experts])
    offsets[num_experts] = T * K
    offsets[num_experts + 1] = T * K + counts[num_experts]
    pairs = np.nonzero(valid)[0]
    order = pairs[np.argsort(flat[pairs], kind="stable")]   # by expert, then by flat index t*K+k
    routed_tok = np.full(T * K, -1, dtype=np.int64)
    routed_tok[:order.size] = order // K
    sorted_token = np.concatenate([routed_tok, np.arange(T) if num_shared else np.zeros(0, np.int64)])
    inv = np.full(T * K, -1, dtype=np.int64)
    inv[order] = np.arange(order.size)
    return Dispatch(counts, offsets, sorted_token, inv.reshape(T, K))


# ----------------------------------------------------------------------------------
# expert FFN ([R] 二, 四) and combine
# ----------------------------------------------------------------------------------
def swiglu(g: np.ndarray, u: np.ndarray, limit: float = 0.0) -> np.ndarray:
    """a = silu(g) * u, silu(z) = z / (1 + e^-z); limit > 0 clamps a to [-limit, limit]."""
    a = g / (1.0 + np.exp(-g)) * u
    if limit and limit > 0:
        a = np.clip(a, -limit, limit)
    return a


def expert_hidden(xrows, gate, up, limit=0.0):
    """h = swiglu(x W_gate^T, x W_up^T): [n,H] -> [n,I]."""
    return swiglu(xrows @ gate.T, xrows @ up.T, limit)


def expert_forward(xrows, gate, up, down, limit=0.0, act_quant: str = "none"):
    """One SwiGLU expert ([R] 二: three matrices gate / up / down): [n,H] -> [n,H].

    act_quant="mxfp8": the expert's two matrix products take MXFP8 activations (the
    8-bit-activation reading of [Q] table 模型一览's "FP8 + MXFP4"): x is rounded to MXFP8
    along H before gate/up, and h (after SwiGLU and the clamp) along I before down."""
    if act_quant == "none":
        return expert_hidden(xrows, gate, up, limit) @ down.T
    if act_quant != "mxfp8":
        raise ValueError(act_quant)
    h = expert_hidden(act_mxfp8(xrows), gate, up, limit)
    return act_mxfp8(h) @ down.T


ExpertGetter = Callable[[int], tuple]   # e -> (gate [I,H], up [I,H], down [H,I]) float64


def moe_layer(x: np.ndarray, router_w: np.ndarray, bias: Optional[np.ndarray],
              get_expert: ExpertGetter, shared: Optional[tuple], *, n_group: int,
              topk_group: int, top_k: int, routed_scaling_factor: float = 2.5,
              norm_topk_prob: bool = True, swiglu_limit: float = 0.0,
              shared_swiglu_limit: float = 0.0, decision: str = "fp32", act_quant: str = "none"):
    """Forward of the whole block: route, run each chosen expert on its tokens, sum the
    weighted outputs per token in ascending expert order, add the shared expert.
    act_quant applies to the routed experts only (see expert_forward); the shared expert
    always takes the exact activations.  Returns (out [T,H] float64, Routing)."""
    x = np.asarray(x, np.float64)
    T, H = x.shape
    r = route(router_logits(x, router_w), bias, n_group, topk_group, top_k,
              routed_scaling_factor, norm_topk_prob, decision)
    out = np.zeros((T, H))
    for e in np.unique(r.topk_idx):
        tok, slot = np.nonzero(r.topk_idx == e)
        g, u, d = get_expert(int(e))
        y = expert_forward(x[tok], g, u, d, swiglu_limit, act_quant)
        out[tok] += r.topk_w[tok, slot][:, None] * y
    if shared is not None:
        out += expert_forward(x, *shared, shared_swiglu_limit)
    return out, r


# ----------------------------------------------------------------------------------
# expert-bias update (the step after the layer in training)
# ----------------------------------------------------------------------------------
def update_expert_bias(bias: np.ndarray, counts: np.ndarray, gamma: float) -> np.ndarray:
    """[R] section 三.3: every routed expert carries a selection bias that is lowered for
    experts that receive many tokens and raised for those that receive few, so that the load
    evens out without an auxiliary loss.  The page gives neither the rule nor the rate; the
    reading taken here is the sign rule with a fixed step gamma: an expert above the mean
    count moves down by gamma, one below it moves up by gamma, one exactly at the mean stays.
    "Above the mean" is decided in integers (count_e * E against the total of the E counts),
    so no rounding enters the decision; the bias is router state, kept in fp32 ([R] section
    四), so the new value is the fp32 sum bias + (+-gamma).

    bias: [E] fp32; counts: the E routed counts (a longer array, such as the [E+1] counts
    with the shared expert last, is cut to E)."""
    b = np.asarray(bias, dtype=np.float32)
    E = b.shape[0]
    c = np.asarray(counts, dtype=np.int64)[:E]
    side = np.sign(c.sum() - E * c)  # +1 below the mean, -1 above, 0 at the mean
    step = np.float32(gamma) * side.astype(np.float32)
    return (b + step).astype(np.float32)
