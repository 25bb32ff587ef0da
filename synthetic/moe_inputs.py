"""Seeded synthetic inputs for one BailingMoeV3 sparse MoE layer.

This module only *draws* inputs: activations, router weight, expert bias and expert
weights (bf16 bit patterns, plus an MXFP4 encoding of them for the quantised-expert
workload).  It holds none of the layer's arithmetic, so both the CPU oracle and the
HIP path may take their inputs from here without sharing any compute code.

Shapes and distributions follow the layer the Ling-3.0-flash(-VL) pages describe
(routing walk-through page, lqnn.cn "MoE 稀疏路由", section 二: hidden 2560, 512
routed experts of intermediate 768, one shared expert) and the five synthetic
workloads this repository measures:

  tiny     T=32,    H=512,  E=64,  I=128, 8 groups / top-4 groups / top-8
  decode   T=64,    H=2560, E=512, I=768
  prefill  T=8192,  same layer
  skewed   T=16384, tokens from 16 Gaussian clusters, bias N(0, 0.5),
           SwiGLU clamp 4 (routed) / 7 (shared)
  mxfp4    T=4096,  routed expert weights in MXFP4 (e2m1 + e8m0 per 32 along K)

Randomness: every tensor (and every expert, and every 64-row block of tokens) has
its own numpy ``SeedSequence(seed, spawn_key=(tag, index))`` stream.  That makes a
single expert's weights reproducible without drawing all 512, lets the bulk draw
run on many threads, and makes the first T' rows of x identical for any T >= T'.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

# stream tags (first element of the SeedSequence spawn key)
TAG_X, TAG_ROUTER, TAG_BIAS, TAG_GATE, TAG_UP, TAG_DOWN = 0, 1, 2, 3, 4, 5
TAG_SH_GATE, TAG_SH_UP, TAG_SH_DOWN, TAG_CENTRES, TAG_CLUSTER = 6, 7, 8, 9, 10
X_BLOCK = 64  # token rows per x stream


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """One synthetic workload.  Field names follow the model's text_config."""
    name: str
    T: int                      # tokens (batch x sequence, flattened)
    hidden_size: int            # H
    num_experts: int            # E routed experts
    moe_intermediate_size: int  # I
    shared_intermediate_size: int  # I_s
    n_group: int                # G
    topk_group: int             # TG
    num_experts_per_tok: int    # K
    routed_scaling_factor: float = 2.5
    norm_topk_prob: bool = True
    num_shared_experts: int = 1
    swiglu_limit: float = 0.0          # <= 0: no clamp
    shared_swiglu_limit: float = 0.0   # <= 0: no clamp
    weight_format: str = "bf16"        # "bf16" | "mxfp4" | "mxfp8" (routed experts only)
    act_format: str = "bf16"           # "bf16" | "mxfp8": activations of the routed experts' products
    x_dist: str = "normal"             # "normal" | "clusters"
    bias_dist: str = "uniform"         # "uniform" U(-0.1,0.1) | "normal" N(0,0.5) | "zero"
    weight_std: float = 0.02
    n_clusters: int = 16
    cluster_spread: float = 0.3

    # short aliases used throughout the tests
    @property
    def H(self): return self.hidden_size
    @property
    def E(self): return self.num_experts
    @property
    def I(self): return self.moe_intermediate_size
    @property
    def I_s(self): return self.shared_intermediate_size
    @property
    def G(self): return self.n_group
    @property
    def TG(self): return self.topk_group
    @property
    def K(self): return self.num_experts_per_tok

    def with_(self, **kw) -> "LayerShape":
        return dataclasses.replace(self, **kw)


_FULL = dict(hidden_size=2560, num_experts=512, moe_intermediate_size=768,
             shared_intermediate_size=768, n_group=8, topk_group=4, num_experts_per_tok=8)

CONFIGS = {
    "tiny": LayerShape("tiny", T=32, hidden_size=512, num_experts=64, moe_intermediate_size=128,
                       shared_intermediate_size=128, n_group=8, topk_group=4, num_experts_per_tok=8),
    "decode": LayerShape("decode", T=64, **_FULL),
    "prefill": LayerShape("prefill", T=8192, **_FULL),
    "skewed": LayerShape("skewed", T=16384, **_FULL, swiglu_limit=4.0, shared_swiglu_limit=7.0,
                         x_dist="clusters", bias_dist="normal"),
    "mxfp4": LayerShape("mxfp4", T=4096, **_FULL, weight_format="mxfp4"),
    # the "FP8 + MXFP4" variants: routed experts in MXFP8 (bf16 activations), and MXFP4 or
    # MXFP8 routed experts with MXFP8 activations (scaled MFMA)
    "mxfp8": LayerShape("mxfp8", T=4096, **_FULL, weight_format="mxfp8"),
    "mxfp4_a8": LayerShape("mxfp4_a8", T=4096, **_FULL, weight_format="mxfp4", act_format="mxfp8"),
    "mxfp8_a8": LayerShape("mxfp8_a8", T=4096, **_FULL, weight_format="mxfp8", act_format="mxfp8"),
}


# ----------------------------------------------------------------------------------
# bf16 bit patterns (format conversion only)
# ----------------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit pattern (uint16), round to nearest even.  Inputs are finite."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    return ((u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int, tag: int, idx: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(tag, idx)))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------------
# activations, router, bias
# ----------------------------------------------------------------------------------
def gen_x(shape: LayerShape, seed: int = 0, T: int | None = None) -> np.ndarray:
    """x [T, H] as bf16 bits.  N(0,1) rows, or the 16-cluster mixture for the skewed workload."""
    T = shape.T if T is None else T
    H = shape.H
    out = np.empty((T, H), dtype=np.uint16)
    centres = None
    if shape.x_dist == "clusters":
        centres = _rng(seed, TAG_CENTRES).standard_normal((shape.n_clusters, H), dtype=np.float32)

    def block(b):
        r0, r1 = b * X_BLOCK, min(T, (b + 1) * X_BLOCK)
        rng = _rng(seed, TAG_X, b)
        noise = rng.standard_normal((X_BLOCK, H), dtype=np.float32)[: r1 - r0]
        if centres is not None:
            which = _rng(seed, TAG_CLUSTER, b).integers(0, shape.n_clusters, size=X_BLOCK)[: r1 - r0]
            noise = centres[which] + np.float32(shape.cluster_spread) * noise
        out[r0:r1] = f32_to_bf16_bits(noise)

    nb = (T + X_BLOCK - 1) // X_BLOCK
    if nb > 8:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(block, range(nb)))
    else:
        for b in range(nb):
            block(b)
    return out


def gen_router(shape: LayerShape, seed: int = 0) -> np.ndarray:
    """Router weight [E, H] float32, N(0, 0.02)."""
    w = _rng(seed, TAG_ROUTER).standard_normal((shape.E, shape.H), dtype=np.float32)
    return (w * np.float32(shape.weight_std)).astype(np.float32)


def gen_bias(shape: LayerShape, seed: int = 0) -> np.ndarray:
    """Per-expert selection bias [E] float32."""
    rng = _rng(seed, TAG_BIAS)
    if shape.bias_dist == "uniform":
        return rng.uniform(-0.1, 0.1, size=shape.E).astype(np.float32)
    if shape.bias_dist == "normal":
        return (rng.standard_normal(shape.E) * 0.5).astype(np.float32)
    if shape.bias_dist == "zero":
        return np.zeros(shape.E, dtype=np.float32)
    raise ValueError(shape.bias_dist)


# ----------------------------------------------------------------------------------
# expert weights (bf16 bits, PyTorch [out, in] layout)
# ----------------------------------------------------------------------------------
def _normal_bf16(seed, tag, idx, rows, cols, std):
    a = _rng(seed, tag, idx).standard_normal((rows, cols), dtype=np.float32)
    a *= np.float32(std)
    return f32_to_bf16_bits(a)


def gen_expert(shape: LayerShape, e: int, seed: int = 0) -> dict:
    """Routed expert e: gate [I,H], up [I,H], down [H,I] as bf16 bits (before any quantisation)."""
    I, H, s = shape.I, shape.H, shape.weight_std
    return dict(gate=_normal_bf16(seed, TAG_GATE, e, I, H, s),
                up=_normal_bf16(seed, TAG_UP, e, I, H, s),
                down=_normal_bf16(seed, TAG_DOWN, e, H, I, s))


def gen_shared(shape: LayerShape, seed: int = 0) -> dict:
    """Shared expert: gate [I_s,H], up [I_s,H], down [H,I_s] as bf16 bits."""
    I, H, s = shape.I_s, shape.H, shape.weight_std
    return dict(gate=_normal_bf16(seed, TAG_SH_GATE, 0, I, H, s),
                up=_normal_bf16(seed, TAG_SH_UP, 0, I, H, s),
                down=_normal_bf16(seed, TAG_SH_DOWN, 0, H, I, s))


def gen_experts(shape: LayerShape, seed: int = 0, threads: int | None = None) -> dict:
    """All routed experts stacked: gate [E,I,H], up [E,I,H], down [E,H,I] (bf16 bits).

    For weight_format "mxfp4" / "mxfp8" the stacked arrays are that encoding instead:
    gate_q [E,I,H/2] (MXFP4) or [E,I,H] (MXFP8), gate_s [E,I,H/32], ... (see quantise_mxfp4,
    quantise_mxfp8)."""
    E, I, H = shape.E, shape.I, shape.H
    mx = shape.weight_format in ("mxfp4", "mxfp8")
    quant = quantise_mxfp4 if shape.weight_format == "mxfp4" else quantise_mxfp8
    if mx:
        cd = 2 if shape.weight_format == "mxfp4" else 1  # values per byte
        out = dict(gate_q=np.empty((E, I, H // cd), np.uint8), gate_s=np.empty((E, I, H // 32), np.uint8),
                   up_q=np.empty((E, I, H // cd), np.uint8), up_s=np.empty((E, I, H // 32), np.uint8),
                   down_q=np.empty((E, H, I // cd), np.uint8), down_s=np.empty((E, H, I // 32), np.uint8))
    else:
        out = dict(gate=np.empty((E, I, H), np.uint16), up=np.empty((E, I, H), np.uint16),
                   down=np.empty((E, H, I), np.uint16))

    def one(e):
        w = gen_expert(shape, e, seed)
        if mx:
            for k in ("gate", "up", "down"):
                q, s = quant(w[k])
                out[k + "_q"][e], out[k + "_s"][e] = q, s
        else:
            for k in ("gate", "up", "down"):
                out[k][e] = w[k]

    with ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(one, range(E)))
    return out


def gen_expert_encoded(shape: LayerShape, e: int, seed: int = 0) -> dict:
    """One routed expert in the workload's storage format (bf16 bits or MXFP4 pieces)."""
    w = gen_expert(shape, e, seed)
    if shape.weight_format == "bf16":
        return w
    quant = quantise_mxfp4 if shape.weight_format == "mxfp4" else quantise_mxfp8
    out = {}
    for k in ("gate", "up", "down"):
        out[k + "_q"], out[k + "_s"] = quant(w[k])
    return out


# ----------------------------------------------------------------------------------
# MXFP4 encoder (input preparation for the quantised-expert workload)
# ----------------------------------------------------------------------------------
# e2m1 magnitudes indexed by the 3-bit code (exponent bias 1, one mantissa bit).
_E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_E2M1_MIDS = (_E2M1_GRID[1:] + _E2M1_GRID[:-1]) / 2


def quantise_mxfp4(w_bits: np.ndarray):
    """bf16 weight [N, K] -> (packed e2m1 uint8 [N, K/2], e8m0 scales uint8 [N, K/32]).

    Follows the OCP Microscaling (MX) v1.0 conversion: per block of 32 consecutive K
    values, shared exponent X = floor(log2(max|v|)) - 2 (2 = largest e2m1 exponent),
    each value v / 2^X rounded to the nearest e2m1 value (ties to the even code),
    saturating at +-6.  Byte layout: low nibble = even k, high nibble = odd k;
    nibble = sign<<3 | magnitude code.  An all-zero block gets X = -127."""
    v = bf16_bits_to_f32(w_bits).astype(np.float64)
    N, K = v.shape
    assert K % 32 == 0
    blk = v.reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2, -127).astype(np.int64)
    X = np.clip(X, -127, 127)
    scaled = blk / np.exp2(X.astype(np.float64))[:, :, None]
    mag = np.abs(scaled)
    # nearest grid point; c = number of midpoints strictly below |v|, so an exact
    # midpoint lands on the lower code, which is moved up when that code is odd
    c = np.searchsorted(_E2M1_MIDS, mag, side="left")
    at_mid = (c < 7) & (mag == _E2M1_MIDS[np.minimum(c, 6)]) & ((c & 1) == 1)
    code = (c + at_mid).astype(np.int64)                # |v| > 5 saturates to code 7 (= 6.0)
    sign = (scaled < 0) & (code != 0)
    nib = (code | (sign.astype(np.int64) << 3)).astype(np.uint8).reshape(N, K)
    packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    scales = (X + 127).astype(np.uint8)
    return packed, scales


def quantise_mxfp8(w_bits: np.ndarray):
    """bf16 weight [N, K] -> (E4M3 codes uint8 [N, K], e8m0 scales uint8 [N, K/32]).

    The OCP Microscaling (MX) v1.0 conversion with E4M3 elements: per block of 32 consecutive
    K values, X = floor(log2(max|v|)) - 8 (8 = the exponent of E4M3's largest normal, 448);
    each v / 2^X is rounded to nearest on the E4M3 grid of its binade (3 mantissa bits; below
    2^-6 the fixed subnormal step 2^-9), ties to even, and saturated at 448.  Code = sign<<7 |
    exponent (bias 7) << 3 | mantissa.  An all-zero block gets X = -127."""
    v = bf16_bits_to_f32(w_bits).astype(np.float64)
    N, K = v.shape
    assert K % 32 == 0
    blk = v.reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        X = np.where(amax > 0, np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 8, -127).astype(np.int64)
    X = np.clip(X, -127, 127)
    mag = np.abs(blk) / np.exp2(X.astype(np.float64))[:, :, None]
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    ex = np.clip(ex, -6, 8)                      # binade (subnormals share the step of 2^-6)
    step = np.exp2(ex - 3)
    q = np.minimum(np.rint(mag / step) * step, 448.0)   # rint: ties to even
    # encode q: a rounding up may have reached the next binade, so take its exponent again
    with np.errstate(divide="ignore"):
        eq = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    sub = q < 2.0 ** -6
    e_field = np.where(sub, 0, eq + 7)
    m_field = np.where(sub, q / 2.0 ** -9, (q / np.exp2(eq) - 1.0) * 8)
    code = (e_field.astype(np.int64) << 3) | m_field.astype(np.int64)
    sign = (blk < 0) & (code != 0)
    codes = (code | (sign.astype(np.int64) << 7)).astype(np.uint8).reshape(N, K)
    return codes, (X + 127).astype(np.uint8)


# ----------------------------------------------------------------------------------
# everything for one workload
# ----------------------------------------------------------------------------------
def gen_layer(shape: LayerShape, seed: int = 0, with_experts: bool = True) -> dict:
    d = dict(x=gen_x(shape, seed), router_w=gen_router(shape, seed), bias=gen_bias(shape, seed))
    if shape.num_shared_experts:
        d["shared"] = gen_shared(shape, seed)
    if with_experts:
        d["experts"] = gen_experts(shape, seed)
    return d
