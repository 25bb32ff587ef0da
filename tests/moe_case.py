"""Test helpers: build one workload's inputs (from the seeded generators), upload them for the
HIP library, and evaluate the CPU oracle on the same inputs.  Nothing here computes the layer
itself; the oracle does that on the CPU and the library on the GPU."""
from __future__ import annotations

import dataclasses

import numpy as np

import oracle
from synthetic import (LayerShape, gen_bias, gen_expert_encoded, gen_experts, gen_router, gen_shared, gen_x)

# per-token score gap under which a routing difference is a near-tie, not an error
TIE_EPS = 1e-6


WEIGHT_FORMATS = {"bf16": 0, "mxfp4": 1, "mxfp8": 2}   # moe_weight_format_t
ACT_FORMATS = {"bf16": 0, "mxfp8": 1}                   # moe_act_format_t


def cfg_for(shape: LayerShape):
    from sparse_moe_layer_bailingmoev3_amd import MoEConfig
    return MoEConfig(hidden_size=shape.H, num_experts=shape.E, num_experts_per_tok=shape.K, n_group=shape.G,
                     topk_group=shape.TG, moe_intermediate_size=shape.I,
                     num_shared_experts=shape.num_shared_experts, shared_intermediate_size=shape.I_s,
                     norm_topk_prob=int(shape.norm_topk_prob), routed_scaling_factor=shape.routed_scaling_factor,
                     swiglu_limit=shape.swiglu_limit, shared_swiglu_limit=shape.shared_swiglu_limit,
                     expert_weight_format=WEIGHT_FORMATS[shape.weight_format],
                     expert_act_format=ACT_FORMATS[shape.act_format])


@dataclasses.dataclass
class HostCase:
    shape: LayerShape
    seed: int
    x: np.ndarray          # [T,H] bf16 bits
    router_w: np.ndarray   # [E,H] fp32
    bias: np.ndarray       # [E] fp32
    experts: dict          # stacked bf16 bits or MXFP4 pieces
    shared: dict           # bf16 bits

    def expert_f64(self, e: int):
        """(gate, up, down) of routed expert e as float64 (decoded from the stored format)."""
        cache = getattr(self, "_cache", None)
        if cache is not None and e in cache:
            return tuple(a.astype(np.float64) for a in cache[e])
        return self._decode(e)

    def prefetch(self, experts, threads: int = 16):
        """Decode the given routed experts on a thread pool ahead of an oracle run (the
        MXFP4 decode takes ~0.25 s per full-size expert); kept as float32, which holds every
        bf16 and every decoded MXFP4 value exactly."""
        from concurrent.futures import ThreadPoolExecutor
        todo = sorted(set(int(e) for e in experts))
        with ThreadPoolExecutor(threads) as pool:
            dec = list(pool.map(lambda e: tuple(a.astype(np.float32) for a in self._decode(e)), todo))
        self._cache = dict(zip(todo, dec))

    def _decode(self, e: int):
        if self.shape.weight_format in ("mxfp4", "mxfp8"):
            ex = self.experts
            dq = oracle.mxfp4_dequant if self.shape.weight_format == "mxfp4" else oracle.mxfp8_dequant
            return tuple(dq(ex[k + "_q"][e], ex[k + "_s"][e]) for k in ("gate", "up", "down"))
        return tuple(oracle.bf16_to_f64(self.experts[k][e]) for k in ("gate", "up", "down"))

    def shared_f64(self):
        if not self.shape.num_shared_experts:
            return None
        return tuple(oracle.bf16_to_f64(self.shared[k]) for k in ("gate", "up", "down"))


def host_case(shape: LayerShape, seed: int = 0, T: int | None = None, experts: dict | None = None,
              x: np.ndarray | None = None, bias: np.ndarray | None = None,
              router_w: np.ndarray | None = None) -> HostCase:
    T = shape.T if T is None else T
    shape = shape.with_(T=T)
    return HostCase(shape, seed,
                    gen_x(shape, seed) if x is None else x,
                    gen_router(shape, seed) if router_w is None else router_w,
                    gen_bias(shape, seed) if bias is None else bias,
                    gen_experts(shape, seed) if experts is None else experts,
                    gen_shared(shape, seed) if shape.num_shared_experts else {})


def oracle_route(c: HostCase, rows=None):
    s = c.shape
    x = oracle.bf16_to_f64(c.x if rows is None else c.x[rows])
    return oracle.route(oracle.router_logits(x, c.router_w), c.bias, s.G, s.TG, s.K, s.routed_scaling_factor,
                        s.norm_topk_prob, tie_eps=TIE_EPS)


def oracle_forward(c: HostCase, rows=None):
    """Oracle layer output (float64) for all tokens or for the selected rows only."""
    s = c.shape
    x = oracle.bf16_to_f64(c.x if rows is None else c.x[rows])
    return oracle.moe_layer(x, c.router_w, c.bias, c.expert_f64, c.shared_f64(), n_group=s.G,
                            topk_group=s.TG, top_k=s.K, routed_scaling_factor=s.routed_scaling_factor,
                            norm_topk_prob=s.norm_topk_prob, swiglu_limit=s.swiglu_limit,
                            shared_swiglu_limit=s.shared_swiglu_limit,
                            act_quant="mxfp8" if s.act_format == "mxfp8" else "none")


# ----------------------------------------------------------------------------------
# device side (torch is only the allocator here)
# ----------------------------------------------------------------------------------
def to_dev(a: np.ndarray, bf16: bool = False):
    import torch
    if bf16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def to_bits(t) -> np.ndarray:
    """bf16 device tensor -> uint16 bit pattern on the host."""
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceCase:
    def __init__(self, c: HostCase):
        import torch
        from sparse_moe_layer_bailingmoev3_amd import MoEExpertWeights, moe_workspace_size
        self.c = c
        s = c.shape
        self.cfg = cfg_for(s)
        self.x = to_dev(c.x, bf16=True)
        self.router_w = to_dev(c.router_w)
        self.bias = to_dev(c.bias)
        sh = [to_dev(c.shared[k], bf16=True) for k in ("gate", "up", "down")] if s.num_shared_experts else [None] * 3
        if s.weight_format in ("mxfp4", "mxfp8"):
            ex = c.experts
            self.weights = MoEExpertWeights(to_dev(ex["gate_q"]), to_dev(ex["up_q"]), to_dev(ex["down_q"]),
                                            to_dev(ex["gate_s"]), to_dev(ex["up_s"]), to_dev(ex["down_s"]), *sh)
        else:
            self.weights = MoEExpertWeights(*[to_dev(c.experts[k], bf16=True) for k in ("gate", "up", "down")],
                                            shared_gate=sh[0], shared_up=sh[1], shared_down=sh[2])
        T = s.T
        self.T = T
        self.ws = torch.empty(max(moe_workspace_size(self.cfg, T), 256), dtype=torch.uint8, device="cuda")

    def forward(self, bias=True):
        import torch
        from sparse_moe_layer_bailingmoev3_amd import moe_forward
        s = self.c.shape
        out = torch.empty((self.T, s.H), dtype=torch.bfloat16, device="cuda")
        idx = torch.empty((self.T, s.K), dtype=torch.int32, device="cuda")
        w = torch.empty((self.T, s.K), dtype=torch.float32, device="cuda")
        cnt = torch.empty((s.E + 1,), dtype=torch.int32, device="cuda")
        moe_forward(self.cfg, self.T, self.x, self.router_w, self.bias if bias else None, self.weights, out, idx, w,
                    cnt, self.ws)
        torch.cuda.synchronize()
        return out, idx, w, cnt


def compare_routing(r, idx_gpu: np.ndarray, w_gpu: np.ndarray, rows=None):
    """Indices must match exactly off near-ties; returns (n_near_tie, n_mismatch_at_ties)."""
    near = r.near_tie
    ref_idx = r.topk_idx
    ok = ~near
    bad = np.nonzero((idx_gpu[ok] != ref_idx[ok]).any(1))[0]
    assert bad.size == 0, f"{bad.size} tokens route differently off near-ties, first {np.nonzero(ok)[0][bad[:5]]}"
    np.testing.assert_allclose(w_gpu[ok], r.topk_w[ok], rtol=2e-5, atol=1e-6)
    mism = int((idx_gpu[near] != ref_idx[near]).any(1).sum())
    return int(near.sum()), mism


def expected_counts(r, idx_gpu: np.ndarray, E: int, T: int, S: int):
    """Counts from the oracle's routing, with near-tie tokens taking the GPU's choice."""
    idx = r.topk_idx.copy()
    idx[r.near_tie] = idx_gpu[r.near_tie]
    c = np.bincount(idx.ravel(), minlength=E)
    return np.concatenate([c, [T * S]])


def rms(a):
    return float(np.sqrt(np.mean(np.square(a, dtype=np.float64))))
