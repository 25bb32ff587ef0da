#!/usr/bin/env python3
"""Benchmark of one BailingMoeV3 sparse MoE layer forward (hidden 2560, 512 routed experts of
intermediate 768 in 8 groups, top-4 groups, top-8, one shared expert) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload decode|prefill|skewed|mxfp4]

A step is one moe_forward call (router, dispatch, expert FFNs, combine) over one batch of
seeded synthetic tokens already resident in HBM.  Prints one JSON line with tokens/s, the
roofline of the dominant kernel (timed live with HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.  The secondary object `prefill` holds
the T=8192 measurement the headline metric also names.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, TFLOP/s (the scaled MFMA with an E4M3 operand)


def mfma_peak(shape):
    return FP8_PEAK_TFLOPS if shape.act_format == "mxfp8" else BF16_PEAK_TFLOPS


PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_RECORD = os.path.join(PROFILES, "traffic.json")


def kernel_source_hash() -> str:
    """sha256 over the library's kernel sources and C header: a traffic record taken on other
    sources no longer describes the kernels that run."""
    import glob
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_moe_layer_bailingmoev3_amd", "csrc")
    for f in sorted(glob.glob(os.path.join(csrc, "*.hip")) + glob.glob(os.path.join(csrc, "*.h")) +
                    [os.path.join(ROOT, "include", "moe.h")]):
        h.update(os.path.basename(f).encode())
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def recorded_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 record, or
    None when there is none or it was taken on different kernel sources."""
    try:
        with open(TRAFFIC_RECORD) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    e = rec.get(workload, {}).get(kernel)
    if not e or e.get("source_sha256") != kernel_source_hash():
        return None
    return int(e["fetch_bytes"] + e["write_bytes"])


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# ----------------------------------------------------------------------------------
# HIP events on the library's stream (torch's events only see torch's current stream)
# ----------------------------------------------------------------------------------
class Hip:
    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        for n in ("hipEventCreate", "hipEventDestroy", "hipEventSynchronize", "hipEventElapsedTime",
                  "hipEventRecord"):
            getattr(self.lib, n).restype = ctypes.c_int

    def event(self) -> int:
        ev = ctypes.c_void_p()
        assert self.lib.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def record(self, ev, stream):
        assert self.lib.hipEventRecord(ctypes.c_void_p(ev), ctypes.c_void_p(stream)) == 0

    def elapsed_ms(self, a, b) -> float:
        ms = ctypes.c_float()
        assert self.lib.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value


# ----------------------------------------------------------------------------------
# workload
# ----------------------------------------------------------------------------------
def upload(shape, experts, seed=0):
    import torch
    from synthetic import gen_bias, gen_router, gen_shared, gen_x
    import sparse_moe_layer_bailingmoev3_amd as moe

    def dev(a, bf16=False):
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else np.ascontiguousarray(a))
        t = t.cuda()
        return t.view(torch.bfloat16) if bf16 else t

    x_bits = gen_x(shape, seed)
    d = dict(x_bits=x_bits, x=dev(x_bits, True), router_w_np=gen_router(shape, seed), bias_np=gen_bias(shape, seed))
    d["router_w"], d["bias"] = dev(d["router_w_np"]), dev(d["bias_np"])
    sh = gen_shared(shape, seed)
    d["shared_np"] = sh
    shared = [dev(sh[k], True) for k in ("gate", "up", "down")]
    if shape.weight_format in ("mxfp4", "mxfp8"):
        arrs = [dev(experts[k]) for k in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")]
        # block-format experts in the kernels' tiled order, packed once on the device as at load
        pack = moe.moe_pack_mxfp4 if shape.weight_format == "mxfp4" else moe.moe_pack_mxfp8
        E, I, H = shape.E, shape.I, shape.H
        for j, (N, Kd) in enumerate(((I, H), (I, H), (H, I))):
            qo, so = torch.empty_like(arrs[j]), torch.empty_like(arrs[3 + j])
            pack(arrs[j], arrs[3 + j], E, N, Kd, qo, so)
            arrs[j], arrs[3 + j] = qo, so
        torch.cuda.synchronize()
        w = moe.MoEExpertWeights(*arrs, *shared)
    else:
        w = moe.MoEExpertWeights(*[dev(experts[k], True) for k in ("gate", "up", "down")],
                                 shared_gate=shared[0], shared_up=shared[1], shared_down=shared[2])
    d["weights"] = w
    return d


def cfg_for(shape):
    import sparse_moe_layer_bailingmoev3_amd as moe
    return moe.MoEConfig(hidden_size=shape.H, num_experts=shape.E, num_experts_per_tok=shape.K, n_group=shape.G,
                         topk_group=shape.TG, moe_intermediate_size=shape.I,
                         num_shared_experts=shape.num_shared_experts, shared_intermediate_size=shape.I_s,
                         norm_topk_prob=int(shape.norm_topk_prob), routed_scaling_factor=shape.routed_scaling_factor,
                         swiglu_limit=shape.swiglu_limit, shared_swiglu_limit=shape.shared_swiglu_limit,
                         expert_weight_format={"bf16": moe.MOE_WEIGHTS_BF16, "mxfp4": moe.MOE_WEIGHTS_MXFP4_TILED,
                                               "mxfp8": moe.MOE_WEIGHTS_MXFP8_TILED}[shape.weight_format],
                         expert_act_format=moe.MOE_ACT_MXFP8 if shape.act_format == "mxfp8" else moe.MOE_ACT_BF16)


def dtype_of(shape):
    """Arithmetic types of the step: weights / activations of the routed experts' products."""
    if shape.weight_format == "bf16":
        return "bf16"
    return f"{shape.weight_format}-w/{'mxfp8' if shape.act_format == 'mxfp8' else 'bf16'}-a"


def expert_bytes(shape):
    """Bytes of one routed expert's weights (gate, up, down) in its storage format."""
    n = 3 * shape.H * shape.I
    return {"mxfp4": n // 2 + n // 32, "mxfp8": n + n // 32}.get(shape.weight_format, 2 * n)


def measure(shape, d, steps, warmup, hip):
    """Time `steps` forwards; returns dict with ms/step and per-kernel mean durations."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    cfg = cfg_for(shape)
    T = shape.T
    ws = torch.empty(moe.moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    out = torch.empty((T, shape.H), dtype=torch.bfloat16, device="cuda")
    idx = torch.empty((T, shape.K), dtype=torch.int32, device="cuda")
    wts = torch.empty((T, shape.K), dtype=torch.float32, device="cuda")
    cnt = torch.empty((shape.E + 1,), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(warmup):
        moe.moe_forward(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, idx, wts, cnt, ws)
    torch.cuda.synchronize()

    # per-kernel breakdown, outside the timed region: forwards with an event after every kernel
    # (each recorded event adds a few microseconds of queue time to the step)
    nev = 24
    nb = max(3, min(steps, 10))
    events = [[hip.event() for _ in range(nev)] for _ in range(nb)]
    names = None
    for s in range(nb):
        names = moe.moe_forward_traced(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, ws, events[s])
    torch.cuda.synchronize()
    per_kernel = {}
    for s in range(nb):
        for i, n in enumerate(names):
            per_kernel.setdefault(n, []).append(hip.elapsed_ms(events[s][i], events[s][i + 1]))
    kmean = {n: float(np.mean(v)) for n, v in per_kernel.items()}
    dom = max(("expert_gate_up", "expert_down"), key=lambda n: kmean.get(n, 0.0))
    k = names.index(dom)

    # timed region: `steps` forwards; in each, the dominant kernel is timed by two events bound
    # to its own dispatch (moe_forward_timed), which add no packets to the queue
    timed = [(hip.event(), hip.event()) for _ in range(steps)]
    t_start, t_end = hip.event(), hip.event()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    hip.record(t_start, stream)
    for s in range(steps):
        moe.moe_forward_timed(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, ws, k, *timed[s])
    hip.record(t_end, stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    ev_ms = hip.elapsed_ms(t_start, t_end) / steps
    dom_all = [hip.elapsed_ms(*timed[s]) for s in range(steps)]
    dom_ms = float(np.mean(dom_all))
    # per-step spread, outside the timed region: the same forwards with one event between
    # consecutive steps (each event adds a few microseconds of queue time to its step)
    marks = [hip.event() for _ in range(steps + 1)]
    hip.record(marks[0], stream)
    for s in range(steps):
        moe.moe_forward(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, None, None, None, ws)
        hip.record(marks[s + 1], stream)
    torch.cuda.synchronize()
    step_ms = np.array([hip.elapsed_ms(marks[s], marks[s + 1]) for s in range(steps)])
    # cold caches, outside the timed region: before each step a 512 MB buffer is read (twice
    # the 256 MB Infinity Cache, so no weight byte of the previous step is still cached; read,
    # not written, so that no dirty lines are written back during the step), then the step
    # runs between two events
    flush = torch.ones(128 << 20, dtype=torch.float32, device="cuda")
    sink = torch.empty((), dtype=torch.float32, device="cuda")
    cold = [(hip.event(), hip.event()) for _ in range(steps)]
    for s in range(steps):
        torch.amax(flush, dim=0, out=sink)
        hip.record(cold[s][0], stream)
        moe.moe_forward(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, None, None, None, ws)
        hip.record(cold[s][1], stream)
    torch.cuda.synchronize()
    cold_ms = [hip.elapsed_ms(a, b) for a, b in cold]
    del flush, sink
    # routing of the last step (for algorithmic bytes)
    moe.moe_forward(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, idx, wts, cnt, ws)
    torch.cuda.synchronize()
    counts = cnt.cpu().numpy()
    return dict(wall_ms=wall_ms, event_ms=ev_ms, kernels=kmean, dom=dom, dom_ms=dom_ms, counts=counts, out=out,
                idx=idx.cpu().numpy(), dom_dist=_dist(dom_all), step_dist=_dist(step_ms), cold_dist=_dist(cold_ms))


def _dist(v):
    v = np.asarray(v, np.float64)
    return {"median": round(float(np.median(v)), 4), "p10": round(float(np.percentile(v, 10)), 4),
            "p90": round(float(np.percentile(v, 90)), 4), "n": int(v.size)}


def load_stats(shape, counts):
    """Routing load of one step from the per-expert counts: touched experts, max and mean
    count, and the share of assignments taken by the busiest 10 % of experts (the skewed
    workload is built so that it exceeds one half)."""
    c = np.sort(np.asarray(counts[:shape.E], np.int64))[::-1]
    total = int(c.sum())
    p = c[c > 0] / max(1, total)
    # routing entropy -sum p log p of the assignment shares, in nats (a diagnostic; a uniform
    # spread over the experts gives log E)
    return {"touched_experts": int((c > 0).sum()), "max_count": int(c[0]), "mean_count": round(total / shape.E, 2),
            "top10pct_share": round(float(c[: max(1, shape.E // 10)].sum()) / max(1, total), 4),
            "entropy_nats": round(float(-(p * np.log(p)).sum()), 3), "entropy_uniform_nats": round(float(np.log(shape.E)), 3)}


def time_bias_update(shape, counts, hip, reps=200):
    """Mean duration of the expert-bias update (one workgroup) on the counts of a real step:
    reps back-to-back launches between two events.  Bytes it must move: E counts read, E
    biases read and written (12 bytes per expert); it is a single-workgroup, latency-bound
    kernel, so its figure is a duration, not a bandwidth."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    cfg = cfg_for(shape)
    cnt = torch.from_numpy(np.ascontiguousarray(counts[:shape.E + 1]).astype(np.int32)).cuda()
    bias = torch.zeros(shape.E, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for _ in range(5):
        moe.moe_update_expert_bias(cfg, cnt, bias, 1e-3)
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(a, stream)
    for _ in range(reps):
        moe.moe_update_expert_bias(cfg, cnt, bias, 1e-3)
    hip.record(b, stream)
    us = hip.elapsed_ms(a, b) * 1e3 / reps
    return {"us_per_call": round(us, 2), "bytes": 12 * shape.E, "calls": reps,
            "note": "sign-rule expert-bias update from the step's counts; one workgroup, latency-bound"}


def measure_dense(T, H, I, steps, warmup, hip):
    """The dense SwiGLU FFN (moe_dense_ffn) at T tokens: seeded bf16 inputs, `steps` timed calls
    between two events, the calls cycling through enough weight sets (600 MB or more in all)
    that none is still in the 256 MB Infinity Cache from its previous call, as in a model
    whose other layers run in between.  Algorithmic bytes: the three weight matrices once
    (3*I*H*2) + x read + out written; flops 6*T*H*I."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    g = torch.Generator(device="cuda").manual_seed(0)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    nsets = max(2, -(-600_000_000 // (3 * I * H * 2)))
    sets = []
    for _ in range(nsets):
        wg, wu = (torch.randn((I, H), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16) for _ in range(2))
        wd = torch.randn((H, I), generator=g, device="cuda").mul_(0.02).to(torch.bfloat16)
        sets.append((wg, wu, wd))
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_dense_ffn_workspace_size(H, I, T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        moe.moe_dense_ffn(H, I, 0.0, T, x, *sets[i % nsets], out, ws)
    a, b = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(a, stream)
    for i in range(steps):
        moe.moe_dense_ffn(H, I, 0.0, T, x, *sets[i % nsets], out, ws)
    hip.record(b, stream)
    ms = hip.elapsed_ms(a, b) / steps
    byts = 3 * I * H * 2 + 2 * T * H * 2
    flops = 6.0 * T * H * I
    hbm, mfma = byts / (ms * 1e-3) / 1e9, flops / (ms * 1e-3) / 1e12
    bound = "hbm" if byts / (HBM_PEAK_GBS * 1e9) >= flops / (BF16_PEAK_TFLOPS * 1e12) else "mfma"
    frac = hbm / HBM_PEAK_GBS if bound == "hbm" else mfma / BF16_PEAK_TFLOPS
    return {"workload": f"dense SwiGLU FFN: T={T}, hidden {H}, intermediate {I}", "value": round(T / (ms * 1e-3), 1),
            "unit": "tokens/s", "ms_per_call": round(ms, 4), "bound": bound, "frac": round(frac, 4),
            "hbm_GBps": round(hbm, 1), "bf16_TFLOPs": round(mfma, 1), "algorithmic_bytes": byts, "flops": flops,
            "weight_sets": nsets}


def measure_stack(shape, L, steps, warmup, hip):
    """L MoE layers of the same shape, each with its own weights and its own N(0,1) input
    (drawn on the GPU from the same distributions as the single layer), run back to back: a
    decode step through a stack of distinct layers, so that no layer's weights can be found
    in a cache from the step before.  The layers are not chained: without the model's
    residual stream and norms, one layer's raw output (RMS ~0.03) would route every token of
    the next layer to the same few experts.  Returns ms per step and per layer."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    E, H, I, T = shape.E, shape.H, shape.I, shape.T
    g = torch.Generator(device="cuda").manual_seed(1)

    def normal_bf16(*dims):
        out = torch.empty(dims, dtype=torch.bfloat16, device="cuda")
        for i in range(0, dims[0], 64):  # in slices: no full-size fp32 temporary
            out[i:i + 64] = torch.randn((min(64, dims[0] - i),) + dims[1:], generator=g, device="cuda").mul_(0.02)
        return out

    cfg = cfg_for(shape)
    layers = []
    for _ in range(L):
        w = moe.MoEExpertWeights(normal_bf16(E, I, H), normal_bf16(E, I, H), normal_bf16(E, H, I),
                                 shared_gate=normal_bf16(shape.I_s, H), shared_up=normal_bf16(shape.I_s, H),
                                 shared_down=normal_bf16(H, shape.I_s))
        rw = torch.randn((E, H), generator=g, device="cuda").mul_(0.02)
        b = torch.rand((E,), generator=g, device="cuda").mul_(0.2).sub_(0.1)
        layers.append((rw, b, w))
    xs = [torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16) for _ in range(L)]
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_workspace_size(cfg, T), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def step():
        for l, (rw, b, w) in enumerate(layers):
            moe.moe_forward(cfg, T, xs[l], rw, b, w, out, None, None, None, ws)

    for _ in range(warmup):
        step()
    a, e = hip.event(), hip.event()
    torch.cuda.synchronize()
    hip.record(a, stream)
    for _ in range(steps):
        step()
    hip.record(e, stream)
    ms = hip.elapsed_ms(a, e) / steps
    return {"workload": f"decode through {L} distinct layers: T={T}, hidden {H}, {E} experts", "layers": L,
            "ms_per_step": round(ms, 4), "ms_per_layer": round(ms / L, 4),
            "tokens_per_s_per_layer": round(T / (ms / L * 1e-3), 1), "weights_GB": round(L * expert_bytes(shape) * E / 1e9, 1)}


def y_value_bytes(shape) -> int:
    """Bytes per value of the expert outputs y inside moe_forward: fp16 on every path."""
    return 2


def roofline(shape, r, workload=None, measured=None):
    """Roofline of the dominant kernel (the longer of gate/up and down), timed by two events
    bound to its dispatch in every step of the timed region.

    Algorithmic bytes per launch (what the method has to move, once):
      expert_gate_up: (touched routed experts + shared) * 2*I*H weights in their storage
                      format + x [T,H] bf16 read + h [T*K + T, I] bf16 written;
      expert_down:    (touched + shared) * H*I weights + h read + y [T*K + T, H] fp16 written.
    bf16 FLOPs per launch: 4*H*I per (token, expert) pair for gate/up, 2*H*I for down."""
    counts = r["counts"]
    E, H, I, K, T = shape.E, shape.H, shape.I, shape.K, shape.T
    touched = int((counts[:E] > 0).sum())
    S = shape.num_shared_experts
    pairs = T * K + T * S
    eb = expert_bytes(shape)
    per_mat = eb // 3
    sh_mat = 2 * H * I  # shared expert is bf16
    dom = r["dom"]
    routed = T * K
    if shape.weight_format != "bf16":
        # block-format weights: the timed launch is the routed experts' alone (the shared expert
        # runs in bf16 launches of its own)
        S, pairs = 0, routed
    if shape.act_format == "mxfp8":
        # x and h move as E4M3 codes plus one scale byte per 32 values
        x_b, h_b = T * H * 33 // 32, routed * I * 33 // 32
    else:
        x_b, h_b = T * H * 2, pairs * I * 2
    if dom == "expert_gate_up":
        byts = touched * 2 * per_mat + S * 2 * sh_mat + x_b + h_b
        flops = 4.0 * H * I * pairs
    else:
        byts = touched * per_mat + S * sh_mat + h_b + pairs * H * y_value_bytes(shape)
        flops = 2.0 * H * I * pairs
    ms = r["dom_ms"]
    gbs = byts / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    hbm_time = byts / (HBM_PEAK_GBS * 1e9)
    mpeak = mfma_peak(shape)
    mfma_time = flops / (mpeak * 1e12)
    if hbm_time >= mfma_time:
        rl = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        rl = dict(bound="mfma", achieved=round(tflops, 1), peak=mpeak, unit="TFLOP/s", frac=round(tflops / mpeak, 4))
    rl.update(kernel=dom, kernel_ms=round(ms, 4), kernel_ms_dist=r.get("dom_dist"), algorithmic_bytes=int(byts),
              flops=flops, touched_experts=touched, traffic=recorded_traffic(workload or shape.name, dom))
    if measured:
        # HBM-bound kernels here mostly read: the measured read rate is their ceiling
        rl["frac_of_measured"] = round(gbs / measured["read_GBps"], 4) if rl["bound"] == "hbm" else \
            round(tflops / measured["fp8_mfma_TFLOPs" if mfma_peak(shape) == FP8_PEAK_TFLOPS else "bf16_mfma_TFLOPs"], 4)
    return rl


def measured_peaks(hip, nbytes=1 << 30, n=4096):
    """Achievable rates on this GPU, beside the nominal peaks, from the probe kernels of
    libmoe_probe.so (package/probe/peak_probe.hip): a plain 1 GiB HBM read, a plain 1 GiB copy
    (bytes read + written) and loops of independent MFMAs (bf16 16x16x32; scaled 16x16x128 on
    E4M3 and on E2M1 operands), each the best over
    a few grid sizes and 3 runs, timed with events; plus torch's bf16 GEMM (hipBLASLt) at
    n x n x n as a library reference."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    lib = ctypes.CDLL(os.path.join(os.path.dirname(moe.lib_path()), "libmoe_probe.so"))
    stream = torch.cuda.current_stream().cuda_stream
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    b = torch.empty_like(a)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    n16 = nbytes // 16
    V, S, I = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int

    def best(launch, grids, reps=3):
        t = 1e9
        for g in grids:
            launch(g)  # warm
            for _ in range(reps):
                e0, e1 = hip.event(), hip.event()
                hip.record(e0, stream)
                assert launch(g) == 0
                hip.record(e1, stream)
                t = min(t, hip.elapsed_ms(e0, e1))
        return t
    grids = (1024, 2048, 4096, 8192, 16384)
    t_read = best(lambda g: lib.moe_probe_read(V(a.data_ptr()), S(n16), V(sink.data_ptr()), I(g), V(stream)), grids)
    t_copy = best(lambda g: lib.moe_probe_copy(V(a.data_ptr()), V(b.data_ptr()), S(n16), I(g), V(stream)), grids)
    # MFMA loops: grid workgroups of 4 waves, `chains` independent MFMAs per wave and iteration
    iters, chains = 1000, lib.moe_probe_mfma_chains()

    def mfma_rate(launch, flops_per_mfma):
        rate = 0.0
        for g in (1024, 2048, 4096):
            t = best(lambda gg: launch(gg), (g,))
            rate = max(rate, g * 4 * iters * chains * flops_per_mfma / (t * 1e-3) / 1e12)
        return rate
    sp = V(sink.data_ptr())
    mfma_tflops = mfma_rate(lambda g: lib.moe_probe_mfma_bf16(I(iters), I(g), sp, V(stream)), 2 * 16 * 16 * 32)
    fp8_tflops = mfma_rate(lambda g: lib.moe_probe_mfma_scaled(I(0), I(iters), I(g), sp, V(stream)), 2 * 16 * 16 * 128)
    fp4_tflops = mfma_rate(lambda g: lib.moe_probe_mfma_scaled(I(4), I(iters), I(g), sp, V(stream)), 2 * 16 * 16 * 128)
    A = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    B = torch.randn((n, n), device="cuda").to(torch.bfloat16)
    C = torch.empty((n, n), device="cuda", dtype=torch.bfloat16)
    t_mm = best(lambda g: (torch.matmul(A, B, out=C), 0)[1], (0,), reps=5)
    del a, b, A, B, C
    return {"read_GBps": round(nbytes / (t_read * 1e-3) / 1e9, 1),
            "copy_GBps": round(2 * nbytes / (t_copy * 1e-3) / 1e9, 1),
            "bf16_mfma_TFLOPs": round(mfma_tflops, 1),
            "fp8_mfma_TFLOPs": round(fp8_tflops, 1),
            "fp4_mfma_TFLOPs": round(fp4_tflops, 1),
            "bf16_gemm_TFLOPs": round(2.0 * n ** 3 / (t_mm * 1e-3) / 1e12, 1),
            "note": "probe kernels (1 GiB read; 1 GiB copy, read + written bytes; loops of independent bf16 "
                    "16x16x32 MFMAs and of scaled 16x16x128 MFMAs on E4M3 and E2M1 operands) and torch bf16 matmul "
                    "4096^3 (hipBLASLt); best over grids and runs"}


def layout_probe(hip, rows=225 * 1536, K=2560, reps=5):
    """The decode gate/up weight stream alone (225 experts x 1536 rows x 2560 bf16, the decode
    workload's touched experts) read by the probe kernel in the few-token kernel's pattern, from
    the row-major layout and from a blocked one (each wave-step's 16 rows x 256 values
    contiguous): what a blocked weight layout would buy the decode kernels."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    lib = ctypes.CDLL(os.path.join(os.path.dirname(moe.lib_path()), "libmoe_probe.so"))
    stream = torch.cuda.current_stream().cuda_stream
    w = torch.empty(rows * K, dtype=torch.int16, device="cuda").random_(-32768, 32767)
    sink = torch.zeros(rows // 64, dtype=torch.int32, device="cuda")
    V, I = ctypes.c_void_p, ctypes.c_int
    res = {}
    for name, blocked in (("row_major_GBps", 0), ("blocked_GBps", 1)):
        launch = lambda: lib.moe_probe_frag_read(V(w.data_ptr()), I(rows), I(K), I(blocked), V(sink.data_ptr()), V(stream))  # noqa: E731
        assert launch() == 0
        t = 1e9
        for _ in range(reps):
            e0, e1 = hip.event(), hip.event()
            hip.record(e0, stream)
            assert launch() == 0
            hip.record(e1, stream)
            t = min(t, hip.elapsed_ms(e0, e1))
        res[name] = round(rows * K * 2 / (t * 1e-3) / 1e9, 1)
    del w
    torch.cuda.empty_cache()
    res["bytes"] = rows * K * 2
    return res


def layer_summary(shape, r, measured=None):
    """Whole-layer figures: algorithmic bytes of the step and fractions of both peaks."""
    counts = r["counts"]
    E, H, I, K, T = shape.E, shape.H, shape.I, shape.K, shape.T
    touched = int((counts[:E] > 0).sum())
    S = shape.num_shared_experts
    byts = touched * expert_bytes(shape) + S * 3 * H * I * 2 + E * H * 4 + E * 4 + 2 * T * H * 2
    flops = 6.0 * H * I * (T * K + T * S)
    ms = r["wall_ms"]
    hbm_t, mfma_t = byts / (HBM_PEAK_GBS * 1e9), flops / (mfma_peak(shape) * 1e12)
    return dict(algorithmic_bytes=int(byts), hbm_frac=round(byts / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                flops=flops, mfma_peak_TFLOPs=mfma_peak(shape),
                mfma_frac=round(flops / (ms * 1e-3) / (mfma_peak(shape) * 1e12), 4),
                binding_roofline_frac=round(max(hbm_t, mfma_t) / (ms * 1e-3), 4),
                hbm_frac_of_measured_read=round(byts / (ms * 1e-3) / 1e9 / measured["read_GBps"], 4) if measured else None,
                router_fp32_flops=2.0 * T * H * E, touched_experts=touched, step_ms_dist=r.get("step_dist"),
                cold=cold_summary(shape, r), load=load_stats(shape, counts))


def cold_summary(shape, r):
    """The step with cold caches (a 512 MB read before each step, outside the events): median
    and spread of the step, its tokens/s, and its fraction of the HBM peak on the same
    algorithmic bytes as the warm figure."""
    cd = r.get("cold_dist")
    if not cd:
        return None
    return {"step_ms_dist": cd, "value": round(shape.T / (cd["median"] * 1e-3), 1), "unit": "tokens/s",
            "note": "512 MB read between steps (twice the Infinity Cache); one event pair per step"}


def library_gemm(shape, d, idx, hip, reps=10):
    """For comparison only (not part of the product): the same expert products as torch's
    batched bf16 matmul (hipBLASLt on ROCm), with the tokens already gathered per expert and
    every expert padded or cut to P positions, P = the mean tokens per expert rounded up to 16
    (about the same flops as the routed work of the step; experts above P lose their extra
    tokens).  gate and up are two products of [E,I,H] x [E,H,P] and down one of [E,H,I] x
    [E,I,P]; weights as the left operand, so no transposed right operand reaches the batched
    product."""
    import torch
    E, H, I, T, K = shape.E, shape.H, shape.I, shape.T, shape.K
    P = int(np.ceil(T * K / E / 16) * 16)
    gate, up, down = d["weights"]._keep[:3]
    e = torch.from_numpy(idx.astype(np.int64).reshape(-1)).cuda()
    tok = torch.arange(T, device="cuda").repeat_interleave(K)
    order = torch.argsort(e, stable=True)
    es, ts = e[order], tok[order]
    cnt = torch.bincount(e, minlength=E)
    rank = torch.arange(es.numel(), device="cuda") - (torch.cumsum(cnt, 0) - cnt)[es]
    keep = rank < P
    xp = torch.zeros((E, P, H), dtype=torch.bfloat16, device="cuda")
    xp[es[keep], rank[keep]] = d["x"][ts[keep]]
    xT = xp.transpose(1, 2).contiguous()                       # [E, H, P]
    hT = torch.zeros((E, I, P), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream().cuda_stream

    def timed(fn):
        for _ in range(3):
            fn()
        ev = [hip.event() for _ in range(reps + 1)]
        hip.record(ev[0], stream)
        for i in range(reps):
            fn()
            hip.record(ev[i + 1], stream)
        torch.cuda.synchronize()
        return float(np.median([hip.elapsed_ms(ev[i], ev[i + 1]) for i in range(reps)]))

    gu_ms = timed(lambda: (torch.bmm(gate, xT), torch.bmm(up, xT)))
    dn_ms = timed(lambda: torch.bmm(down, hT))
    flops_gu, flops_dn = 2.0 * E * P * 2 * I * H, 2.0 * E * P * H * I
    del xp, xT, hT
    torch.cuda.empty_cache()
    return {"positions_per_expert": P, "gate_up_ms": round(gu_ms, 4), "down_ms": round(dn_ms, 4),
            "gate_up_TFLOPs": round(flops_gu / gu_ms * 1e-9, 1), "down_TFLOPs": round(flops_dn / dn_ms * 1e-9, 1),
            "note": "torch.bmm (hipBLASLt) on tokens gathered and padded to P per expert beforehand; "
                    "comparison only, the gather, SwiGLU and combine are not in these times"}


def routing_check(shape, d, idx_gpu):
    """The oracle's routing of every token of a measured step against the GPU's (part of the
    CPU leg): tokens whose group or expert score gap is below 1e-6 are near ties, counted and
    excused; every other token must route identically."""
    import oracle
    T = shape.T
    x = oracle.bf16_to_f64(d["x_bits"])
    r = oracle.route(oracle.router_logits(x, d["router_w_np"]), d["bias_np"], shape.G, shape.TG, shape.K,
                     shape.routed_scaling_factor, shape.norm_topk_prob, tie_eps=1e-6)
    diff = (np.asarray(idx_gpu) != r.topk_idx).any(1)
    return {"tokens": T, "near_ties": int(r.near_tie.sum()), "differ_at_near_ties": int((diff & r.near_tie).sum()),
            "differ_elsewhere": int((diff & ~r.near_tie).sum()), "tie_eps": 1e-6}


def check_rows(T, n=16):
    """Rows of the output the benchmark compares with the oracle: the first, the last and
    evenly spaced ones in between."""
    return np.unique(np.linspace(0, T - 1, n).round().astype(np.int64))


def sampled_output(shape, out):
    """The bf16 bits of the sampled rows of a step's output, copied to the host."""
    import torch
    rows = torch.from_numpy(check_rows(shape.T)).to(out.device)
    return out.index_select(0, rows).view(torch.int16).cpu().numpy().view(np.uint16)


def output_check(shape, d, experts, got_bits):
    """The float64 oracle forward of the sampled rows (part of the CPU leg) against the GPU's
    rows: max|err| / RMS(oracle) over the rows whose routing has no near tie, beside the bar
    (2e-2 for bf16 and MXFP8 weights, 5e-2 for MXFP4 weights and for MXFP8 activations)."""
    import oracle
    rows = check_rows(shape.T)
    x = oracle.bf16_to_f64(d["x_bits"][rows])

    def get(e):
        if shape.weight_format in ("mxfp4", "mxfp8"):
            dq = oracle.mxfp4_dequant if shape.weight_format == "mxfp4" else oracle.mxfp8_dequant
            return tuple(dq(experts[k + "_q"][e], experts[k + "_s"][e]) for k in ("gate", "up", "down"))
        return tuple(oracle.bf16_to_f64(experts[k][e]) for k in ("gate", "up", "down"))
    sh = tuple(oracle.bf16_to_f64(d["shared_np"][k]) for k in ("gate", "up", "down"))
    ref, r = oracle.moe_layer(x, d["router_w_np"], d["bias_np"], get, sh, n_group=shape.G, topk_group=shape.TG,
                              top_k=shape.K, routed_scaling_factor=shape.routed_scaling_factor,
                              norm_topk_prob=shape.norm_topk_prob, swiglu_limit=shape.swiglu_limit,
                              shared_swiglu_limit=shape.shared_swiglu_limit,
                              act_quant="mxfp8" if shape.act_format == "mxfp8" else "none")
    got = oracle.bf16_to_f64(got_bits)
    keep = ~r.near_tie
    rms = float(np.sqrt(np.mean(ref ** 2)))
    err = float(np.abs(got - ref)[keep].max()) if keep.any() else 0.0
    bar = 5e-2 if (shape.weight_format == "mxfp4" or shape.act_format == "mxfp8") else 2e-2
    return {"rows": int(len(rows)), "near_tie_rows": int((~keep).sum()), "max_abs_err_over_rms": round(err / rms, 5),
            "bar": bar}


def cpu_baseline(shape, d, experts, max_tokens):
    """The float64 oracle on the host cores, on the first `max_tokens` tokens of the workload."""
    import oracle
    T = min(shape.T, max_tokens)
    x = oracle.bf16_to_f64(d["x_bits"][:T])

    def get(e):
        if shape.weight_format in ("mxfp4", "mxfp8"):
            dq = oracle.mxfp4_dequant if shape.weight_format == "mxfp4" else oracle.mxfp8_dequant
            return tuple(dq(experts[k + "_q"][e], experts[k + "_s"][e]) for k in ("gate", "up", "down"))
        return tuple(oracle.bf16_to_f64(experts[k][e]) for k in ("gate", "up", "down"))
    sh = tuple(oracle.bf16_to_f64(d["shared_np"][k]) for k in ("gate", "up", "down"))
    # the whole sample again until about 10 s of CPU work have been timed
    passes, dt = 0, 0.0
    while passes == 0 or (dt < 10.0 and passes < 50):
        t0 = time.perf_counter()
        oracle.moe_layer(x, d["router_w_np"], d["bias_np"], get, sh, n_group=shape.G, topk_group=shape.TG,
                         top_k=shape.K, routed_scaling_factor=shape.routed_scaling_factor,
                         norm_topk_prob=shape.norm_topk_prob, swiglu_limit=shape.swiglu_limit,
                         shared_swiglu_limit=shape.shared_swiglu_limit,
                         act_quant="mxfp8" if shape.act_format == "mxfp8" else "none")
        dt += time.perf_counter() - t0
        passes += 1
    # routing alone (logits, sigmoid, grouped top-k, weights) on the same sample
    rpasses, rdt = 0, 0.0
    while rpasses == 0 or (rdt < 2.0 and rpasses < 200):
        t0 = time.perf_counter()
        oracle.route(oracle.router_logits(x, d["router_w_np"]), d["bias_np"], n_group=shape.G,
                     topk_group=shape.TG, top_k=shape.K, routed_scaling_factor=shape.routed_scaling_factor,
                     norm_topk_prob=shape.norm_topk_prob)
        rdt += time.perf_counter() - t0
        rpasses += 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    model = ""
    try:
        with open("/proc/cpuinfo") as fh:
            model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), "")
    except OSError:
        pass
    return dict(value=round(T * passes / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"float64 oracle forward of the first {T} tokens of the {shape.name} workload "
                       f"(H{shape.H}/E{shape.E}/top{shape.K}), {passes} passes, {dt:.1f} s",
                routing_only_value=round(T * rpasses / rdt, 1), cpu_model=model)


# ----------------------------------------------------------------------------------
# rocprofv3 summaries (profiles/*.md) and the traffic record (profiles/traffic.json)
# ----------------------------------------------------------------------------------
# kernel symbol in rocprofv3 output -> the step name moe_forward_traced reports
SYMBOL_STEPS = [(r"^ffn_tile_kernel<0,", "expert_gate_up"), (r"^ffn_tile_kernel<1,", "expert_down"),
                (r"^ffn_kernel<\d+, \d+, \d+, \d+, 0,", "expert_gate_up"),
                (r"^ffn_kernel<\d+, \d+, \d+, \d+, 1,", "expert_down"),
                (r"^router_logits_(kwaves_)?kernel", "router_logits"), (r"^router_topk_kernel", "router_topk"),
                (r"^fill_u32_kernel", "dispatch_clear"), (r"^dispatch_mark_kernel", "dispatch_mark"),
                (r"^dispatch_finish_kernel", "dispatch_finish"), (r"^dispatch_count_kernel", "dispatch_count"),
                (r"^tile_prefix_kernel", "expert_tiles"), (r"^mx8_quant_kernel", "act_quant"),
                (r"^combine_kernel", "combine"), (r"^__amd_rocclr_copyBuffer", "copy")]


def _symbol(name: str) -> str:
    import re
    n = name.replace("void ", "").replace("moe::(anonymous namespace)::", "").replace("moe::", "")
    return re.sub(r"\(.*", "", n)


def _step(sym: str):
    import re
    for pat, step in SYMBOL_STEPS:
        if re.match(pat, sym):
            return step
    return None


def profile_commands(workload: str, out: str = "$OUT"):
    b = (f"python3 $R/bench.py --workload {workload} --steps 10 --warmup 3 --no-cpu-baseline --no-secondary "
         f"--no-peaks --copy-probe")
    return [f"rocprofv3 --kernel-trace --stats -f csv -d {out}/kt -o kt -- {b}",
            f"rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/fetch -o fetch -- {b}",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/write -o write -- {b}",
            f"rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil LdsBankConflict -f csv -d {out}/util -o util -- {b}",
            f"rocprofv3 --pmc VmemLatency -f csv -d {out}/lat -o lat -- {b}",
            f"python3 $R/bench.py --summarize {out} --workload {workload}"]


def summarize(src: str, workload: str):
    """Turn the rocprofv3 runs of profile_commands() into profiles/<kernel>_<workload>.md
    and the workload's entry in profiles/traffic.json (HBM bytes per launch of each step, with
    the kernel-source hash they were taken on)."""
    import csv
    import glob
    from synthetic import CONFIGS
    shape = CONFIGS[workload]

    def one(pattern):
        f = glob.glob(os.path.join(src, pattern))
        if not f:
            raise SystemExit(f"missing {os.path.join(src, pattern)}")
        return f[0]
    stats = [(_symbol(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3, float(r["Percentage"]))
             for r in csv.DictReader(open(one("kt/*kernel_stats.csv")))]

    def counters(path, cname):
        per = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] == cname:
                per.setdefault(_symbol(r["Kernel_Name"]), []).append(float(r["Counter_Value"]))
        return per
    fetch = counters(one("fetch/*counter_collection.csv"), "FETCH_SIZE")
    write = counters(one("write/*counter_collection.csv"), "WRITE_SIZE")
    util_f = glob.glob(os.path.join(src, "util/*counter_collection.csv"))
    util = {n: counters(util_f[0], n) for n in ("MfmaUtil", "VALUBusy", "LdsUtil", "LdsBankConflict")} \
        if util_f else {}
    lat_f = glob.glob(os.path.join(src, "lat/*counter_collection.csv"))
    if lat_f:
        util["VmemLatency"] = counters(lat_f[0], "VmemLatency")
    copy_f, copy_w = max(fetch["__amd_rocclr_copyBuffer"]), max(write["__amd_rocclr_copyBuffer"])
    sf, sw = (1 << 30) / (copy_f * 1024), (1 << 30) / (copy_w * 1024)
    steps = {}
    # a step launched twice (the routed and the shared experts' kernels on the MXFP8-activation
    # path) keeps its longer launch under its name and the other as <step>_shared
    seen = {}
    for sym, c, avg, pct in sorted(stats, key=lambda t: -t[2]):
        st = _step(sym)
        if st in ("expert_gate_up", "expert_down"):
            seen[st] = seen.get(st, 0) + 1
            if seen[st] > 1:
                st += "_shared"
        if st and st != "copy":
            steps[st] = dict(symbol=sym, calls=c, avg_us=avg, pct=pct,
                             fetch_bytes=float(np.mean(fetch.get(sym, [0.0]))) * 1024 * sf,
                             write_bytes=float(np.mean(write.get(sym, [0.0]))) * 1024 * sw,
                             util={n: round(float(np.mean(v[sym])), 2) for n, v in util.items() if sym in v})
    dom = max(("expert_gate_up", "expert_down"), key=lambda k: steps.get(k, {}).get("avg_us", 0.0))
    cmds = profile_commands(workload)
    lines = [f"# {dom} on the {workload} workload (T={shape.T}, H{shape.H}/E{shape.E}/top{shape.K}, "
             f"{shape.weight_format} experts)", "",
             "Commands (from /tmp with TMPDIR=/tmp; $R = repository root, $OUT = an output folder):", "", "```",
             *cmds, "```", "", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | step | calls | average us | % of GPU time |", "|---|---|---|---|---|"]
    for sym, c, avg, pct in stats:
        st = next((k for k, e in steps.items() if e["symbol"] == sym), _step(sym) or "")
        lines.append(f"| `{sym}` | {st} | {c} | {avg:.1f} | {pct:.1f} |")
    lines += ["", "## HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"A plain 1 GiB device copy in the same runs reads FETCH_SIZE = {copy_f:.0f} KiB and "
              f"WRITE_SIZE = {copy_w:.0f} KiB, so bytes = FETCH_SIZE * 1024 * {sf:.3f} and "
              f"WRITE_SIZE * 1024 * {sw:.3f}.", "",
              "| step | kernel | read MB | write MB |", "|---|---|---|---|"]
    for st, e in sorted(steps.items(), key=lambda kv: -kv[1]["avg_us"]):
        lines.append(f"| {st} | `{e['symbol']}` | {e['fetch_bytes'] / 1e6:.1f} | {e['write_bytes'] / 1e6:.1f} |")
    if util:
        lines += ["", "## Utilisation per launch (rocprofv3 --pmc MfmaUtil VALUBusy LdsUtil LdsBankConflict; "
                  "then VmemLatency)", "",
                  "MfmaUtil = MFMA busy cycles / (GPU cycles x SIMDs) in %; VALUBusy = VALU instruction cycles "
                  "per CU in %; LdsUtil = LDS busy cycles per CU in %; LdsBankConflict = conflict cycles per "
                  "conflict-free LDS cycle; VmemLatency = mean cycles a vector memory instruction is in flight "
                  "(issue to completion).", "",
                  "| step | MfmaUtil % | VALUBusy % | LdsUtil % | LdsBankConflict | VmemLatency cycles |",
                  "|---|---|---|---|---|---|"]
        for st, e in sorted(steps.items(), key=lambda kv: -kv[1]["avg_us"]):
            u = e["util"]
            lines.append(f"| {st} | {u.get('MfmaUtil', float('nan')):.1f} | {u.get('VALUBusy', float('nan')):.1f} | "
                         f"{u.get('LdsUtil', float('nan')):.1f} | {u.get('LdsBankConflict', float('nan')):.3f} | "
                         f"{u.get('VmemLatency', float('nan')):.0f} |")
    os.makedirs(PROFILES, exist_ok=True)
    md = os.path.join(PROFILES, f"{dom}_{workload}_T{shape.T}.md")
    with open(md, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    try:
        with open(TRAFFIC_RECORD) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        rec = {}
    h = kernel_source_hash()
    rec[workload] = {st: dict(symbol=e["symbol"], fetch_bytes=round(e["fetch_bytes"]),
                              write_bytes=round(e["write_bytes"]), avg_us=round(e["avg_us"], 2), util=e["util"],
                              source_sha256=h)
                     for st, e in steps.items()}
    with open(TRAFFIC_RECORD, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(open(md).read())


def copy_probe(hip, nbytes=1 << 30):
    """A plain device copy of known size, for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE."""
    import torch
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy probe: {nbytes} bytes read and written per copy")


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "skewed", "mxfp4", "mxfp8", "mxfp4_a8", "mxfp8_a8"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", "--no-prefill", dest="no_secondary", action="store_true",
                    help="skip the secondary workloads (prefill T=8192, skewed, MXFP4)")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured copy and GEMM rates")
    ap.add_argument("--stack", type=int, default=0, metavar="L",
                    help="instead: decode (T=64) through L distinct layers, each with its own weights (L <= 32)")
    ap.add_argument("--dense", type=int, default=0, metavar="I",
                    help="instead: the dense SwiGLU FFN (moe_dense_ffn) of intermediate size I")
    ap.add_argument("--dense-tokens", default="1,64,512,8192", metavar="T,T,...",
                    help="token counts of the --dense measurement")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="tokens in the CPU oracle sample")
    ap.add_argument("--copy-probe", action="store_true")
    ap.add_argument("--layout-probe", action="store_true",
                    help="also read the decode weight stream from the row-major and a blocked layout")
    ap.add_argument("--library-gemm", action="store_true",
                    help="also time the expert products as torch's batched bf16 matmul (hipBLASLt), for comparison")
    ap.add_argument("--summarize", metavar="DIR", help="write profiles/ from the rocprofv3 runs in DIR and exit")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.workload)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this layer is built and timed on a single MI355X, "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch
    from synthetic import CONFIGS, gen_experts
    import sparse_moe_layer_bailingmoev3_amd as moe
    moe.load_library()  # no fallback: fails loudly without the HIP library
    if args.stack:
        if not 1 <= args.stack <= 32:
            sys.exit("--stack takes 1 to 32 layers (6 GB of weights each)")
        hip = Hip()
        res = measure_stack(CONFIGS["decode"], args.stack, max(args.steps, 5), args.warmup, hip)
        print(json.dumps({"metric": "MoE-layer tokens/s through a stack of distinct layers", "dtype": "bf16",
                          "data": "synthetic (seeded, drawn on the GPU)", "n_gpus": 1, **res}), flush=True)
        return
    if args.dense:
        hip = Hip()
        H = CONFIGS["decode"].H
        res = [measure_dense(T, H, args.dense, max(args.steps, 10), args.warmup, hip) for T in map(int, args.dense_tokens.split(","))]
        print(json.dumps({"metric": "dense SwiGLU FFN tokens/s", "dtype": "bf16", "data": "synthetic (seeded)",
                          "n_gpus": 1, "results": res}), flush=True)
        return
    assert torch.cuda.is_available(), "no GPU visible"
    hip = Hip()

    if args.copy_probe:
        copy_probe(hip)

    shape = CONFIGS[args.workload]
    measured = None if args.no_peaks else measured_peaks(hip)
    t0 = time.perf_counter()
    log(f"drawing {shape.E} experts ({shape.weight_format}) ...")
    experts = gen_experts(shape, seed=0)
    log(f"  {time.perf_counter() - t0:.1f} s; uploading")
    d = upload(shape, experts)
    torch.cuda.synchronize()
    log(f"measuring {shape.name} T={shape.T}: warmup {args.warmup}, steps {args.steps}")
    r = measure(shape, d, args.steps, args.warmup, hip)
    ms = r["wall_ms"]
    line = {
        "metric": "MoE-layer tokens/s, H2560/E512/top8, T=64 & T=8192; % of HBM or MFMA peak",
        "value": round(shape.T / (ms * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": dtype_of(shape),
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": f"{shape.name}: T={shape.T}, hidden {shape.H}, {shape.E} experts (I={shape.I}) "
                               f"in {shape.G} groups, top-{shape.TG} groups, top-{shape.K}, 1 shared expert",
                   "T": shape.T, "hidden_size": shape.H, "num_experts": shape.E, "moe_intermediate_size": shape.I,
                   "n_group": shape.G, "topk_group": shape.TG, "num_experts_per_tok": shape.K,
                   "weights": shape.weight_format + (" (tiled order, packed once at load)"
                                                     if shape.weight_format != "bf16" else ""),
                   "parallelism": "single GPU"},
        "roofline": roofline(shape, r, measured=measured),
        "layer": layer_summary(shape, r, measured),
        "kernels_ms": {k: round(v, 4) for k, v in r["kernels"].items()},
        "kernels_ms_from": "forwards with an event after every kernel, outside the timed region",
        "event_ms_per_step": round(r["event_ms"], 4),
        "measured_peaks": measured,
        "expert_bias_update": time_bias_update(shape, r["counts"], hip),
    }
    if args.layout_probe:
        line["layout_probe"] = layout_probe(hip)
    if args.library_gemm and shape.weight_format == "bf16":
        line["library_gemm"] = library_gemm(shape, d, r["idx"], hip)
    host = ("x_bits", "router_w_np", "bias_np", "shared_np")
    checks = [(shape, {k: d[k] for k in host}, r["idx"])]
    outs = {shape.name: (experts, sampled_output(shape, r["out"]))}
    if not args.no_secondary and shape.name == "decode":
        # the other workloads on the same layer: prefill (the metric's T=8192), skewed routing
        # with the deep-layer clamp, and the routed experts in MXFP4 (quantised from the same
        # bf16 draw, as the MXFP4 workload's generator does)
        from synthetic import quantise_mxfp4
        from concurrent.futures import ThreadPoolExecutor
        line["secondary"] = {}
        from synthetic import quantise_mxfp8
        quantised = {}

        def encoded(fmt):
            # the bf16 draw in a block format, once per format (as gen_experts would encode it)
            if fmt not in quantised:
                log(f"quantising the experts to {fmt} ...")
                cd = 2 if fmt == "mxfp4" else 1
                quant = quantise_mxfp4 if fmt == "mxfp4" else quantise_mxfp8
                ex = {k + sfx: np.empty((experts[k].shape[0], experts[k].shape[1], experts[k].shape[2] // div), np.uint8)
                      for k in ("gate", "up", "down") for sfx, div in (("_q", cd), ("_s", 32))}

                def q(e):
                    for k in ("gate", "up", "down"):
                        ex[k + "_q"][e], ex[k + "_s"][e] = quant(experts[k][e])
                with ThreadPoolExecutor(16) as pool:
                    list(pool.map(q, range(len(experts["gate"]))))
                quantised[fmt] = ex
            return quantised[fmt]
        for name in ("prefill", "skewed", "mxfp4", "mxfp4_a8", "mxfp8", "mxfp8_a8"):
            p = CONFIGS[name]
            ex = experts if p.weight_format == "bf16" else encoded(p.weight_format)
            dp = upload(p, ex)
            log(f"measuring {name} T={p.T}")
            rp = measure(p, dp, max(5, args.steps // 3), 3, hip)
            desc = {"skewed": ", clamp 4 / 7, clustered tokens, bias N(0,0.5)", "mxfp4": ", routed experts MXFP4 (tiled order)",
                    "mxfp8": ", routed experts MXFP8 (tiled order)",
                    "mxfp4_a8": ", routed experts MXFP4 (tiled order), MXFP8 activations",
                    "mxfp8_a8": ", routed experts MXFP8 (tiled order), MXFP8 activations"}.get(name, "")
            line["secondary"][name] = {
                "workload": f"{name}: T={p.T}, same layer{desc}",
                "value": round(p.T / (rp["wall_ms"] * 1e-3), 1), "unit": "tokens/s",
                "ms_per_step": round(rp["wall_ms"], 4),
                "dtype": dtype_of(p),
                "roofline": roofline(p, rp, measured=measured), "layer": layer_summary(p, rp, measured),
                "kernels_ms": {k: round(v, 4) for k, v in rp["kernels"].items()}}
            checks.append((p, {k: dp[k] for k in host}, rp["idx"]))
            outs[name] = (ex, sampled_output(p, rp["out"]))
            del dp
            torch.cuda.empty_cache()
        line["prefill"] = line["secondary"]["prefill"]
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(shape, d, experts, args.cpu_tokens)
        # the oracle's routing of every measured step, beside the GPU's
        line["routing_check"] = {c[0].name: routing_check(*c) for c in checks}
        log("checking sampled output rows against the oracle ...")
        line["output_check"] = {c[0].name: output_check(c[0], c[1], *outs[c[0].name]) for c in checks}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
