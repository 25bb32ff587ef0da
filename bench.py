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
    if shape.weight_format == "mxfp4":
        w = moe.MoEExpertWeights(*[dev(experts[k]) for k in ("gate_q", "up_q", "down_q", "gate_s", "up_s", "down_s")],
                                 *shared)
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
                         expert_weight_format=moe.MOE_WEIGHTS_MXFP4 if shape.weight_format == "mxfp4"
                         else moe.MOE_WEIGHTS_BF16)


def expert_bytes(shape):
    """Bytes of one routed expert's weights (gate, up, down) in its storage format."""
    n = 3 * shape.H * shape.I
    return n // 2 + n // 32 if shape.weight_format == "mxfp4" else 2 * n


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
    dom_ms = float(np.mean([hip.elapsed_ms(*timed[s]) for s in range(steps)]))
    # routing of the last step (for algorithmic bytes)
    moe.moe_forward(cfg, T, d["x"], d["router_w"], d["bias"], d["weights"], out, idx, wts, cnt, ws)
    torch.cuda.synchronize()
    counts = cnt.cpu().numpy()
    return dict(wall_ms=wall_ms, event_ms=ev_ms, kernels=kmean, dom=dom, dom_ms=dom_ms, counts=counts, out=out)


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


def roofline(shape, r, workload=None):
    """Roofline of the dominant kernel (the longer of gate/up and down), timed by two events
    bound to its dispatch in every step of the timed region.

    Algorithmic bytes per launch (what the method has to move, once):
      expert_gate_up: (touched routed experts + shared) * 2*I*H weights in their storage
                      format + x [T,H] bf16 read + h [T*K + T, I] bf16 written;
      expert_down:    (touched + shared) * H*I weights + h read + y [T*K + T, H] fp32 written.
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
    if dom == "expert_gate_up":
        byts = touched * 2 * per_mat + S * 2 * sh_mat + T * H * 2 + pairs * I * 2
        flops = 4.0 * H * I * pairs
    else:
        byts = touched * per_mat + S * sh_mat + pairs * I * 2 + pairs * H * 4
        flops = 2.0 * H * I * pairs
    ms = r["dom_ms"]
    gbs = byts / (ms * 1e-3) / 1e9
    tflops = flops / (ms * 1e-3) / 1e12
    hbm_time = byts / (HBM_PEAK_GBS * 1e9)
    mfma_time = flops / (BF16_PEAK_TFLOPS * 1e12)
    if hbm_time >= mfma_time:
        rl = dict(bound="hbm", achieved=round(gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(gbs / HBM_PEAK_GBS, 4))
    else:
        rl = dict(bound="mfma", achieved=round(tflops, 1), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                  frac=round(tflops / BF16_PEAK_TFLOPS, 4))
    rl.update(kernel=dom, kernel_ms=round(ms, 4), algorithmic_bytes=int(byts), bf16_flops=flops,
              touched_experts=touched, traffic=recorded_traffic(workload or shape.name, dom))
    return rl


def layer_summary(shape, r):
    """Whole-layer figures: algorithmic bytes of the step and fractions of both peaks."""
    counts = r["counts"]
    E, H, I, K, T = shape.E, shape.H, shape.I, shape.K, shape.T
    touched = int((counts[:E] > 0).sum())
    S = shape.num_shared_experts
    byts = touched * expert_bytes(shape) + S * 3 * H * I * 2 + E * H * 4 + E * 4 + 2 * T * H * 2
    flops = 6.0 * H * I * (T * K + T * S)
    ms = r["wall_ms"]
    return dict(algorithmic_bytes=int(byts), hbm_frac=round(byts / (ms * 1e-3) / (HBM_PEAK_GBS * 1e9), 4),
                bf16_flops=flops, mfma_frac=round(flops / (ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12), 4),
                router_fp32_flops=2.0 * T * H * E, touched_experts=touched)


def cpu_baseline(shape, d, experts, max_tokens):
    """The float64 oracle on the host cores, on the first `max_tokens` tokens of the workload."""
    import oracle
    T = min(shape.T, max_tokens)
    x = oracle.bf16_to_f64(d["x_bits"][:T])

    def get(e):
        if shape.weight_format == "mxfp4":
            return tuple(oracle.mxfp4_dequant(experts[k + "_q"][e], experts[k + "_s"][e]) for k in ("gate", "up", "down"))
        return tuple(oracle.bf16_to_f64(experts[k][e]) for k in ("gate", "up", "down"))
    sh = tuple(oracle.bf16_to_f64(d["shared_np"][k]) for k in ("gate", "up", "down"))
    # the whole sample again until about 10 s of CPU work have been timed
    passes, dt = 0, 0.0
    while passes == 0 or (dt < 10.0 and passes < 50):
        t0 = time.perf_counter()
        oracle.moe_layer(x, d["router_w_np"], d["bias_np"], get, sh, n_group=shape.G, topk_group=shape.TG,
                         top_k=shape.K, routed_scaling_factor=shape.routed_scaling_factor,
                         norm_topk_prob=shape.norm_topk_prob, swiglu_limit=shape.swiglu_limit,
                         shared_swiglu_limit=shape.shared_swiglu_limit)
        dt += time.perf_counter() - t0
        passes += 1
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return dict(value=round(T * passes / dt, 3), unit="tokens/s", cores=cores, kind="oracle",
                sample=f"float64 oracle forward of the first {T} tokens of the {shape.name} workload "
                       f"(H{shape.H}/E{shape.E}/top{shape.K}), {passes} passes, {dt:.1f} s")


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
                (r"^tile_prefix_kernel", "expert_tiles"),
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
    b = f"python3 $R/bench.py --workload {workload} --steps 10 --warmup 3 --no-cpu-baseline --no-prefill --copy-probe"
    return [f"rocprofv3 --kernel-trace --stats -f csv -d {out}/kt -o kt -- {b}",
            f"rocprofv3 --pmc FETCH_SIZE -f csv -d {out}/fetch -o fetch -- {b}",
            f"rocprofv3 --pmc WRITE_SIZE -f csv -d {out}/write -o write -- {b}",
            f"python3 $R/bench.py --summarize {out} --workload {workload}"]


def summarize(src: str, workload: str):
    """Turn the three rocprofv3 runs of profile_commands() into profiles/<kernel>_<workload>.md
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
    copy_f, copy_w = max(fetch["__amd_rocclr_copyBuffer"]), max(write["__amd_rocclr_copyBuffer"])
    sf, sw = (1 << 30) / (copy_f * 1024), (1 << 30) / (copy_w * 1024)
    steps = {}
    for sym, c, avg, pct in stats:
        st = _step(sym)
        if st and st != "copy":
            steps[st] = dict(symbol=sym, calls=c, avg_us=avg, pct=pct,
                             fetch_bytes=float(np.mean(fetch.get(sym, [0.0]))) * 1024 * sf,
                             write_bytes=float(np.mean(write.get(sym, [0.0]))) * 1024 * sw)
    dom = max(("expert_gate_up", "expert_down"), key=lambda k: steps.get(k, {}).get("avg_us", 0.0))
    cmds = profile_commands(workload)
    lines = [f"# {dom} on the {workload} workload (T={shape.T}, H{shape.H}/E{shape.E}/top{shape.K}, "
             f"{shape.weight_format} experts)", "",
             "Commands (from /tmp with TMPDIR=/tmp; $R = repository root, $OUT = an output folder):", "", "```",
             *cmds, "```", "", "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
             "| kernel | step | calls | average us | % of GPU time |", "|---|---|---|---|---|"]
    for sym, c, avg, pct in stats:
        lines.append(f"| `{sym}` | {_step(sym) or ''} | {c} | {avg:.1f} | {pct:.1f} |")
    lines += ["", "## HBM traffic per launch (rocprofv3 --pmc FETCH_SIZE, then WRITE_SIZE)", "",
              f"A plain 1 GiB device copy in the same runs reads FETCH_SIZE = {copy_f:.0f} KiB and "
              f"WRITE_SIZE = {copy_w:.0f} KiB, so bytes = FETCH_SIZE * 1024 * {sf:.3f} and "
              f"WRITE_SIZE * 1024 * {sw:.3f}.", "",
              "| step | kernel | read MB | write MB |", "|---|---|---|---|"]
    for st, e in sorted(steps.items(), key=lambda kv: -kv[1]["avg_us"]):
        lines.append(f"| {st} | `{e['symbol']}` | {e['fetch_bytes'] / 1e6:.1f} | {e['write_bytes'] / 1e6:.1f} |")
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
                              write_bytes=round(e["write_bytes"]), avg_us=round(e["avg_us"], 2), source_sha256=h)
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
    ap.add_argument("--workload", default="decode", choices=["decode", "prefill", "skewed", "mxfp4"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="skip the secondary T=8192 measurement")
    ap.add_argument("--stack", type=int, default=0, metavar="L",
                    help="instead: decode (T=64) through L distinct layers, each with its own weights (L <= 32)")
    ap.add_argument("--dense", type=int, default=0, metavar="I",
                    help="instead: the dense SwiGLU FFN (moe_dense_ffn) of intermediate size I")
    ap.add_argument("--dense-tokens", default="1,64,512,8192", metavar="T,T,...",
                    help="token counts of the --dense measurement")
    ap.add_argument("--cpu-tokens", type=int, default=64, help="tokens in the CPU oracle sample")
    ap.add_argument("--copy-probe", action="store_true")
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
    t0 = time.perf_counter()
    base = CONFIGS["decode"] if shape.weight_format != "mxfp4" else shape
    log(f"drawing {shape.E} experts ({shape.weight_format}) ...")
    experts = gen_experts(base if shape.weight_format != "mxfp4" else shape, seed=0)
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
        "dtype": "bf16" if shape.weight_format == "bf16" else "mxfp4-w/bf16",
        "data": "synthetic (seeded; random-init weights of the layer's shape)",
        "config": {"workload": f"{shape.name}: T={shape.T}, hidden {shape.H}, {shape.E} experts (I={shape.I}) "
                               f"in {shape.G} groups, top-{shape.TG} groups, top-{shape.K}, 1 shared expert",
                   "T": shape.T, "hidden_size": shape.H, "num_experts": shape.E, "moe_intermediate_size": shape.I,
                   "n_group": shape.G, "topk_group": shape.TG, "num_experts_per_tok": shape.K,
                   "weights": shape.weight_format, "parallelism": "single GPU"},
        "roofline": roofline(shape, r),
        "layer": layer_summary(shape, r),
        "kernels_ms": {k: round(v, 4) for k, v in r["kernels"].items()},
        "kernels_ms_from": "forwards with an event after every kernel, outside the timed region",
        "event_ms_per_step": round(r["event_ms"], 4),
        "expert_bias_update": time_bias_update(shape, r["counts"], hip),
    }
    if not args.no_prefill and shape.name == "decode":
        p = CONFIGS["prefill"]
        dp = upload(p, experts)
        log(f"measuring prefill T={p.T}")
        rp = measure(p, dp, max(5, args.steps // 3), 3, hip)
        line["prefill"] = {"workload": f"prefill: T={p.T}, same layer", "value": round(p.T / (rp["wall_ms"] * 1e-3), 1),
                           "unit": "tokens/s", "ms_per_step": round(rp["wall_ms"], 4), "roofline": roofline(p, rp),
                           "layer": layer_summary(p, rp), "kernels_ms": {k: round(v, 4) for k, v in rp["kernels"].items()}}
        del dp
    if not args.no_cpu_baseline:
        log("timing the CPU oracle ...")
        line["cpu_baseline"] = cpu_baseline(shape, d, experts, args.cpu_tokens)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
