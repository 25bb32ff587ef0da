"""GPU parity: the HIP library (called through the C ABI) against the CPU oracle on seeded
synthetic inputs.

Bar: expert indices and per-expert counts bit-exact except on tokens whose routing score gap is
below 1e-6 (counted and reported); outputs within max|err| <= 2e-2 * RMS(oracle output) for
bf16 expert weights and 5e-2 * RMS for MXFP4 (against the oracle on the decoded weights)."""
import sys

import numpy as np
import pytest

import oracle
from synthetic import CONFIGS, gen_experts, quantise_mxfp4, quantise_mxfp8

from moe_case import (DeviceCase, compare_routing, expected_counts, host_case, oracle_forward, oracle_route, rms,
                      to_bits, to_dev)

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2
TOL_MXFP4 = 5e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def check_forward(c, rows=None, tol=TOL_BF16, dev=None):
    """Run moe_forward on the whole case; compare routing for every token and the output on
    `rows` (all tokens if None)."""
    s = c.shape
    say(f"[gpu] moe_forward {s.name} T={s.T} H={s.H} E={s.E} fmt={s.weight_format} seed={c.seed}")
    dev = dev or DeviceCase(c)
    out, idx, w, cnt = dev.forward()
    out_b = oracle.bf16_to_f64(to_bits(out))
    idx, w, cnt = idx.cpu().numpy(), w.cpu().numpy(), cnt.cpu().numpy()
    r_all = oracle_route(c)
    n_tie, n_mis = compare_routing(r_all, idx, w)
    say(f"      near-ties {n_tie} (routing differs on {n_mis} of them; those are the only tokens excused)")
    np.testing.assert_array_equal(cnt, expected_counts(r_all, idx, s.E, s.T, s.num_shared_experts))
    if callable(rows):
        rows = rows(r_all)
    if rows is not None:
        say(f"      output checked on {len(rows)} rows")
        c.prefetch(np.unique(r_all.topk_idx[rows]))
    ref, r = oracle_forward(c, rows)
    got = out_b if rows is None else out_b[rows]
    keep = ~r.near_tie
    err = np.abs(got - ref)[keep]
    bound = tol * rms(ref)
    say(f"      max|err| = {err.max():.3e}, RMS(ref) = {rms(ref):.3e}, ratio {err.max() / rms(ref):.3e} (bar {tol})")
    assert err.max() <= bound
    return dev, out


# ----------------------------------------------------------------------------------
# tiny layer: every token, every stage
# ----------------------------------------------------------------------------------
@pytest.mark.parametrize("T", [32, 1, 17, 63, 64, 65, 200, 256, 257, 1000])  # 256 / 257: the last fused dispatch and the first separate one
def test_forward_tiny(T):
    check_forward(host_case(CONFIGS["tiny"], seed=0, T=T))


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_forward_tiny_seeds(seed):
    check_forward(host_case(CONFIGS["tiny"], seed=seed, T=96))


def test_forward_tiny_clamped():
    c = host_case(CONFIGS["tiny"].with_(swiglu_limit=0.002, shared_swiglu_limit=0.003), seed=5, T=77)
    check_forward(c)


def test_forward_tiny_no_shared_no_norm():
    c = host_case(CONFIGS["tiny"].with_(num_shared_experts=0, norm_topk_prob=False), seed=6, T=50)
    check_forward(c)


def test_stages_tiny():
    """Each entry point alone, fed the oracle's outputs of the previous stage."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    c = host_case(CONFIGS["tiny"], seed=7, T=130)
    s = c.shape
    T, K, E, H = s.T, s.K, s.E, s.H
    dev = DeviceCase(c)
    say("[gpu] moe_route tiny T=130")
    idx = torch.empty((T, K), dtype=torch.int32, device="cuda")
    w = torch.empty((T, K), dtype=torch.float32, device="cuda")
    moe.moe_route(dev.cfg, T, dev.x, dev.router_w, dev.bias, idx, w, dev.ws)
    torch.cuda.synchronize()
    r = oracle_route(c)
    compare_routing(r, idx.cpu().numpy(), w.cpu().numpy())

    say("[gpu] moe_dispatch tiny T=130 (oracle routing in)")
    d = oracle.dispatch(r.topk_idx, E, 1)
    idx_in = to_dev(r.topk_idx.astype(np.int32))
    counts = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 2, dtype=torch.int32, device="cuda")
    sorted_token = torch.empty(T * K + T, dtype=torch.int32, device="cuda")
    inv = torch.empty((T, K), dtype=torch.int32, device="cuda")
    moe.moe_dispatch(dev.cfg, T, idx_in, counts, offsets, sorted_token, inv, dev.ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(counts.cpu().numpy(), d.counts)
    np.testing.assert_array_equal(offsets.cpu().numpy(), d.offsets)
    np.testing.assert_array_equal(sorted_token.cpu().numpy(), d.sorted_token)
    np.testing.assert_array_equal(inv.cpu().numpy(), d.inv_perm)

    say("[gpu] moe_expert_ffn tiny T=130 (oracle dispatch in)")
    y = torch.empty((T * K + T, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(dev.cfg, T, dev.x, to_dev(d.offsets.astype(np.int32)), to_dev(d.sorted_token.astype(np.int32)),
                       dev.weights, y, dev.ws)
    torch.cuda.synchronize()
    x = oracle.bf16_to_f64(c.x)
    y_ref = np.zeros((T * K + T, H))
    for e in range(E + 1):
        p0, p1 = d.offsets[e], d.offsets[e + 1]
        if p1 > p0:
            wts = c.expert_f64(e) if e < E else c.shared_f64()
            y_ref[p0:p1] = oracle.expert_forward(x[d.sorted_token[p0:p1]], *wts)
    y_got = y.cpu().numpy().astype(np.float64)
    assert np.abs(y_got - y_ref).max() <= TOL_BF16 * rms(y_ref)

    say("[gpu] moe_combine tiny T=130 (oracle expert outputs in, rounded to fp32)")
    y32 = y_ref.astype(np.float32)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(dev.cfg, T, to_dev(y32), to_dev(d.inv_perm.astype(np.int32)),
                    to_dev(r.topk_w.astype(np.float32)), out)
    torch.cuda.synchronize()
    yb = y32.astype(np.float64)
    ref = (r.topk_w[:, :, None] * yb[d.inv_perm]).sum(1) + yb[T * K:]
    got = oracle.bf16_to_f64(to_bits(out))
    # only fp32 accumulation and the final bf16 rounding separate the two
    assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6 * rms(ref))


def test_stages_tiny_ignored_ids():
    """moe_dispatch given ids outside [0, E) (never produced by the router; the library's
    contract drops them): counts, offsets, sorted tokens and inv_perm bit-exact against the
    oracle's dispatch (the shared expert's block still at T*K, the gap filled with -1); then
    the FFN and combine on the GPU's dispatch, against the oracle with those slots dropped."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    c = host_case(CONFIGS["tiny"], seed=19, T=100)
    s = c.shape
    T, K, E, H = s.T, s.K, s.E, s.H
    dev = DeviceCase(c)
    r = oracle_route(c)
    idx = r.topk_idx.copy()
    rng = np.random.default_rng(19)
    drop = rng.random((T, K)) < 0.15
    idx[drop] = rng.choice([-1, -3, E, E + 9], size=int(drop.sum()))
    say(f"[gpu] moe_dispatch tiny T={T} with {int(drop.sum())} ignored ids")
    d = oracle.dispatch(idx, E, 1)
    counts = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 2, dtype=torch.int32, device="cuda")
    sorted_token = torch.full((T * K + T,), 12345, dtype=torch.int32, device="cuda")
    inv = torch.empty((T, K), dtype=torch.int32, device="cuda")
    moe.moe_dispatch(dev.cfg, T, to_dev(idx.astype(np.int32)), counts, offsets, sorted_token, inv, dev.ws)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(counts.cpu().numpy(), d.counts)
    np.testing.assert_array_equal(offsets.cpu().numpy(), d.offsets)
    np.testing.assert_array_equal(sorted_token.cpu().numpy(), d.sorted_token)
    np.testing.assert_array_equal(inv.cpu().numpy(), d.inv_perm)

    say(f"[gpu] moe_expert_ffn + moe_combine tiny T={T} on that dispatch")
    y = torch.empty((T * K + T, H), dtype=torch.float32, device="cuda")
    moe.moe_expert_ffn(dev.cfg, T, dev.x, offsets, sorted_token, dev.weights, y, dev.ws)
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    moe.moe_combine(dev.cfg, T, y, inv, to_dev(r.topk_w.astype(np.float32)), out)
    torch.cuda.synchronize()
    x = oracle.bf16_to_f64(c.x)
    ref = oracle.expert_forward(x, *c.shared_f64())
    for t in range(T):
        for k in range(K):
            if not drop[t, k]:
                ref[t] += r.topk_w[t, k] * oracle.expert_forward(x[t:t + 1], *c.expert_f64(int(idx[t, k])))[0]
    got = oracle.bf16_to_f64(to_bits(out))
    err = np.abs(got - ref).max() / rms(ref)
    say(f"      max|err| / RMS = {err:.3e} (bar {TOL_BF16})")
    assert err <= TOL_BF16


def test_forward_tile_kernel_short_items():
    """The 256-position tile kernel with work items of exactly one prefetch distance (two
    steps): hidden 768 and intermediate 128 give down items of one 256-row block and 128
    k-values, and at T = 20000 (312 tokens per expert) workgroups take three or more of them
    in a row.  Every output row against the oracle."""
    s = CONFIGS["tiny"].with_(hidden_size=768, num_experts=512, moe_intermediate_size=128,
                              shared_intermediate_size=128)
    check_forward(host_case(s, seed=21, T=20000))


@pytest.mark.parametrize("T", [385, 2048, 4099])
def test_forward_tiny_large_tiles(T):
    # T*K/E above 48 tokens per expert selects the 256-position tile kernels; at T = 2048 and
    # 4099 many experts span two or more tiles and the last tile of each is ragged
    check_forward(host_case(CONFIGS["tiny"], seed=14, T=T))


def test_forward_tiles_unsupported_shape():
    # hidden 384 is not a multiple of the 256-row down block: many tokens per expert must
    # still be served, by the small-tile kernels
    check_forward(host_case(CONFIGS["tiny"].with_(hidden_size=384), seed=15, T=1000))


# T = 40: 16-token tiles; 600 (75 tokens per expert): 64-token tiles; 1000: 128-token tiles;
# the clamped cases put the SwiGLU limits on the MXFP4 epilogue (routed) and the bf16 one (shared)
@pytest.mark.parametrize("T,limit", [(40, 0.0), (600, 0.0), (1000, 0.0), (40, 0.002), (600, 0.002)])
def test_forward_tiny_mxfp4(T, limit):
    s = CONFIGS["tiny"].with_(weight_format="mxfp4")
    if limit:
        s = s.with_(swiglu_limit=limit, shared_swiglu_limit=1.5 * limit)
    bf = gen_experts(CONFIGS["tiny"], seed=16)
    ex = {}
    for k in ("gate", "up", "down"):
        qs = [quantise_mxfp4(bf[k][e]) for e in range(s.E)]
        ex[k + "_q"] = np.stack([a for a, _ in qs])
        ex[k + "_s"] = np.stack([b for _, b in qs])
    check_forward(host_case(s, seed=16, T=T, experts=ex), tol=TOL_MXFP4)


def _tiny_block_experts(fmt, seed):
    """The tiny layer's bf16 experts encoded in a block format (MXFP4 or MXFP8)."""
    quant = quantise_mxfp4 if fmt == "mxfp4" else quantise_mxfp8
    bf = gen_experts(CONFIGS["tiny"], seed=seed)
    ex = {}
    for k in ("gate", "up", "down"):
        qs = [quant(bf[k][e]) for e in range(CONFIGS["tiny"].E)]
        ex[k + "_q"] = np.stack([a for a, _ in qs])
        ex[k + "_s"] = np.stack([b for _, b in qs])
    return ex


# MXFP8 weights decoded exactly to bf16: the bf16 bar.  T = 40: 16-token tiles, 600: 64-token
# tiles, 1000: 128-token tiles; clamped on both epilogues
@pytest.mark.parametrize("T,limit", [(40, 0.0), (600, 0.0), (1000, 0.0), (40, 0.002), (600, 0.002)])
def test_forward_tiny_mxfp8(T, limit):
    s = CONFIGS["tiny"].with_(weight_format="mxfp8")
    if limit:
        s = s.with_(swiglu_limit=limit, shared_swiglu_limit=1.5 * limit)
    check_forward(host_case(s, seed=22, T=T, experts=_tiny_block_experts("mxfp8", 22)), tol=TOL_BF16)


def _tiled_case(dev):
    """A copy of a device case whose MXFP4 or MXFP8 experts are packed on the GPU into the
    tiled order (moe_pack_mxfp4 / moe_pack_mxfp8) and named so in the config."""
    import copy
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    s = dev.c.shape
    fp4 = s.weight_format == "mxfp4"
    pack = moe.moe_pack_mxfp4 if fp4 else moe.moe_pack_mxfp8
    keep = dev.weights._keep
    packed = []
    for q, sc, (N, Kd) in zip(keep[0:3], keep[3:6], ((s.I, s.H), (s.I, s.H), (s.H, s.I))):
        qo, so = torch.empty_like(q), torch.empty_like(sc)
        pack(q, sc, s.E, N, Kd, qo, so)
        packed.append((qo, so))
    torch.cuda.synchronize()
    t = copy.copy(dev)
    t.cfg = type(dev.cfg).from_buffer_copy(dev.cfg)
    t.cfg.expert_weight_format = moe.MOE_WEIGHTS_MXFP4_TILED if fp4 else moe.MOE_WEIGHTS_MXFP8_TILED
    t.weights = moe.MoEExpertWeights(*[p[0] for p in packed], *[p[1] for p in packed], *keep[6:9])
    return t


def _assert_same_forward(a, b):
    import torch
    for u, v in zip(a.forward(), b.forward()):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)


def test_pack_mxfp4_layout():
    """moe_pack_mxfp4 against the tiled order as moe.h defines it, written out with numpy
    reshapes: codes in 1 KB blocks (b, s) whose 16 bytes at 16*(16q + r) are row 16b + r's
    bytes 64s + 16q .. +15; scales in 128-byte blocks (b, t) whose byte 8r + i is row 16b + r's
    scale 8t + i.  Two shapes: three 48 x 512 matrices, and two of the down projection's
    2560 x 768 (an odd number of 256-value scale blocks per row)."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    rng = np.random.default_rng(31)
    for M, N, Kd in ((3, 48, 512), (2, 2560, 768)):
        say(f"[gpu] moe_pack_mxfp4 {M}x{N}x{Kd}")
        q = rng.integers(0, 256, size=(M, N, Kd // 2), dtype=np.uint8)
        sc = rng.integers(0, 256, size=(M, N, Kd // 32), dtype=np.uint8)
        qo = torch.empty(q.size, dtype=torch.uint8, device="cuda")
        so = torch.empty(sc.size, dtype=torch.uint8, device="cuda")
        moe.moe_pack_mxfp4(to_dev(q), to_dev(sc), M, N, Kd, qo, so)
        torch.cuda.synchronize()
        want_q = q.reshape(M, N // 16, 16, Kd // 128, 4, 16).transpose(0, 1, 3, 4, 2, 5).ravel()
        want_s = sc.reshape(M, N // 16, 16, Kd // 256, 8).transpose(0, 1, 3, 2, 4).ravel()
        np.testing.assert_array_equal(qo.cpu().numpy(), want_q)
        np.testing.assert_array_equal(so.cpu().numpy(), want_s)


def test_pack_mxfp8_layout():
    """moe_pack_mxfp8 against moe.h's tiled MXFP8 order, written out with numpy reshapes: 2 KB
    blocks (b, s) whose 16 bytes at 1024p + 16*(16q + r) are row 16b + r's bytes
    128s + 64p + 16q .. +15; scales as for MXFP4."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    rng = np.random.default_rng(32)
    for M, N, Kd in ((3, 48, 512), (2, 2560, 768)):
        say(f"[gpu] moe_pack_mxfp8 {M}x{N}x{Kd}")
        q = rng.integers(0, 256, size=(M, N, Kd), dtype=np.uint8)
        sc = rng.integers(0, 256, size=(M, N, Kd // 32), dtype=np.uint8)
        qo = torch.empty(q.size, dtype=torch.uint8, device="cuda")
        so = torch.empty(sc.size, dtype=torch.uint8, device="cuda")
        moe.moe_pack_mxfp8(to_dev(q), to_dev(sc), M, N, Kd, qo, so)
        torch.cuda.synchronize()
        want_q = q.reshape(M, N // 16, 16, Kd // 128, 2, 4, 16).transpose(0, 1, 3, 4, 5, 2, 6).ravel()
        want_s = sc.reshape(M, N // 16, 16, Kd // 256, 8).transpose(0, 1, 3, 2, 4).ravel()
        np.testing.assert_array_equal(qo.cpu().numpy(), want_q)
        np.testing.assert_array_equal(so.cpu().numpy(), want_s)


# Tiled MXFP4 / MXFP8 weights give the row-major layer bit for bit (the same products in the
# same order), with bf16 and MXFP8 activations, 16-, 64- and 128-token tiles; intermediate 256
# (the tiled order needs multiples of 256); and the tiled layer against the oracle once
@pytest.mark.parametrize("wfmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("act", ["bf16", "mxfp8"])
@pytest.mark.parametrize("T", [40, 600, 3000])
def test_forward_tiny_block_tiled(wfmt, act, T):
    base = CONFIGS["tiny"].with_(moe_intermediate_size=256, shared_intermediate_size=256)
    s = base.with_(weight_format=wfmt, act_format=act)
    quant = quantise_mxfp4 if wfmt == "mxfp4" else quantise_mxfp8
    bf = gen_experts(base, seed=25)
    ex = {}
    for k in ("gate", "up", "down"):
        qs = [quant(bf[k][e]) for e in range(s.E)]
        ex[k + "_q"] = np.stack([a for a, _ in qs])
        ex[k + "_s"] = np.stack([b for _, b in qs])
    c = host_case(s, seed=25, T=T, experts=ex)
    dev = DeviceCase(c)
    tiled = _tiled_case(dev)
    say(f"[gpu] moe_forward tiny I=256 T={T} {wfmt} act={act}: tiled against row-major")
    _assert_same_forward(dev, tiled)
    if T == 600:
        check_forward(c, tol=TOL_BF16 if (wfmt, act) == ("mxfp8", "bf16") else TOL_MXFP4, dev=tiled)


def test_quantise_mxfp8_bit_exact():
    """The device MXFP8 rounding (moe_quantise_mxfp8, the code the 8-bit-activation path runs on
    x and, in the gate/up epilogue, on h) against the oracle's quantiser, code for code and
    scale for scale: bf16 rows over 2^-133 .. 2^20, exact ties between E4M3 neighbours,
    saturating blocks, all-zero blocks and bf16 subnormals."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    from synthetic import f32_to_bf16_bits
    rng = np.random.default_rng(23)
    R, C = 96, 512
    v = rng.standard_normal((R, C)) * np.exp2(rng.integers(-40, 20, size=(R, 1)))
    v[1] = 0.0
    v[2, :32] = 2.0 ** -133 * np.arange(32)                      # bf16 subnormals
    ties = np.array([1.0625, 1.1875, 1.3125, -1.4375, 3.25, 0.2578125, 448 / 256, 480 / 256])
    v[3, :32] = 1.0
    v[3, 1:1 + ties.size] = ties                                  # amax 1 -> scaled by 256: ties and 448, 480
    v[4, :32] = np.linspace(-1.9, 1.9, 32)                        # saturation at both ends
    bits = f32_to_bf16_bits(v.astype(np.float32))
    say(f"[gpu] moe_quantise_mxfp8 {R}x{C}")
    x = to_dev(bits, bf16=True)
    codes = torch.empty((R, C), dtype=torch.uint8, device="cuda")
    scales = torch.empty((R, C // 32), dtype=torch.uint8, device="cuda")
    moe.moe_quantise_mxfp8(x, R, C, codes, scales)
    torch.cuda.synchronize()
    want_c, want_s = oracle.mxfp8_quantise(oracle.bf16_to_f64(bits))
    np.testing.assert_array_equal(scales.cpu().numpy(), want_s)
    got = codes.cpu().numpy()
    # +0 and -0 are the same value: compare decoded values, and codes where the value is nonzero
    np.testing.assert_array_equal(oracle.e4m3_value(got), oracle.e4m3_value(want_c))
    nz = oracle.e4m3_value(want_c) != 0
    np.testing.assert_array_equal(got[nz], want_c[nz])


# MXFP8 activations on the routed experts (scaled MFMA), against the oracle's act_quant="mxfp8"
# mode; MXFP4 and MXFP8 weights; 16-, 64- and 128-token tiles; the clamp before h's rounding
@pytest.mark.parametrize("wfmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("T,limit", [(40, 0.0), (600, 0.0), (1000, 0.0), (40, 0.002), (3000, 0.002)])
def test_forward_tiny_act_mxfp8(wfmt, T, limit):
    s = CONFIGS["tiny"].with_(weight_format=wfmt, act_format="mxfp8")
    if limit:
        s = s.with_(swiglu_limit=limit, shared_swiglu_limit=1.5 * limit)
    check_forward(host_case(s, seed=24, T=T, experts=_tiny_block_experts(wfmt, 24)), tol=TOL_MXFP4)


# the MXFP8-activation down GEMM keeps a tile's whole h in LDS when its reduction is three
# steps: intermediate 384 (128-value steps) and 768 (256-value steps); several row blocks per
# workgroup (hidden 512: four 128-row blocks) reuse it
@pytest.mark.parametrize("wfmt", ["mxfp4", "mxfp8"])
@pytest.mark.parametrize("I,T", [(384, 40), (384, 600), (768, 600), (768, 3000)])
def test_forward_tiny_act_mxfp8_resident_h(wfmt, I, T):
    base = CONFIGS["tiny"].with_(moe_intermediate_size=I, shared_intermediate_size=I)
    s = base.with_(weight_format=wfmt, act_format="mxfp8")
    quant = quantise_mxfp4 if wfmt == "mxfp4" else quantise_mxfp8
    bf = gen_experts(base, seed=26)
    ex = {}
    for k in ("gate", "up", "down"):
        qs = [quant(bf[k][e]) for e in range(s.E)]
        ex[k + "_q"] = np.stack([a for a, _ in qs])
        ex[k + "_s"] = np.stack([b for _, b in qs])
    check_forward(host_case(s, seed=26, T=T, experts=ex), tol=TOL_MXFP4)


def test_determinism_tiny_tiles():
    import torch
    c = host_case(CONFIGS["tiny"], seed=17, T=2048)
    dev = DeviceCase(c)
    say("[gpu] moe_forward twice, tiny T=2048 (256-position tiles)")
    a = [t.clone() for t in dev.forward()]
    b = dev.forward()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)


# other expert counts, group layouts and fan-outs: one case per top-k kernel instantiation
# (experts per lane 1, 2, 4, 8, 16) and the degenerate group settings
LAYOUTS = [
    dict(num_experts=128, n_group=8, topk_group=4, num_experts_per_tok=8),     # 2 experts per lane
    dict(num_experts=256, n_group=4, topk_group=2, num_experts_per_tok=6),     # 4 per lane
    dict(num_experts=1024, n_group=16, topk_group=8, num_experts_per_tok=16),  # 16 per lane, K at its maximum
    dict(num_experts=64, n_group=1, topk_group=1, num_experts_per_tok=1),      # one group, top-1
    dict(num_experts=64, n_group=64, topk_group=8, num_experts_per_tok=8),     # one expert per group
]


@pytest.mark.parametrize("layout", LAYOUTS, ids=lambda d: "E{num_experts}_G{n_group}_TG{topk_group}_K{num_experts_per_tok}".format(**d))
@pytest.mark.parametrize("T", [70, 1100])
def test_forward_layouts(layout, T):
    s = CONFIGS["tiny"].with_(hidden_size=256, **layout)
    check_forward(host_case(s, seed=18, T=T))


def test_determinism_tiny():
    import torch
    c = host_case(CONFIGS["tiny"], seed=8, T=300)
    dev = DeviceCase(c)
    say("[gpu] moe_forward twice, tiny T=300")
    a = [t.clone() for t in dev.forward()]
    b = dev.forward()
    for u, v in zip(a, b):
        assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                           v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)


def test_forwards_from_two_threads_block_format():
    """With block-format experts moe_forward runs the shared expert on the library's second
    stream, forked and joined under a mutex: two host threads that enqueue forwards at the same
    time, each on its own stream with its own workspace, get the bits of forwards run one by
    one."""
    import threading
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    devs = []
    for seed, wfmt in ((41, "mxfp4"), (42, "mxfp8")):
        c = host_case(CONFIGS["tiny"].with_(weight_format=wfmt), seed=seed, T=600,
                      experts=_tiny_block_experts(wfmt, seed))
        devs.append(DeviceCase(c))
    say("[gpu] moe_forward from two host threads on two streams, tiny T=600 mxfp4 / mxfp8")
    refs = [[t.clone() for t in d.forward()] for d in devs]
    n = 12
    outs = []
    for d in devs:
        s = d.c.shape
        outs.append([(torch.empty((d.T, s.H), dtype=torch.bfloat16, device="cuda"),
                      torch.empty((d.T, s.K), dtype=torch.int32, device="cuda"),
                      torch.empty((d.T, s.K), dtype=torch.float32, device="cuda"),
                      torch.empty((s.E + 1,), dtype=torch.int32, device="cuda")) for _ in range(n)])
    streams = [torch.cuda.Stream() for _ in devs]  # default priority
    torch.cuda.synchronize()
    errors = []

    def run(i):
        try:
            d = devs[i]
            for o in outs[i]:
                moe.moe_forward(d.cfg, d.T, d.x, d.router_w, d.bias, d.weights, *o, d.ws, stream=streams[i])
        except Exception as e:  # reported after the join
            errors.append(e)
    threads = [threading.Thread(target=run, args=(i,)) for i in range(len(devs))]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for ref, runs in zip(refs, outs):
        for o in runs:
            for u, v in zip(ref, o):
                assert torch.equal(u.view(torch.uint8) if u.dtype == torch.bfloat16 else u,
                                   v.view(torch.uint8) if v.dtype == torch.bfloat16 else v)


@pytest.mark.parametrize("T,wfmt", [(40, "bf16"), (700, "bf16"), (2048, "bf16"), (40, "mxfp4"), (600, "mxfp8")])
def test_traced_and_timed_forwards_match_forward(T, wfmt):
    """The profiling entry points compute the same layer, bit for bit; every kernel of the
    step can be timed by events bound to its dispatch, and an index past the last kernel is
    an error (after the layer ran).  With block-format experts, moe_forward and
    moe_forward_timed run the shared expert on the library's second stream and
    moe_forward_traced runs every kernel on the caller's: the same bits either way.  (T = 2048
    puts the bf16 layer on the 256-position tile kernels.)"""
    import ctypes
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    if wfmt == "bf16":
        c = host_case(CONFIGS["tiny"], seed=11, T=T)
    else:
        c = host_case(CONFIGS["tiny"].with_(weight_format=wfmt), seed=11, T=T,
                      experts=_tiny_block_experts(wfmt, 11))
    dev = DeviceCase(c)
    say(f"[gpu] moe_forward / moe_forward_traced / moe_forward_timed, tiny T={T} {wfmt} experts")
    ref = dev.forward()[0].clone()
    hip = ctypes.CDLL("libamdhip64.so.7")

    def event():
        ev = ctypes.c_void_p()
        assert hip.hipEventCreate(ctypes.byref(ev)) == 0
        return ev.value

    def elapsed(a, b):
        ms = ctypes.c_float()
        assert hip.hipEventSynchronize(ctypes.c_void_p(b)) == 0
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) == 0
        return ms.value

    out = torch.empty_like(ref)
    events = [event() for _ in range(16)]
    names = moe.moe_forward_traced(dev.cfg, T, dev.x, dev.router_w, dev.bias, dev.weights, out, dev.ws, events)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    assert names[0] in ("router_logits", "router_split") and names[-1] == "combine" and "expert_gate_up" in names
    for k, name in enumerate(names):
        out.zero_()
        a, b = event(), event()
        moe.moe_forward_timed(dev.cfg, T, dev.x, dev.router_w, dev.bias, dev.weights, out, dev.ws, k, a, b)
        torch.cuda.synchronize()
        ms = elapsed(a, b)
        say(f"      kernel {k} {name}: {ms * 1e3:.1f} us")
        assert 0.0 < ms < 1000.0
        assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
    a, b = event(), event()
    with pytest.raises(moe.MoEError):
        moe.moe_forward_timed(dev.cfg, T, dev.x, dev.router_w, dev.bias, dev.weights, out, dev.ws, len(names), a, b)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_expert_bias_update_matches_oracle(name):
    """The bias update from a forward's own counts, on the same stream, bit for bit against
    the oracle (routing walk-through page, section 三.3, sign rule); then a balanced
    histogram, which must leave the bias as it is."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    s = CONFIGS[name]
    c = host_case(s, seed=12, T=64) if name == "tiny" else None
    if c is None:
        cfg = moe.MoEConfig(hidden_size=s.H, num_experts=s.E, num_experts_per_tok=s.K, n_group=s.G,
                            topk_group=s.TG, moe_intermediate_size=s.I, num_shared_experts=1,
                            shared_intermediate_size=s.I_s, norm_topk_prob=1, routed_scaling_factor=2.5,
                            swiglu_limit=0.0, shared_swiglu_limit=0.0, expert_weight_format=moe.MOE_WEIGHTS_BF16)
        rng = np.random.default_rng(12)
        counts_h = rng.poisson(1.0, size=s.E + 1).astype(np.int32)
        counts = torch.from_numpy(counts_h).cuda()
    else:
        dev = DeviceCase(c)
        cfg = dev.cfg
        counts = dev.forward()[3]
        counts_h = counts.cpu().numpy()
    say(f"[gpu] moe_update_expert_bias {name} E={s.E}")
    rng = np.random.default_rng(13)
    bias_h = rng.uniform(-0.1, 0.1, size=s.E).astype(np.float32)
    bias_h[:3] = [0.0, -0.0, 1.0]
    bias = torch.from_numpy(bias_h.copy()).cuda()
    gamma = 1e-3
    moe.moe_update_expert_bias(cfg, counts, bias, gamma)
    torch.cuda.synchronize()
    want = oracle.update_expert_bias(bias_h, counts_h, gamma)
    got = bias.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    # a second step from a balanced histogram changes nothing
    flat = torch.full((s.E + 1,), 5, dtype=torch.int32, device="cuda")
    moe.moe_update_expert_bias(cfg, flat, bias, gamma)
    torch.cuda.synchronize()
    assert np.array_equal(bias.cpu().numpy().view(np.uint32), oracle.update_expert_bias(want, np.full(s.E + 1, 5), gamma).view(np.uint32))


# up to 10 tokens the dense FFN runs its own kernels (the reduction split over the waves of a
# workgroup; 32-value steps where the preferred step does not divide a wave's slice, as at
# H = 384 and I = 640); up to 4096 tokens the expert FFN kernels with tiles computed from T (16
# to 256 tokens, no dispatch or combine; up to 512 tokens the down reduction split over
# workgroups and summed in order by a last kernel); beyond, the 256-position tile kernel as a
# one-expert layer
@pytest.mark.parametrize("H,I,T,limit", [(512, 384, 1, 0.0), (384, 640, 9, 0.0), (512, 768, 10, 0.003),
                                         (2560, 6912, 1, 0.0), (2560, 6912, 8, 0.0), (512, 768, 11, 0.0),
                                         (2560, 6912, 16, 0.0), (384, 640, 13, 0.0), (512, 768, 17, 0.0),
                                         (512, 768, 29, 0.003), (512, 384, 32, 0.0), (384, 2048, 50, 0.0),
                                         (512, 384, 64, 0.002), (2560, 6912, 64, 0.0), (512, 384, 70, 0.0),
                                         (512, 384, 129, 0.0), (512, 384, 257, 0.0), (512, 640, 300, 0.002),
                                         (512, 640, 513, 0.002), (512, 384, 1500, 0.0), (2560, 6912, 1100, 0.0),
                                         (384, 384, 2049, 0.0), (512, 384, 3000, 0.0), (512, 384, 4100, 0.002)])
def test_dense_ffn_matches_oracle(H, I, T, limit):
    """Dense SwiGLU FFN (the layers before the MoE stack) against the oracle's SwiGLU FFN in
    float64: every output row at small sizes, 64 sampled rows at the full hidden size."""
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    rng = np.random.default_rng(20 + T)
    say(f"[gpu] moe_dense_ffn H={H} I={I} T={T} limit={limit}")

    def bf16(shape, scale):
        v = (rng.standard_normal(shape) * scale).astype(np.float32)
        return (v.view(np.uint32) >> 16).astype(np.uint16)  # truncation keeps it exactly bf16

    x, g, u, d = bf16((T, H), 1.0), bf16((I, H), 0.02), bf16((I, H), 0.02), bf16((H, I), 0.02)
    dev = [to_dev(a, bf16=True) for a in (x, g, u, d)]
    out = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.moe_dense_ffn_workspace_size(H, I, T), dtype=torch.uint8, device="cuda")
    moe.moe_dense_ffn(H, I, limit, T, *dev, out, ws)
    torch.cuda.synchronize()
    rows = np.arange(T) if T * H <= 512 * 1500 else np.sort(rng.choice(T, size=64, replace=False))
    xf, gf, uf, df = (oracle.bf16_to_f64(a) for a in (x, g, u, d))
    ref = oracle.expert_forward(xf[rows], gf, uf, df, limit)
    got = oracle.bf16_to_f64(to_bits(out))[rows]
    err = np.abs(got - ref).max() / rms(ref)
    say(f"      max|err| / RMS = {err:.3e} (bar {TOL_BF16})")
    assert err <= TOL_BF16


# ----------------------------------------------------------------------------------
# adversarial fixtures (tiny layer)
# ----------------------------------------------------------------------------------
def test_fixture_negative_biased_scores():
    # every biased score below zero: experts of dropped groups must stay excluded
    s = CONFIGS["tiny"]
    c = host_case(s, seed=9, T=64, bias=np.full(s.E, -2.0, np.float32))
    check_forward(c)


def test_fixture_exact_ties_lower_index_wins():
    # experts 2j and 2j+1 get identical router rows and biases, so their scores are bitwise
    # equal on both sides; whenever only one of a pair is chosen it must be the lower one.
    # K = 7 is odd, so the pair at the K-th place is always split.
    s = CONFIGS["tiny"].with_(num_experts_per_tok=7)
    base = host_case(s, seed=10, T=64)
    rw = np.repeat(base.router_w[::2], 2, axis=0)
    bias = np.repeat(base.bias[::2], 2)
    c = host_case(s, seed=10, T=64, router_w=rw, bias=bias)
    say("[gpu] moe_forward tiny T=64 with tied expert pairs")
    dev = DeviceCase(c)
    out, idx, w, cnt = dev.forward()
    idx = idx.cpu().numpy()
    r = oracle_route(c)
    compare_routing(r, idx, w.cpu().numpy())
    for t in range(c.shape.T):
        chosen = set(idx[t].tolist())
        for e in chosen:
            if e % 2 == 1:
                assert e - 1 in chosen, (t, sorted(chosen))
    # the rule was exercised: some chosen expert's partner was left out
    assert any(sum((e ^ 1) in set(row.tolist()) for e in row) < len(row) for row in idx)


def test_fixture_all_tokens_same_experts():
    # a huge bias on 8 experts of one group sends every token to them (count = T each)
    s = CONFIGS["tiny"]
    bias = np.zeros(s.E, np.float32)
    hot = [8, 9, 10, 11, 12, 13, 14, 15]
    bias[hot] = 5.0
    c = host_case(s, seed=11, T=517, bias=bias)
    dev, _ = check_forward(c)
    out, idx, w, cnt = dev.forward()
    cnt = cnt.cpu().numpy()
    assert (cnt[hot] == 517).all() and cnt[:s.E].sum() == 517 * 8


def test_fixture_identical_experts():
    # all routed experts equal: out = 2.5 * FFN(x) + shared(x) whatever the routing
    s = CONFIGS["tiny"]
    ex = gen_experts(s, seed=12)
    for k in ("gate", "up", "down"):
        ex[k][:] = ex[k][3]
    c = host_case(s, seed=12, T=90, experts=ex)
    dev, out = check_forward(c)
    x = oracle.bf16_to_f64(c.x)
    want = 2.5 * oracle.expert_forward(x, *c.expert_f64(0)) + oracle.expert_forward(x, *c.shared_f64())
    got = oracle.bf16_to_f64(to_bits(out))
    assert np.abs(got - want).max() <= TOL_BF16 * rms(want)


def test_fixture_no_bias_pointer():
    import torch
    s = CONFIGS["tiny"]
    c = host_case(s, seed=13, T=40, bias=np.zeros(s.E, np.float32))
    dev = DeviceCase(c)
    a = dev.forward(bias=True)
    b = dev.forward(bias=False)
    for u, v in zip(a, b):
        assert torch.equal(u, v)


# ----------------------------------------------------------------------------------
# full-size layer (H 2560, 512 experts, intermediate 768)
# ----------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def full_experts():
    say("[host] drawing the 512 full-size experts (bf16)")
    return gen_experts(CONFIGS["decode"], seed=0)


@pytest.mark.slow
def test_forward_decode_full(full_experts):
    check_forward(host_case(CONFIGS["decode"], seed=0, experts=full_experts))


def _sample_rows(T, n=24):
    rng = np.random.default_rng(T)
    return np.unique(np.concatenate([[0, T - 1], rng.choice(T, n - 2, replace=False)]))


def tile_rows(bm, n_random=24, at_least=256):
    """Rows to check on a full-size run, chosen from the oracle's routing so that every tile
    of bm sorted positions of every expert (the shared expert's included) holds the first
    and the last token of that tile: a fault confined to one work item of the FFN kernels
    (a tile and its row blocks) then shows on a checked row.  Plus random rows, and more
    random rows up to `at_least`."""
    def pick(r):
        T = r.topk_idx.shape[0]
        E = r.counts.shape[0]
        d = oracle.dispatch(r.topk_idx, E, 1)
        rows = set()
        for e in range(E + 1):
            p0, n = int(d.offsets[e]), int(d.counts[e])
            for j0 in range(0, n, bm):
                rows.add(int(d.sorted_token[p0 + j0]))
                rows.add(int(d.sorted_token[p0 + min(n, j0 + bm) - 1]))
        rows.update(_sample_rows(T, n_random).tolist())
        rng = np.random.default_rng(T + 1)
        while len(rows) < min(at_least, T):
            rows.add(int(rng.integers(T)))
        return np.array(sorted(rows))
    return pick


@pytest.mark.slow
def test_forward_prefill_full(full_experts):
    c = host_case(CONFIGS["prefill"], seed=0, experts=full_experts)
    check_forward(c, rows=tile_rows(256))  # 256-position tiles of the tile kernels


@pytest.mark.slow
def test_forward_skewed_full(full_experts):
    c = host_case(CONFIGS["skewed"], seed=0, experts=full_experts)
    r = oracle_route(c)
    cnt = np.sort(r.counts)[::-1]
    top = cnt[: c.shape.E // 10].sum() / cnt.sum()
    say(f"      skew: top-10% experts take {top:.3f} of assignments; {(cnt > 0).sum()} experts touched")
    assert top > 0.5
    check_forward(c, rows=tile_rows(256))


@pytest.mark.slow
def test_forward_mxfp4_full(full_experts):
    from concurrent.futures import ThreadPoolExecutor
    s = CONFIGS["mxfp4"]
    E, I, H = s.E, s.I, s.H
    ex = dict(gate_q=np.empty((E, I, H // 2), np.uint8), gate_s=np.empty((E, I, H // 32), np.uint8),
              up_q=np.empty((E, I, H // 2), np.uint8), up_s=np.empty((E, I, H // 32), np.uint8),
              down_q=np.empty((E, H, I // 2), np.uint8), down_s=np.empty((E, H, I // 32), np.uint8))

    def q(e):
        for k in ("gate", "up", "down"):
            ex[k + "_q"][e], ex[k + "_s"][e] = quantise_mxfp4(full_experts[k][e])
    say("[host] quantising the 512 experts to MXFP4")
    with ThreadPoolExecutor(16) as pool:
        list(pool.map(q, range(E)))
    c = host_case(s, seed=0, experts=ex)
    dev, _ = check_forward(c, rows=tile_rows(64), tol=TOL_MXFP4)  # 64-token tiles at 64 tokens per expert
    say("[gpu] the same layer with the experts in the tiled MXFP4 order: bit-exact")
    _assert_same_forward(dev, _tiled_case(dev))


@pytest.mark.slow
def test_forward_mxfp8_full(full_experts):
    from concurrent.futures import ThreadPoolExecutor
    s = CONFIGS["mxfp8"]
    E, I, H = s.E, s.I, s.H
    ex = dict(gate_q=np.empty((E, I, H), np.uint8), gate_s=np.empty((E, I, H // 32), np.uint8),
              up_q=np.empty((E, I, H), np.uint8), up_s=np.empty((E, I, H // 32), np.uint8),
              down_q=np.empty((E, H, I), np.uint8), down_s=np.empty((E, H, I // 32), np.uint8))

    def q(e):
        for k in ("gate", "up", "down"):
            ex[k + "_q"][e], ex[k + "_s"][e] = quantise_mxfp8(full_experts[k][e])
    say("[host] quantising the 512 experts to MXFP8")
    with ThreadPoolExecutor(16) as pool:
        list(pool.map(q, range(E)))
    c = host_case(s, seed=0, experts=ex)
    dev, _ = check_forward(c, rows=tile_rows(64), tol=TOL_BF16)
    say("[gpu] the same layer with the experts in the tiled MXFP8 order: bit-exact")
    _assert_same_forward(dev, _tiled_case(dev))


@pytest.mark.slow
@pytest.mark.parametrize("wfmt", ["mxfp4", "mxfp8"])
def test_forward_act_mxfp8_full(full_experts, wfmt):
    """The full-size layer with MXFP4 / MXFP8 routed experts and MXFP8 activations at T = 4096
    (64-token tiles), against the oracle's 8-bit-activation mode on every tile's first and
    last token."""
    from concurrent.futures import ThreadPoolExecutor
    s = CONFIGS[wfmt + "_a8"]
    E, I, H = s.E, s.I, s.H
    cd = 2 if wfmt == "mxfp4" else 1
    quant = quantise_mxfp4 if wfmt == "mxfp4" else quantise_mxfp8
    ex = dict(gate_q=np.empty((E, I, H // cd), np.uint8), gate_s=np.empty((E, I, H // 32), np.uint8),
              up_q=np.empty((E, I, H // cd), np.uint8), up_s=np.empty((E, I, H // 32), np.uint8),
              down_q=np.empty((E, H, I // cd), np.uint8), down_s=np.empty((E, H, I // 32), np.uint8))

    def q(e):
        for k in ("gate", "up", "down"):
            ex[k + "_q"][e], ex[k + "_s"][e] = quant(full_experts[k][e])
    say(f"[host] quantising the 512 experts to {wfmt}")
    with ThreadPoolExecutor(16) as pool:
        list(pool.map(q, range(E)))
    c = host_case(s, seed=0, experts=ex)
    dev, _ = check_forward(c, rows=tile_rows(64), tol=TOL_MXFP4)
    say(f"[gpu] the same layer with the experts in the tiled {wfmt} order: bit-exact")
    _assert_same_forward(dev, _tiled_case(dev))
