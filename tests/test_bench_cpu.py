"""Host-side checks of bench.py: the rocprofv3 summariser, the source-keyed traffic record
and the refusal of more than one GPU (no GPU needed)."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


@pytest.fixture()
def fake_profile(tmp_path, monkeypatch):
    src = tmp_path / "prof"
    gu = "void moe::(anonymous namespace)::ffn_kernel<4, 2, 1, 4, 0, 0>(moe::(anonymous namespace)::FfnArgs)"
    dn = "void moe::(anonymous namespace)::ffn_kernel<4, 2, 1, 4, 1, 0>(moe::(anonymous namespace)::FfnArgs)"
    cp = "__amd_rocclr_copyBuffer"
    _write(str(src / "kt" / "kt_kernel_stats.csv"), ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"],
           [[gu, 10, 3_000_000, 300_000.0, 60.0], [dn, 10, 1_500_000, 150_000.0, 30.0], [cp, 5, 500_000, 100_000, 10.0]])
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # copy of 1 GiB: FETCH_SIZE reads half the bytes it moves (factor 2), WRITE_SIZE all (factor 1)
    _write(str(src / "fetch" / "fetch_counter_collection.csv"), hdr,
           [[cp, "FETCH_SIZE", 524288.0], [cp, "FETCH_SIZE", 12.0], [gu, "FETCH_SIZE", 1000.0], [gu, "FETCH_SIZE", 1002.0],
            [dn, "FETCH_SIZE", 500.0]])
    _write(str(src / "write" / "write_counter_collection.csv"), hdr,
           [[cp, "WRITE_SIZE", 1048576.0], [gu, "WRITE_SIZE", 4.0], [dn, "WRITE_SIZE", 8.0]])
    out = tmp_path / "profiles"
    monkeypatch.setattr(bench, "PROFILES", str(out))
    monkeypatch.setattr(bench, "TRAFFIC_RECORD", str(out / "traffic.json"))
    return str(src), out


def test_summarize_scales_counters_by_the_copy(fake_profile):
    src, out = fake_profile
    bench.summarize(src, "decode")
    rec = json.load(open(out / "traffic.json"))["decode"]
    assert rec["expert_gate_up"]["fetch_bytes"] == round(1001.0 * 1024 * 2.0)
    assert rec["expert_gate_up"]["write_bytes"] == round(4.0 * 1024 * 1.0)
    assert rec["expert_down"]["fetch_bytes"] == round(500.0 * 1024 * 2.0)
    assert rec["expert_gate_up"]["source_sha256"] == bench.kernel_source_hash()
    md = (out / "expert_gate_up_decode_T64.md").read_text()
    assert "rocprofv3 --pmc FETCH_SIZE" in md and "ffn_kernel<4, 2, 1, 4, 0, 0>" in md


def test_traffic_is_null_once_the_sources_change(fake_profile, monkeypatch):
    src, out = fake_profile
    bench.summarize(src, "decode")
    assert bench.recorded_traffic("decode", "expert_gate_up") == round(1001.0 * 1024 * 2.0) + round(4.0 * 1024)
    assert bench.recorded_traffic("prefill", "expert_gate_up") is None
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 64)
    assert bench.recorded_traffic("decode", "expert_gate_up") is None


def test_symbols_map_to_steps():
    assert bench._step("ffn_tile_kernel<0, 8, 2, 3>") == "expert_gate_up"
    assert bench._step("ffn_tile_kernel<1, 16, 2, 3>") == "expert_down"
    assert bench._step("ffn_kernel<8, 1, 8, 4, 1, 1>") == "expert_down"
    assert bench._step("router_topk_kernel<8, true>") == "router_topk"
    assert bench._step("router_logits_kwaves_kernel<4>") == "router_logits"
    assert bench._step("router_logits_kernel<8, 2>") == "router_logits"
    assert bench._step("dispatch_count_kernel") == "dispatch_count"
    assert bench._step("something_else") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2 and "single MI355X" in r.stderr


def test_output_check_measures_against_the_oracle():
    """The benchmark's sampled output check: rows equal to the oracle's rounded to bf16 sit
    below the bar (the output's own bf16 rounding costs ~1.4 % of RMS), and a planted error in
    one row is reported at its size."""
    import numpy as np
    import oracle
    from synthetic import CONFIGS, gen_bias, gen_experts, gen_router, gen_shared, gen_x
    s = CONFIGS["tiny"].with_(T=100)
    d = dict(x_bits=gen_x(s, 0), router_w_np=gen_router(s), bias_np=gen_bias(s), shared_np=gen_shared(s))
    ex = gen_experts(s)
    rows = bench.check_rows(s.T)
    assert rows[0] == 0 and rows[-1] == s.T - 1 and len(rows) == 16
    ref, _ = oracle.moe_layer(oracle.bf16_to_f64(d["x_bits"][rows]), d["router_w_np"], d["bias_np"],
                              lambda e: tuple(oracle.bf16_to_f64(ex[k][e]) for k in ("gate", "up", "down")),
                              tuple(oracle.bf16_to_f64(d["shared_np"][k]) for k in ("gate", "up", "down")),
                              n_group=s.G, topk_group=s.TG, top_k=s.K)
    bits = (np.round(ref.astype(np.float32).view(np.uint32) / 65536.0)).astype(np.uint32).astype(np.uint16)
    ok = bench.output_check(s, d, ex, bits)
    assert ok["rows"] == 16 and ok["bar"] == 2e-2 and ok["max_abs_err_over_rms"] < 2e-2
    rms = float(np.sqrt(np.mean(ref ** 2)))
    bad = ref.copy()
    bad[3, 7] += 0.1 * rms
    bad_bits = (np.round(bad.astype(np.float32).view(np.uint32) / 65536.0)).astype(np.uint32).astype(np.uint16)
    assert abs(bench.output_check(s, d, ex, bad_bits)["max_abs_err_over_rms"] - 0.1) < 0.02
