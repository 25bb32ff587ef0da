"""moe_forward_noalloc (the forward on the library's static device scratch, for callers that
cannot allocate) against moe_forward with a caller workspace: two calls in a row, the second
with fewer tokens, every output bit for bit; and the host-side rejection of a T whose
workspace does not fit in the scratch."""
import sys

import numpy as np
import pytest

from synthetic import CONFIGS

from moe_case import DeviceCase, host_case

pytestmark = pytest.mark.gpu


def _run(dev, noalloc, T):
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    s = dev.c.shape
    out = torch.full((T, s.H), 7.0, dtype=torch.bfloat16, device="cuda")
    idx = torch.full((T, s.K), -5, dtype=torch.int32, device="cuda")
    w = torch.full((T, s.K), -1.0, dtype=torch.float32, device="cuda")
    cnt = torch.full((s.E + 1,), -9, dtype=torch.int32, device="cuda")
    x = dev.x[:T]
    if noalloc:
        moe.moe_forward_noalloc(dev.cfg, T, x, dev.router_w, dev.bias, dev.weights, out, idx, w, cnt)
    else:
        moe.moe_forward(dev.cfg, T, x, dev.router_w, dev.bias, dev.weights, out, idx, w, cnt, dev.ws)
    torch.cuda.synchronize()
    return [t.view(torch.int16) if t.dtype == torch.bfloat16 else t for t in (out, idx, w, cnt)]


# decode 900 -> 500: the full-size layer near the scratch's limit, on the 256-position tile
# kernels (14 tokens per expert), then on the same scratch with fewer tokens
@pytest.mark.parametrize("name,T0,T1", [("tiny", 300, 40), ("decode", 256, 64), ("decode", 900, 500)])
def test_noalloc_matches_forward_twice(name, T0, T1):
    import torch
    c = host_case(CONFIGS[name], seed=31, T=T0)
    dev = DeviceCase(c)
    for T in (T0, T1):  # the second call with fewer tokens, on the scratch the first one left
        print(f"[gpu] moe_forward_noalloc {name} T={T}", flush=True)
        sys.stdout.flush()
        ref = _run(dev, False, T)
        got = _run(dev, True, T)
        for a, b in zip(ref, got):
            assert torch.equal(a, b)


def test_noalloc_rejects_T_beyond_the_scratch():
    import torch
    import sparse_moe_layer_bailingmoev3_amd as moe
    c = host_case(CONFIGS["decode"].with_(num_experts=64, n_group=8), seed=32, T=8)
    dev = DeviceCase(c)
    T = 4096  # about 0.5 GB of workspace for the full hidden size: rejected on the host
    x = torch.zeros((T, c.shape.H), dtype=torch.bfloat16, device="cuda")
    out = torch.empty_like(x)
    with pytest.raises(moe.MoEError) as ei:
        moe.moe_forward_noalloc(dev.cfg, T, x, dev.router_w, dev.bias, dev.weights, out)
    assert ei.value.status == -4 and "scratch" in str(ei.value)
