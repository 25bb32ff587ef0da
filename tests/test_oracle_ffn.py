"""Pins for the oracle's expert FFN, combine and dispatch (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import (bf16_to_f64, dispatch, expert_forward, moe_layer, route, router_logits,
                    swiglu)
from synthetic import CONFIGS, gen_layer

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_silu_closed_form():
    # silu(0) = 0; silu(1) = 1/(1+1/e); silu(-1) = -1/(1+e); SwiGLU multiplies by up
    g = np.array([0.0, 1.0, -1.0, 40.0])
    u = np.array([5.0, 2.0, 3.0, 0.5])
    want = np.array([0.0, 2.0 / (1 + np.exp(-1.0)), -3.0 / (1 + np.e), 20.0])
    np.testing.assert_allclose(swiglu(g, u), want, rtol=1e-15)


def test_swiglu_gate_and_up_are_not_interchangeable():
    # silu(g) * u != silu(u) * g: catches swapped gate/up
    assert not np.isclose(swiglu(np.array([2.0]), np.array([-1.0]))[0],
                          swiglu(np.array([-1.0]), np.array([2.0]))[0])


def test_clamp():
    rng = np.random.default_rng(0)
    g, u = rng.standard_normal(1000) * 6, rng.standard_normal(1000) * 6
    a = swiglu(g, u)
    a4 = swiglu(g, u, 4.0)
    assert np.abs(a4).max() <= 4.0
    inside = np.abs(a) < 4.0
    np.testing.assert_array_equal(a4[inside], a[inside])
    np.testing.assert_array_equal(np.sign(a4[~inside]) * 4.0, a4[~inside])
    np.testing.assert_array_equal(swiglu(g, u, np.inf), a)   # infinite limit == off
    np.testing.assert_array_equal(swiglu(g, u, 0.0), a)      # limit <= 0 == off


def test_expert_forward_structured():
    # x = e_h picks column h of gate/up; the output is down @ a for that single a
    H, I = 6, 4
    rng = np.random.default_rng(1)
    gate, up, down = rng.standard_normal((I, H)), rng.standard_normal((I, H)), rng.standard_normal((H, I))
    x = np.eye(H)[[2]]
    a = gate[:, 2] / (1 + np.exp(-gate[:, 2])) * up[:, 2]
    np.testing.assert_allclose(expert_forward(x, gate, up, down)[0],
                               [sum(down[h, i] * a[i] for i in range(I)) for h in range(H)], rtol=1e-13)


def _tiny_layer(shape, seed=0):
    d = gen_layer(shape, seed)
    x = bf16_to_f64(d["x"])
    ex = {k: bf16_to_f64(d["experts"][k]) for k in ("gate", "up", "down")}
    sh = tuple(bf16_to_f64(d["shared"][k]) for k in ("gate", "up", "down"))
    return d, x, ex, sh


def _dense_reference(x, Wr, b, ex, sh, shape, limit=0.0, slimit=0.0):
    """Every expert on every token; the routing weights (zero off the chosen set) mask
    the sum.  Shares only `route` with the sparse path."""
    r = route(router_logits(x, Wr), b, shape.G, shape.TG, shape.K, shape.routed_scaling_factor,
              shape.norm_topk_prob)
    T = x.shape[0]
    W = np.zeros((T, shape.E))
    np.put_along_axis(W, r.topk_idx, r.topk_w, axis=1)
    out = np.zeros_like(x)
    for e in range(shape.E):
        g = x @ ex["gate"][e].T
        u = x @ ex["up"][e].T
        a = g / (1 + np.exp(-g)) * u
        if limit > 0:
            a = np.minimum(np.maximum(a, -limit), limit)
        out += W[:, e:e + 1] * (a @ ex["down"][e].T)
    g, u = x @ sh[0].T, x @ sh[1].T
    a = g / (1 + np.exp(-g)) * u
    if slimit > 0:
        a = np.minimum(np.maximum(a, -slimit), slimit)
    return out + a @ sh[2].T


@pytest.mark.parametrize("limits", [(0.0, 0.0), (0.01, 0.02)])
def test_sparse_equals_dense_reference(limits):
    shape = CONFIGS["tiny"]
    d, x, ex, sh = _tiny_layer(shape)
    out, r = moe_layer(x, d["router_w"], d["bias"], lambda e: (ex["gate"][e], ex["up"][e], ex["down"][e]),
                       sh, n_group=8, topk_group=4, top_k=8, swiglu_limit=limits[0],
                       shared_swiglu_limit=limits[1])
    ref = _dense_reference(x, d["router_w"], d["bias"], ex, sh, shape, *limits)
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12 * np.abs(ref).max())


def test_identical_experts_invariant():
    # all routed experts identical -> routing cannot matter: out = 2.5 * FFN(x) + shared(x)
    shape = CONFIGS["tiny"]
    d, x, ex, sh = _tiny_layer(shape, seed=3)
    one = (ex["gate"][5], ex["up"][5], ex["down"][5])
    out, _ = moe_layer(x, d["router_w"], d["bias"], lambda e: one, sh, n_group=8, topk_group=4, top_k=8)
    want = 2.5 * expert_forward(x, *one) + expert_forward(x, *sh)
    np.testing.assert_allclose(out, want, rtol=1e-10, atol=1e-13)


def test_zero_shared_and_no_shared():
    shape = CONFIGS["tiny"]
    d, x, ex, sh = _tiny_layer(shape, seed=4)
    get = lambda e: (ex["gate"][e], ex["up"][e], ex["down"][e])
    out_none, _ = moe_layer(x, d["router_w"], d["bias"], get, None, n_group=8, topk_group=4, top_k=8)
    zero = tuple(np.zeros_like(a) for a in sh)
    out_zero, _ = moe_layer(x, d["router_w"], d["bias"], get, zero, n_group=8, topk_group=4, top_k=8)
    np.testing.assert_array_equal(out_none, out_zero)


def test_dispatch_definitions():
    rng = np.random.default_rng(2)
    T, K, E = 37, 4, 10
    idx = np.sort(np.array([rng.choice(E, K, replace=False) for _ in range(T)]), axis=1)
    d = dispatch(idx, E, 1)
    assert d.counts[:E].tolist() == [int((idx == e).sum()) for e in range(E)] and d.counts[E] == T
    assert d.offsets[0] == 0 and np.all(np.diff(d.offsets) == d.counts)
    for e in range(E):
        toks = d.sorted_token[d.offsets[e]:d.offsets[e + 1]]
        assert toks.tolist() == [t for t in range(T) if e in idx[t]]     # ascending tokens
    assert d.sorted_token[d.offsets[E]:].tolist() == list(range(T))
    for t in range(T):
        for k in range(K):
            p = d.inv_perm[t, k]
            assert d.sorted_token[p] == t and d.offsets[idx[t, k]] <= p < d.offsets[idx[t, k] + 1]


def test_dispatch_ignores_out_of_range_ids():
    """Ids outside [0, E) are dropped (the library's contract for such input): they are in no
    count, their inv_perm is -1, the valid pairs keep their places in expert-then-token order,
    the gap they leave holds -1 at the end of the routed range, and the shared expert's block
    still starts at T*K.  Checked against a walk over the pairs written out by hand."""
    rng = np.random.default_rng(3)
    T, K, E = 29, 5, 12
    idx = np.array([rng.choice(E, K, replace=False) for _ in range(T)])
    drop = rng.random((T, K)) < 0.2
    idx[drop] = rng.choice([-1, -7, E, E + 3], size=int(drop.sum()))
    d = dispatch(idx, E, 1)
    valid = (idx >= 0) & (idx < E)
    pos = 0
    for e in range(E):
        assert d.offsets[e] == pos
        for t in range(T):
            for k in range(K):
                if valid[t, k] and idx[t, k] == e:
                    assert d.sorted_token[pos] == t and d.inv_perm[t, k] == pos
                    pos += 1
        assert d.counts[e] == pos - d.offsets[e]
    assert pos == valid.sum() < T * K
    assert np.all(d.sorted_token[pos:T * K] == -1)
    assert d.offsets[E] == T * K and d.offsets[E + 1] == T * K + T and d.counts[E] == T
    assert d.sorted_token[T * K:].tolist() == list(range(T))
    assert np.all(d.inv_perm[~valid] == -1)


def test_layer_constants_match_pages():
    with open(os.path.join(GOLDEN, "layer_constants.json")) as f:
        c = json.load(f)
    s = CONFIGS["decode"]
    assert (s.H, s.E, s.I, s.G, s.TG, s.K) == (c["hidden_size"], c["num_experts"], c["moe_intermediate_size"],
                                              c["n_group"], c["topk_group"], c["num_experts_per_tok"])
    assert s.routed_scaling_factor == c["routed_scaling_factor"] and s.norm_topk_prob == c["norm_topk_prob"]
    assert s.E // s.G == c["experts_per_group"] and s.TG * s.E // s.G == c["candidates"]
    params = 3 * s.H * s.I
    assert params == 5_898_240 and round(params / 1e6, 2) == c["params_per_expert_approx_millions"]
    assert c["moe_layers"] * s.E * 3 == c["expert_tensors"]
    sk = CONFIGS["skewed"]
    assert sk.swiglu_limit == c["routed_swiglu_limit"] and sk.shared_swiglu_limit in c["shared_swiglu_limits"]
