"""Pins for the oracle's routing (CPU only).

The oracle sorts; these tests pin it against other formulations: hand-worked cases
(tests/golden/routing_hand_cases.json), brute-force enumeration of group and expert
subsets on tiny shapes, closed-form special cases and invariants at the real shape.
"""
import itertools
import json
import os

import numpy as np
import pytest

from oracle import route, router_logits, bf16_to_f64
from synthetic import CONFIGS, gen_bias, gen_router, gen_x

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _logit(s):
    s = np.asarray(s, np.float64)
    return np.log(s / (1.0 - s))


# ----------------------------------------------------------------------------------
# hand-worked cases from the page's rules
# ----------------------------------------------------------------------------------
with open(os.path.join(GOLDEN, "routing_hand_cases.json")) as f:
    HAND = json.load(f)["cases"]


@pytest.mark.parametrize("case", HAND, ids=[c["name"] for c in HAND])
@pytest.mark.parametrize("decision", ["fp32", "fp64"])
def test_hand_cases(case, decision):
    l = _logit(case["s"])[None, :]
    r = route(l, np.array(case["bias"], np.float64), case["G"], case["TG"], case["K"],
              case["scale"], case["norm"], decision=decision)
    assert r.topk_idx[0].tolist() == case["idx"]
    np.testing.assert_allclose(r.topk_w[0], case["w"], rtol=2e-6 if decision == "fp32" else 1e-12)


# ----------------------------------------------------------------------------------
# brute force on tiny shapes
# ----------------------------------------------------------------------------------
def _brute_force(c, s, G, TG, K, scale, norm):
    """Enumerate: the kept groups are the TG-subset with the largest sum of group maxima
    (first in lexicographic order among equal sums = lower indices on ties); the chosen
    experts are the K-subset of the kept groups' experts with the largest sum of c
    (same tie rule).  Sums of fp32-valued scores are exact in float64 here."""
    E = c.size
    per = E // G
    gmax = [max(c[g * per:(g + 1) * per]) for g in range(G)]
    best, kept = None, None
    for sub in itertools.combinations(range(G), TG):
        v = sum(gmax[g] for g in sub)
        if best is None or v > best:
            best, kept = v, sub
    cand = [e for g in kept for e in range(g * per, (g + 1) * per)]
    best, chosen = None, None
    for sub in itertools.combinations(sorted(cand), K):
        v = sum(c[e] for e in sub)
        if best is None or v > best:
            best, chosen = v, sub
    w = np.array([s[e] for e in chosen])
    if norm:
        w = w / w.sum()
    return list(chosen), w * scale


TINY_SHAPES = [(16, 4, 2, 3), (12, 3, 2, 4), (24, 6, 3, 5), (8, 1, 1, 3), (16, 4, 4, 16), (16, 4, 1, 4)]


@pytest.mark.parametrize("E,G,TG,K", TINY_SHAPES)
@pytest.mark.parametrize("bias_scale", [0.0, 0.1, 0.5, 3.0])
def test_brute_force_selection(E, G, TG, K, bias_scale):
    rng = np.random.default_rng(1000 + E * 7 + G + TG * 13 + K + int(bias_scale * 10))
    T = 60
    l = rng.standard_normal((T, E)) * 1.5
    b = rng.standard_normal(E) * bias_scale
    for norm in (True, False):
        r = route(l, b, G, TG, K, 2.5, norm, decision="fp32")
        for t in range(T):
            idx, w = _brute_force(r.choice[t], r.scores[t], G, TG, K, 2.5, norm)
            assert r.topk_idx[t].tolist() == idx, (t, r.choice[t])
            np.testing.assert_allclose(r.topk_w[t], w, rtol=1e-12)


def test_brute_force_with_exact_ties():
    # duplicated router rows give exactly equal scores; lower indices must win
    rng = np.random.default_rng(7)
    E, G, TG, K = 16, 4, 2, 3
    base = rng.standard_normal((40, 4))
    l = np.repeat(base, 4, axis=1)            # experts 4j..4j+3 share a logit
    for b in (np.zeros(E), np.repeat(rng.uniform(-0.1, 0.1, 4), 4)):
        r = route(l, b, G, TG, K, 2.5, True, decision="fp32")
        for t in range(l.shape[0]):
            idx, _ = _brute_force(r.choice[t], r.scores[t], G, TG, K, 2.5, True)
            assert r.topk_idx[t].tolist() == idx


# ----------------------------------------------------------------------------------
# closed forms and special cases
# ----------------------------------------------------------------------------------
def test_single_group_no_bias_is_plain_topk():
    # G = TG = 1 and no bias: the chosen set is the top-K of the logits (sigmoid is
    # monotone), which numpy's argsort gives directly
    rng = np.random.default_rng(3)
    l = rng.standard_normal((100, 64))
    r = route(l, None, 1, 1, 8, 2.5, True, decision="fp64")
    want = np.sort(np.argsort(-l, axis=1)[:, :8], axis=1)
    assert np.array_equal(r.topk_idx, want)


def test_logits_of_one_hot_rows_are_router_columns():
    rng = np.random.default_rng(4)
    W = rng.standard_normal((32, 16)).astype(np.float32)
    x = np.eye(16)[[3, 0, 15, 7]]
    np.testing.assert_array_equal(router_logits(x, W), W.astype(np.float64)[:, [3, 0, 15, 7]].T)


def test_logits_against_explicit_dot_products():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((3, 8))
    W = rng.standard_normal((5, 8))
    want = np.array([[sum(x[t, h] * W[e, h] for h in range(8)) for e in range(5)] for t in range(3)])
    np.testing.assert_allclose(router_logits(x, W), want, rtol=1e-13)


def test_sigmoid_values():
    # sigmoid(0) = 1/2, sigmoid(ln 3) = 3/4
    r = route(np.array([[0.0, np.log(3.0), -np.log(3.0), 0.0]]), None, 1, 1, 4, 1.0, False, "fp64")
    np.testing.assert_allclose(r.scores[0], [0.5, 0.75, 0.25, 0.5], rtol=1e-15)


def test_k1_weight_is_scaling_factor():
    rng = np.random.default_rng(6)
    r = route(rng.standard_normal((50, 64)), rng.uniform(-0.1, 0.1, 64), 8, 4, 1, 2.5, True)
    np.testing.assert_allclose(r.topk_w, 2.5, rtol=1e-15)


def test_all_experts_dense_weights():
    # K = E with one group: every expert is chosen, weights = 2.5 * s / sum(s)
    rng = np.random.default_rng(8)
    l = rng.standard_normal((10, 16))
    r = route(l, rng.standard_normal(16), 1, 1, 16, 2.5, True, "fp64")
    s = 1 / (1 + np.exp(-l))
    assert np.array_equal(r.topk_idx, np.tile(np.arange(16), (10, 1)))
    np.testing.assert_allclose(r.topk_w, 2.5 * s / s.sum(1, keepdims=True), rtol=1e-14)


# ----------------------------------------------------------------------------------
# invariants at the real shape
# ----------------------------------------------------------------------------------
@pytest.fixture(scope="module")
def real_routing():
    shp = CONFIGS["decode"]
    x = bf16_to_f64(gen_x(shp, T=256))
    l = router_logits(x, gen_router(shp))
    b = gen_bias(shp)
    return shp, l, b, route(l, b, shp.G, shp.TG, shp.K, 2.5, True)


def test_invariants_real_shape(real_routing):
    shp, l, b, r = real_routing
    T = l.shape[0]
    per = shp.E // shp.G
    assert r.topk_idx.shape == (T, 8)
    for t in range(T):
        idx = r.topk_idx[t]
        assert len(set(idx.tolist())) == 8 and np.all(np.diff(idx) > 0)
        groups = set((idx // per).tolist())
        assert groups <= set(r.kept_groups[t].tolist()) and len(groups) <= 4
        gmax = r.choice[t].reshape(shp.G, per).max(1)
        kept = r.kept_groups[t]
        dropped = np.setdiff1d(np.arange(shp.G), kept)
        assert gmax[kept].min() >= gmax[dropped].max()
        cand = np.concatenate([np.arange(g * per, (g + 1) * per) for g in kept])
        unsel = np.setdiff1d(cand, idx)
        assert r.choice[t][idx].min() >= r.choice[t][unsel].max()
    np.testing.assert_allclose(r.topk_w.sum(1), 2.5, rtol=1e-12)
    # weights are proportional to the unbiased score
    s_sel = np.take_along_axis(r.scores, r.topk_idx, 1)
    ratio = r.topk_w / s_sel
    np.testing.assert_allclose(ratio, np.repeat(ratio[:, :1], 8, axis=1), rtol=1e-12)
    assert r.counts.sum() == T * 8


def test_bias_shift_invariance(real_routing):
    shp, l, b, r = real_routing
    r2 = route(l, b + 0.25, shp.G, shp.TG, shp.K, 2.5, True, decision="fp64")
    r1 = route(l, b, shp.G, shp.TG, shp.K, 2.5, True, decision="fp64")
    assert np.array_equal(r1.topk_idx, r2.topk_idx)
    np.testing.assert_allclose(r1.topk_w, r2.topk_w, rtol=1e-14)


def test_bias_changes_selection_not_weight_formula(real_routing):
    shp, l, b, r = real_routing
    t = 0
    outsider = np.setdiff1d(np.arange(shp.E), r.topk_idx[t])[0]
    b2 = b.copy()
    b2[outsider] += 10.0               # forces it into every token's choice
    r2 = route(l, b2, shp.G, shp.TG, shp.K, 2.5, True)
    assert np.all((r2.topk_idx == outsider).any(1))
    s_sel = np.take_along_axis(r2.scores, r2.topk_idx, 1)
    np.testing.assert_allclose(r2.topk_w, 2.5 * s_sel / s_sel.sum(1, keepdims=True), rtol=1e-12)


def test_fp32_and_fp64_decisions_agree_off_ties(real_routing):
    shp, l, b, r32 = real_routing
    r64 = route(l, b, shp.G, shp.TG, shp.K, 2.5, True, decision="fp64")
    ok = ~(r32.near_tie | r64.near_tie)
    assert np.array_equal(r32.topk_idx[ok], r64.topk_idx[ok])
    np.testing.assert_allclose(r32.topk_w, r64.topk_w, rtol=1e-6)


def test_near_tie_gaps_are_reported():
    # two experts with identical scores across the K-th boundary: gap 0 -> near tie
    l = np.array([[2.0, 1.0, 1.0, -1.0]])
    r = route(l, None, 1, 1, 2, 2.5, True)
    assert r.gap_expert[0] == 0.0 and r.near_tie[0]
    assert r.topk_idx[0].tolist() == [0, 1]


# ----------------------------------------------------------------------------------
# the near-tie detector: hand-worked gaps and brute force
# ----------------------------------------------------------------------------------
with open(os.path.join(GOLDEN, "near_tie_hand_cases.json")) as f:
    TIES = json.load(f)


def _num(v):
    return float("inf") if v == "inf" else float(v)


@pytest.mark.parametrize("case", TIES["cases"], ids=[c["name"] for c in TIES["cases"]])
@pytest.mark.parametrize("decision", ["fp32", "fp64"])
def test_near_tie_hand_cases(case, decision):
    """Gaps at the group and expert boundaries and the near-tie flag, worked by hand (the scores
    are dyadic, so every value is exact): an off-by-one in either boundary, gaps taken on the
    unbiased score, or an expert gap taken over all experts instead of the kept groups' ones
    each change at least one expected value."""
    l = np.array(case["logits"], np.float64)[None, :]
    r = route(l, np.array(case["bias"], np.float64), case["G"], case["TG"], case["K"], 2.5, True,
              decision=decision, tie_eps=TIES["tie_eps"])
    assert r.kept_groups[0].tolist() == case["kept_groups"]
    assert r.topk_idx[0].tolist() == case["idx"]
    assert r.gap_group[0] == _num(case["gap_group"])
    assert r.gap_expert[0] == _num(case["gap_expert"])
    assert bool(r.near_tie[0]) == case["near_tie"]


def _brute_force_gaps(c, G, TG, K):
    """Gaps from their definition, by enumeration: the kept groups are the TG-subset with the
    largest sum of group maxima; gap_group = (TG-th largest group maximum) - ((TG+1)-th);
    gap_expert = (K-th largest biased score among the kept groups' experts) - ((K+1)-th)."""
    E = len(c)
    per = E // G
    gmax = [max(c[g * per:(g + 1) * per]) for g in range(G)]
    best, kept = None, None
    for sub in itertools.combinations(range(G), TG):
        v = sum(gmax[g] for g in sub)
        if best is None or v > best:
            best, kept = v, sub
    ranked = sorted(gmax, reverse=True)
    gap_g = ranked[TG - 1] - ranked[TG] if TG < G else float("inf")
    cand = sorted((c[e] for g in kept for e in range(g * per, (g + 1) * per)), reverse=True)
    gap_e = cand[K - 1] - cand[K] if K < len(cand) else float("inf")
    return gap_g, gap_e


@pytest.mark.parametrize("E,G,TG,K", TINY_SHAPES)
def test_brute_force_gaps(E, G, TG, K):
    # scores on a coarse grid, so that near and exact ties at both boundaries occur often
    rng = np.random.default_rng(2000 + E * 7 + G + TG * 13 + K)
    T = 80
    l = rng.integers(-4, 5, size=(T, E)) * 0.25
    b = rng.integers(-2, 3, size=E) * 2.0 ** -22
    r = route(l, b, G, TG, K, 2.5, True, decision="fp32")
    n_tie = 0
    for t in range(T):
        gg, ge = _brute_force_gaps(list(r.choice[t]), G, TG, K)
        assert r.gap_group[t] == gg and r.gap_expert[t] == ge, (t, r.choice[t])
        assert bool(r.near_tie[t]) == (min(gg, ge) < 1e-6)
        n_tie += bool(r.near_tie[t])
    if TG < G or K < TG * E // G:
        assert 0 < n_tie < T  # both outcomes exercised
