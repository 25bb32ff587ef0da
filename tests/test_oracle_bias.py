"""Pins of the oracle's expert-bias update (routing walk-through page, section 三.3, with the
sign rule read from it): hand-worked cases and properties that hold for any input."""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bias_update_hand_cases.json")


def _cases():
    with open(GOLDEN) as fh:
        return json.load(fh)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_hand_cases(case):
    got = oracle.update_expert_bias(np.array(case["bias"], np.float32), np.array(case["counts"]), case["gamma"])
    assert got.dtype == np.float32
    np.testing.assert_array_equal(got, np.array(case["expected"], np.float32))


def test_properties_on_random_loads():
    rng = np.random.default_rng(3)
    for E in (8, 64, 512):
        counts = rng.poisson(8.0, size=E)
        bias = rng.uniform(-0.1, 0.1, size=E).astype(np.float32)
        gamma = 1e-3
        new = oracle.update_expert_bias(bias, counts, gamma)
        moved = new.astype(np.float64) - bias.astype(np.float64)
        mean = counts.sum() / E
        # direction: busy experts go down, idle ones up, experts at the mean stay
        assert np.all(moved[counts > mean] < 0)
        assert np.all(moved[counts < mean] > 0)
        assert np.all(moved[counts == mean] == 0)
        # size: one step of gamma, up to the fp32 rounding of the sum
        assert np.allclose(np.abs(moved[counts != mean]), gamma, rtol=0, atol=np.spacing(np.float32(0.2)))
        # the order of busyness is respected: the busiest expert never ends above where it
        # started, the idlest never below
        assert moved[np.argmax(counts)] <= 0 and moved[np.argmin(counts)] >= 0


def test_repeated_steps_pull_a_hot_expert_out_of_the_selection():
    # the bias is added to the selection score: after enough steps against an expert that
    # always wins, a rival with a slightly lower score overtakes it (the balancing effect the
    # page describes).  Two experts, one group, top-1.
    logits = np.array([[2.0, 1.9]])
    bias = np.zeros(2, np.float32)
    picks = []
    for _ in range(40):
        r = oracle.route(logits, bias, n_group=1, topk_group=1, top_k=1)
        e = int(r.topk_idx[0, 0])
        picks.append(e)
        counts = np.bincount([e], minlength=2)
        bias = oracle.update_expert_bias(bias, counts, 0.002)
    assert picks[0] == 0 and 1 in picks
