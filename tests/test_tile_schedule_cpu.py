"""The work-item pipeline of the 256-position tile kernel, modelled on the CPU.

A workgroup of that kernel runs several work items back to back through one load pipeline:
the issue side loads step g + D while the compute side works on step g, so the issue side
moves to the next item one chunk of D steps before the compute side does, and hands it over
through a single pending-item slot.  This model follows the kernel's loop (prologue of D
steps, chunks of D steps, the compute side taking the pending item before the issue side
switches) and checks that every computed step is the one that was loaded for it.  The old
order (issue switch first) is kept as a second model to show what it got wrong: with items
of exactly D steps the pending item was replaced before the compute side took it.
"""
import itertools

import pytest


def run_pipeline(lengths, D, consume_first=True):
    """Returns (computed, issued): computed[g] = (item, step) the compute side works on at
    global step g; issued[g] = (item, step) whose data the issue side loaded for step g."""
    assert all(n % D == 0 and n > 0 for n in lengths)
    issued, computed = {}, []
    st = dict(iss=0, isn=0, live=True, nxt=None)

    def issue(g):
        issued[g] = (st["iss"], st["isn"])
        if st["live"]:
            st["isn"] += 1

    def switch_issue():
        if not st["live"] or st["isn"] < lengths[st["iss"]]:
            return
        if st["iss"] + 1 < len(lengths):
            st["iss"] += 1
            st["isn"] = 0
            st["nxt"] = st["iss"]
        else:
            st["live"] = False
            st["isn"] = lengths[st["iss"]] - 1

    for g in range(D):
        issue(g)
    switch_issue()
    cmp, csn, cmp_live, g0 = 0, 0, True, 0

    def consume():
        nonlocal cmp, csn, cmp_live
        if csn == lengths[cmp]:
            if st["nxt"] is not None:
                cmp, csn = st["nxt"], 0
                st["nxt"] = None
            else:
                cmp_live = False

    while cmp_live:
        for j in range(D):
            g = g0 + j
            computed.append((cmp, csn))
            issue(g + D)
            csn += 1
        if consume_first:
            consume()
            switch_issue()
        else:
            switch_issue()
            consume()
        g0 += D
        assert g0 < 10 * sum(lengths) + 10, "pipeline did not drain"
    return computed, issued


def pipeline_ok(lengths, D, consume_first=True):
    computed, issued = run_pipeline(lengths, D, consume_first)
    want = [(i, s) for i, n in enumerate(lengths) for s in range(n)]
    return computed == want and all(issued[g] == c for g, c in enumerate(computed))


@pytest.mark.parametrize("D", [2, 3])
def test_every_item_sequence_is_computed_in_order(D):
    # every sequence of up to five items of D .. 4D steps
    for n in range(1, 6):
        for lens in itertools.product([D, 2 * D, 3 * D, 4 * D], repeat=n):
            assert pipeline_ok(list(lens), D), lens


def test_issue_first_order_misattributes_short_items():
    # the sequences the earlier loop order got wrong, and ones it got right
    D = 2
    for bad in ([4, 2, 2], [2, 2, 4], [6, 2, 6], [2, 2, 2]):
        assert not pipeline_ok(bad, D, consume_first=False), bad
        assert pipeline_ok(bad, D), bad
    for fine in ([2, 2], [4, 4, 2]):
        assert pipeline_ok(fine, D, consume_first=False), fine
