"""Oracle vs hand-worked examples (tests/golden/*.json).

Each fixture was derived by hand from the pages' definitions (maxvio, the
exact S*K-per-rank invariant, row-index addressing of one [E+B, ...] weight
tensor) and the oracle's stated readings; the derivation is written inside
the fixture.  These pin the planner's tie-breaks, the piece/receiver walk,
the token order inside an expert and the cu_seqlens layout.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _check_case(g, idx, B, case):
    E, R = g["E"], g["R"]
    pl = oracle.plan(idx, E, B)
    assert pl.status == case["status"]
    if "T" in case:
        assert pl.T.tolist() == case["T"]
    if "keep" in case:
        assert pl.keep.tolist() == case["keep"]
    got = [dict(expert=m.expert, rank=m.rank, start=m.start, count=m.count, slot=m.slot)
           for m in pl.replicas]
    assert got == case["replicas"]
    for k in ("n_donors", "n_receivers", "n_pieces", "max_needed", "n_relayed"):
        if k in case:
            assert getattr(pl, k) == case[k], k
    if "counts" in case:
        assert pl.counts.tolist() == case["counts"]
    for r in range(R):
        cu, dest, src = oracle.layout(idx, pl, r)
        assert cu.tolist() == case["cu_seqlens"][r]
        assert dest.tolist() == case["dest_pos"]
        assert src.tolist() == case["src_flat"][r]
        cu2, dest2, src2 = oracle.layout_loops(idx, pl, r)
        assert cu2.tolist() == cu.tolist() and dest2.tolist() == dest.tolist()
        assert src2.tolist() == src.tolist()
    if "blob" in case:
        assert pl.to_blob().tolist() == case["blob"]
    if "slot_expert" in case:
        se, ss, sc = pl.slot_table()
        assert se.ravel().tolist() == case["slot_expert"]
        assert ss.ravel().tolist() == case["slot_start"]
        assert sc.ravel().tolist() == case["slot_count"]


@pytest.mark.parametrize("name", ["plan_g1_single_donor.json", "plan_g2_split_piece.json",
                                  "plan_g4_bad_id.json"])
def test_golden_single(name):
    g = _load(name)
    idx = np.array(g["topk_idx"], np.int32)
    assert idx.shape == (g["R"], g["S"], g["K"])
    if "maxvio" in g:
        pl = oracle.plan(idx, g["E"], g["B"])
        assert oracle.maxvio(pl.T, g["R"], g["S"], g["K"], g["E"]) == pytest.approx(g["maxvio"])
    _check_case(g, idx, g["B"], g)


def test_golden_ties_and_overflow():
    g = _load("plan_g3_ties_overflow.json")
    idx = np.array(g["topk_idx"], np.int32)
    for case in g["cases"]:
        _check_case(g, idx, case["B"], case)
    pl = oracle.plan(idx, g["E"], 1)
    assert oracle.maxvio(pl.T, g["R"], g["S"], g["K"], g["E"]) == pytest.approx(g["maxvio"])


def test_maxvio_closed_forms():
    # perfectly balanced -> 0; everything on one expert -> E - 1
    assert oracle.maxvio([5, 5, 5, 5], R=2, S=5, K=2, E=4) == 0.0
    assert oracle.maxvio([20, 0, 0, 0], R=2, S=5, K=2, E=4) == pytest.approx(3.0)
    # one expert with twice the mean load -> 1
    assert oracle.maxvio([8, 4, 2, 2], R=1, S=8, K=2, E=4) == pytest.approx(1.0)
