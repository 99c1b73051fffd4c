"""Pins for the oracle's expert-major dispatch (CPU only).

* A dispatch worked by hand (tests/golden/route_plan_small.json).
* The tiny workload: dispatching its 512 tokens by their top-2 choices must give
  exactly the padded matrix that the workload generator lays out by a separate
  construction (per expert, the tokens that chose it, in token order).
* Against a library routine: the non-pad rows, read in order, are numpy's stable
  argsort of the expert ids.
* Invariants on random routings: counts are the histogram, segments are aligned,
  row_assign and assign_row are inverse maps, pads map to -1.
* The error readings: an out-of-range expert id is dropped with status 2; a layout
  larger than the capacity is cut at the capacity with status 3.
"""
import json
import os

import numpy as np
import pytest

import workloads
from oracle import dispatch

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "route_plan_small.json")


def test_hand_worked_dispatch():
    g = json.load(open(GOLDEN))
    p = dispatch.route_plan(np.array(g["expert_idx"]), g["E"], g["pad_multiple"], g["m_capacity"])
    assert p["offs"].tolist() == g["offs"]
    assert p["counts"].tolist() == g["counts"]
    assert p["row_assign"].tolist() == g["row_assign"]
    assert p["assign_row"].tolist() == g["assign_row"]
    assert p["status"] == 0
    x = np.arange(5)[:, None] * 10 + np.arange(3)[None, :] + 1      # token t -> [10t+1, 10t+2, 10t+3]
    out = dispatch.permute(x, p["row_assign"], 2, 12)
    want = np.array([(10 * t + np.arange(3) + 1) if t >= 0 else np.zeros(3, dtype=int)
                     for t in g["token_of_row"]])
    assert np.array_equal(out, want)


def test_tiny_workload_layout_is_the_dispatch_of_its_tokens():
    tok, idx = workloads.routed_tokens("tiny")
    prob = workloads.mlp_problem("tiny")
    p = dispatch.route_plan(idx, prob["E"], prob["pad"], prob["m_capacity"])
    assert p["counts"].tolist() == prob["counts"]
    assert p["offs"].tolist() == prob["offs"]
    x = dispatch.permute(workloads.bf16_bits(tok), p["row_assign"], idx.shape[1], prob["m_capacity"])
    assert np.array_equal(x, workloads.bf16_bits(prob["x"]))


@pytest.mark.parametrize("seed,n,E,pad", [(0, 1000, 7, 128), (1, 5000, 16, 256), (2, 37, 64, 128), (3, 0, 4, 128)])
def test_plan_invariants_and_stable_order(seed, n, E, pad):
    rng = np.random.default_rng(seed)
    ids = rng.integers(0, E, size=n)
    ids[rng.random(n) < 0.3] = 0             # a skewed expert
    if E > 3:
        ids[ids == 3] = 2                   # an empty expert
    p = dispatch.route_plan(ids, E, pad, 1 << 20)
    offs, counts, ra, ar = p["offs"], p["counts"], p["row_assign"], p["assign_row"]
    assert p["status"] == 0
    assert np.array_equal(counts, np.bincount(ids, minlength=E))
    assert offs[0] == 0 and np.all(offs % pad == 0)
    assert np.array_equal(np.diff(offs), -(-counts // pad) * pad)
    assert len(ra) == offs[-1]
    real = ra >= 0
    assert np.array_equal(ra[real], np.argsort(ids, kind="stable"))
    assert np.array_equal(ar[ra[real]], np.nonzero(real)[0])
    for e in range(E):
        seg = ra[offs[e]:offs[e + 1]]
        assert np.all(seg[:counts[e]] >= 0) and np.all(seg[counts[e]:] == -1)
        assert np.all(ids[seg[:counts[e]]] == e)


def test_bad_expert_id_is_dropped_with_status():
    ids = np.array([[0, 5], [1, -1], [1, 0]])
    p = dispatch.route_plan(ids, 2, 128, 1024)
    assert p["status"] == dispatch.STATUS_BAD_EXPERT
    assert p["counts"].tolist() == [2, 2]
    assert p["assign_row"].tolist() == [0, -1, 128, -1, 129, 1]


def test_capacity_overflow_cuts_rows_with_status():
    ids = np.array([0] * 130 + [1] * 5)
    p = dispatch.route_plan(ids, 2, 128, 256)
    assert p["status"] == dispatch.STATUS_OVERFLOW
    assert p["offs"].tolist() == [0, 256, 384]
    assert len(p["row_assign"]) == 256
    assert np.all(p["assign_row"][130:] == -1) and p["assign_row"][129] == 129
