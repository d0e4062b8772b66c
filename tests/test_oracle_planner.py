"""Pins of the reference group planner (oracle/planner.py).

The DiTango pages (gist.science 2607.15650, "Methodology §1, Anchor-Guided Selection
Planner") fix: anchor steps recompute every partition; decisions are made per group of
spatially adjacent partitions; high-contribution groups are recomputed and the rest
reused.  The pins below:

* brute force over every subset of the non-local groups: the planner's choice maximises
  the summed predicted error e over the recomputed groups,
* uniform importance and constant delta reduce to an oldest-first round robin whose
  pattern is derived by hand,
* the distance rule's selections for the 720p layout (16 query blocks, 8 groups of two
  partitions, 4 recomputed) and for the 32-way share (9 of 32 singleton groups), derived
  by hand from the rule,
* the anchor schedule.
"""
import itertools
import os

import numpy as np
import pytest

from oracle import RefPlanner, group_distance
import workloads as W


def test_bruteforce_top_groups_maximise_error():
    rng = np.random.default_rng(0)
    for trial in range(60):
        G = int(rng.integers(2, 9))
        K = int(rng.integers(1, G + 1))
        local = int(rng.integers(0, G))
        pl = RefPlanner(1, G, list(range(G + 1)), [local], anchor_every=100, recompute_groups=K, mode="wdelta")
        m0, _ = pl.next(0)
        assert m0.all()
        imp = rng.random((1, G)).astype(np.float32)
        pl.observe(0, importance=imp)
        mask, chosen = pl.next(1)
        assert chosen[0][0] == local
        others = [g for g in range(G) if g != local]
        e = {g: float(imp[0, g]) for g in others}   # staleness 1, dhat 1.0 at t=1
        best = max(itertools.combinations(others, K - 1), key=lambda c: sum(e[g] for g in c))
        assert sorted(chosen[0][1:]) == sorted(best)
        assert mask[0].sum() == K
        assert all(mask[0, g] == (g == local or g in best) for g in range(G))


def test_ties_go_to_distance_then_index():
    # all importance equal: the K-1 nearest groups win, lower index on equal distance
    G, K, local = 7, 4, 3
    pl = RefPlanner(1, G, list(range(G + 1)), [local], 100, K, "wdelta")
    pl.next(0)
    pl.observe(0, importance=np.full((1, G), 0.25, np.float32))
    _, chosen = pl.next(1)
    assert chosen[0] == [3, 2, 4, 1]


def test_round_robin_closed_form():
    """Uniform w and constant delta: e_ig = w d (t - last_ig), so the oldest groups win;
    equal age goes to the nearest.  Local = partition 0 of 5 singleton groups, K = 3:
    t=1 refreshes {1, 2} (all aged 1, nearest first), t=2 {3, 4} (aged 2), t=3 {1, 2}, ..."""
    pl = RefPlanner(1, 5, list(range(6)), [0], 100, 3, "wdelta")
    pl.next(0)
    pl.observe(0, importance=np.full((1, 5), 0.2, np.float32))
    seq = []
    for t in range(1, 7):
        _, ch = pl.next(t)
        seq.append(ch[0])
        pl.observe(t, delta=np.array([0.03], np.float32))
    assert seq == [[0, 1, 2], [0, 3, 4], [0, 1, 2], [0, 3, 4], [0, 1, 2], [0, 3, 4]]


def test_anchor_schedule_every_five():
    pl = RefPlanner(2, 8, [0, 4, 8], [0, 5], 5, 1, "wdelta")
    for t in range(10):
        m, _ = pl.next(t)
        pl.observe(t, importance=np.full((2, 8), 0.125, np.float32) if t % 5 == 0 else None,
                   delta=np.array([0.1, 0.2], np.float32) if t > 0 else None)
        if t % 5 == 0:
            assert m.all()
        else:
            assert m.sum() == 8 and m[0, :4].all() and m[1, 4:].all()


def test_delta_prediction_uses_latest_observation():
    # block's local group 0; groups 1 and 2 last refreshed at different steps
    pl = RefPlanner(1, 3, [0, 1, 2, 3], [0], 100, 2, "wdelta")
    pl.next(0)
    pl.observe(0, importance=np.array([[0.5, 0.3, 0.2]], np.float32))
    _, c1 = pl.next(1)                       # e = w: group 1 (0.3) beats 2 (0.2)
    assert c1[0] == [0, 1]
    pl.observe(1, delta=np.array([0.5], np.float32))
    # t=2: e_1 = 0.3 * dhat(2) = 0.3*0.5; e_2 = 0.2 * (dhat(1) + dhat(2)) = 0.2*(0.5+0.5)
    e = pl.scores(2)[0]
    assert e[1] == float(np.float32(0.3)) * 0.5
    assert e[2] == float(np.float32(0.2)) * (0.5 + 0.5)
    _, c2 = pl.next(2)
    assert c2[0] == [0, 2]


GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def load_selection(name):
    """query block -> set of recomputed groups, from a hand-derived golden fixture."""
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            i, gs = line.split(":")
            out[int(i)] = {int(x) for x in gs.split()}
    return out


VIDEO720P_GROUPS = load_selection("video720p_distance_selection.txt")


def test_distance_rule_video720p():
    w = W.workload("video720p")
    pl = RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, 0, w.recompute_groups, "distance")
    mask, chosen = pl.next(0)
    for i in range(16):
        assert set(chosen[i]) == VIDEO720P_GROUPS[i], i
        assert chosen[i][0] == i // 2
        assert mask[i].sum() == 8
        assert mask[i, i] == 1


def test_distance_rule_share32():
    w = W.workload("share32")
    pl = RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, 0, w.recompute_groups, "distance")
    mask, chosen = pl.next(0)
    assert w.recompute_groups == 9
    assert chosen[0] == list(range(9))
    assert mask[0].tolist() == [1] * 9 + [0] * 23


def test_tiny_mask():
    w = W.workload("tiny")
    pl = RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, 0, w.recompute_groups, "distance")
    mask, _ = pl.next(0)
    assert mask.tolist() == [[1, 1, 0, 0]]


def test_group_distance():
    assert group_distance([0, 2, 4, 6], 2, 1) == 3
    assert group_distance([0, 2, 4, 6], 0, 1) == 0
