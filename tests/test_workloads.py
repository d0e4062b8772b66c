"""CPU checks of the seeded input generators (input preparation only)."""
import numpy as np

import workloads as W


def test_trajectory_matches_per_step_generation():
    w = W.workload("longvideo", grid=(3, 6, 8), H=2)
    for t, X in W.trajectory(w):
        Y = W.make_step(w, t)
        assert np.array_equal(X.q, Y.q) and np.array_equal(X.k, Y.k) and np.array_equal(X.v, Y.v), t


def test_prev_step_is_a_perturbation():
    w = W.workload("tiny")
    X, Xp = W.make_step(w, 0), W.make_step(w, -1)
    d = np.abs(W.to_f64(X.v) - W.to_f64(Xp.v))
    assert 0.01 < d.mean() < 0.08   # 0.05 * E|N(0,1)| ~ 0.04


def test_sampled_query_rows_match_full_generation():
    w = W.workload("video720p", grid=(3, 9, 16), H=2)
    full = W.make_step(w, 0).q
    rows = W.sample_rows(w, tiles_per_block=2, tile=8)
    assert np.array_equal(W.q_rows(w, 0, rows), full[:, rows])
