"""The selective step captured in a HIP graph (torch.cuda.CUDAGraph on the library's stream
argument) and replayed: every replay, with eager work and synchronisation between replays,
reproduces the eager step bitwise.  The library enqueues kernels only (no memset nodes, no
allocation, no synchronisation), so a step can be captured once and replayed per layer."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import workloads as W
import _parity as PT
from partitioned_state_reuse_amd import api

pytestmark = pytest.mark.gpu


def _outputs(sa):
    return sa.out.clone(), sa.lse.clone(), sa.delta.clone()


def _same(a, b):
    return all(torch.equal(x.view(torch.int16) if x.dtype == torch.bfloat16 else x,
                           y.view(torch.int16) if y.dtype == torch.bfloat16 else y) for x, y in zip(a, b))


@pytest.mark.parametrize("premerged", [False, True])
def test_step_replayed_from_a_graph_matches_eager(premerged):
    w = W.workload("video720p", grid=(5, 18, 32), H=4)
    mask = np.asarray(PT.masks_from_planners(w)[0], np.uint8)
    ones = np.ones((w.n_qb, w.P), np.uint8)
    Xp, X = W.make_step(w, -1), W.make_step(w, 0)
    sa = api.SelectiveAttention(1, w.S_q, w.S_kv, w.H, w.D, w.q_offsets, w.kv_offsets, w.local_part)
    sa.step(PT.to_dev(Xp.q), PT.to_dev(Xp.k), PT.to_dev(Xp.v), ones)
    q, k, v = PT.to_dev(X.q), PT.to_dev(X.k), PT.to_dev(X.v)

    def step():
        if premerged:
            sa.step_premerged(q, k, v, mask, want_delta=True)
        else:
            sa.step(q, k, v, mask, want_delta=True)

    # eager reference: the second of two identical steps (the local slot then already holds
    # the new state, as it does for every replay)
    step()
    step()
    torch.cuda.synchronize()
    ref = _outputs(sa)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for i in range(3):
        # eager work between replays: clobber the outputs, then replay
        sa.out.fill_(7.0)
        sa.lse.fill_(-3.0)
        sa.delta.fill_(5.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert _same(_outputs(sa), ref), f"replay {i}"
