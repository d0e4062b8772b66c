"""GPU parity on seeded random layouts: random head count, head dim, query-block and
partition splits (empty partitions included, ragged tiles everywhere), random local
partitions and recompute masks.  Each case runs an anchor step (every pair recomputed, with
the importance) and then a selective step with the local change, through the library's one
call (on a step that reuses states the reused states are merged inside the attention
launch), and checks out / lse, the importance and the local change against the oracle."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
import _parity as PT

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


def _random_layout(seed):
    rng = np.random.default_rng(5000 + seed)
    D = int(rng.choice([64, 128]))
    H = int(rng.integers(1, 5))
    S_q = int(rng.integers(1, 600))
    S_kv = S_q + int(rng.integers(0, 500))    # the query rows are the first S_q tokens
    n_qb = int(rng.integers(1, min(8, S_q) + 1))
    cuts = sorted(rng.choice(np.arange(1, S_q), size=n_qb - 1, replace=False).tolist()) if n_qb > 1 else []
    qo = [0] + [int(c) for c in cuts] + [S_q]
    P = int(rng.integers(1, 12))
    kcuts = sorted(rng.integers(0, S_kv + 1, size=P - 1).tolist())   # repeats give empty partitions
    ko = [0] + [int(c) for c in kcuts] + [S_kv]
    nonempty = [p for p in range(P) if ko[p + 1] > ko[p]]
    local = [int(rng.choice(nonempty)) for _ in range(n_qb)]
    mask = (rng.random((n_qb, P)) < rng.uniform(0.2, 0.8)).astype(np.uint8)
    mask[np.arange(n_qb), local] = 1
    w = W.Workload(name=f"random{seed}", H=H, D=D, grid=(S_kv,), P=P, q_token_range=(0, S_q), q_offsets=qo,
                   local_part=local, group_offsets=[0, P], recompute_groups=1, mode="distance", seed=5000 + seed,
                   prev_scale=0.05)
    return w, qo, ko, local, mask


@pytest.mark.parametrize("seed", range(16))
def test_random_layout_anchor_then_selective_step(seed):
    w, qo, ko, local, mask = _random_layout(seed)
    _log(f"seed {seed}: D={w.D} H={w.H} S_q={qo[-1]} S_kv={ko[-1]} q_offsets={qo} kv_offsets={ko} "
         f"local={local} reused={int(mask.size - mask.sum())}")
    rows = np.arange(qo[-1])
    Xp, X = W.make_step(w, -1), W.make_step(w, 0)
    g = PT.GpuRun(w, q_offsets=qo, kv_offsets=ko, local_part=local)
    o = PT.OracleRun(w, rows, q_offsets=qo, kv_offsets=ko, local_part=local)
    ones = np.ones_like(mask)
    # anchor step: no local change yet (the local slots hold nothing), the importance
    assert not g.step(Xp, ones, want_importance=True, want_delta=True)
    res0 = o.step(Xp, ones)
    cmp0 = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res0)
    assert cmp0.ok(), "anchor step: " + str(cmp0)
    imp = g.sa.importance[0].cpu().numpy()
    assert np.abs(imp - oracle.importance(res0.weights, rows, qo)).max() <= PT.IMP_ABS_TOL
    old = o.local_states()
    # selective step with the local change
    assert g.step(X, mask, want_delta=True)
    res = o.step(X, mask)
    cmp = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res)
    _log(f"seed {seed}", cmp)
    assert cmp.ok(), str(cmp)
    d_ref = oracle.local_change(o.local_states(), old, rows, qo)
    assert np.allclose(g.sa.delta[0].cpu().numpy(), d_ref, rtol=PT.DELTA_REL_TOL)


@pytest.mark.parametrize("seed", range(16, 24))
def test_random_layout_fp8_cache(seed):
    """The same kind of random layout with the compressed (e4m3) cache: decoded states, the
    merge of the kernel's own codes and the selective step within the e4m3 bounds of the
    oracle's exact states (the checks of the compressed-cache tests)."""
    from test_gpu_fp8 import run_fp8
    w, qo, ko, local, mask = _random_layout(seed)
    _log(f"seed {seed}: D={w.D} H={w.H} S_q={qo[-1]} S_kv={ko[-1]} q_offsets={qo} kv_offsets={ko} "
         f"local={local} reused={int(mask.size - mask.sum())}")
    run_fp8(w, np.arange(qo[-1]), layout=(qo, ko, local, mask))
