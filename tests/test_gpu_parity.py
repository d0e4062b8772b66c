"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on the same seeded
inputs.  Workloads: the tiny and image-anchor configurations in full, the 720p, 32-way
share and long-video layouts on reduced grids (several query tiles, ragged KV tails),
the two 75,600-token configurations at full size on sampled query rows (same launch
configuration as the benchmark), and edge cases."""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
import _parity as PT
from partitioned_state_reuse_amd import api

pytestmark = pytest.mark.gpu


def _log(*a):
    print(*a, flush=True)


def run_single_step(w, rows=None, want_delta=True, want_importance=True):
    """Cache filled by an all-recompute step on X_prev, then the selective step on X."""
    m_cpp, m_ref, c_cpp, c_ref = PT.masks_from_planners(w)
    assert np.array_equal(m_cpp, m_ref) and c_cpp == c_ref
    mask = m_cpp
    full_rows = rows is None
    rows = np.arange(w.S_q) if rows is None else np.asarray(rows)
    ones = np.ones((w.n_qb, w.P), np.uint8)
    Xp = W.make_step(w, -1)
    X = W.make_step(w, 0)
    g = PT.GpuRun(w)
    g.step(Xp, ones)
    o = PT.OracleRun(w, rows)
    o.step(Xp, ones)
    old_local = o.local_states()
    did = g.step(X, mask, want_importance=want_importance, want_delta=want_delta)
    res = o.step(X, mask)
    cmp = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res)
    _log(w.name, "mask rows recomputed:", int(mask.sum()), cmp)
    assert cmp.ok(), str(cmp)
    # fresh states written into the cache slots (recomputed ones), and untouched reused ones
    blk = oracle.block_of_rows(rows, w.q_offsets)
    cl = g.cache_lse_rows(rows)
    co = g.cache_o_rows(rows)
    for p in range(w.P):
        sel = mask[blk, p].astype(bool)
        if sel.any():
            ref_l = o.cache.stored_lse[p][:, sel]
            fin = np.isfinite(ref_l)
            assert np.array_equal(np.isfinite(cl[p][:, sel]), fin)
            assert np.abs(np.where(fin, cl[p][:, sel] - ref_l, 0)).max() <= PT.LSE_ABS_TOL, p
            PT.assert_rows_close(co[p][sel], o.cache.stored_O[p][sel], f"cache slot plane {p}")
    if did and full_rows:
        d_gpu = g.sa.delta[0].cpu().numpy().astype(np.float64)
        d_ref = oracle.local_change(o.local_states(), old_local, rows, w.q_offsets)
        _log("delta gpu", d_gpu[:4], "oracle", d_ref[:4])
        assert np.allclose(d_gpu, d_ref, rtol=PT.DELTA_REL_TOL, atol=0)
    if want_importance and full_rows:
        w_gpu = g.sa.importance[0].cpu().numpy().astype(np.float64)
        w_ref = oracle.importance(res.weights, rows, w.q_offsets)
        _log("importance max|d|", np.abs(w_gpu - w_ref).max())
        assert np.abs(w_gpu - w_ref).max() <= PT.IMP_ABS_TOL
    return g, o, res


def test_tiny_full():
    w = W.workload("tiny")
    m, _, _, _ = PT.masks_from_planners(w)
    assert m.tolist() == [[1, 1, 0, 0]]
    run_single_step(w)


def test_image_anchor_full():
    w = W.workload("image_anchor")
    X = W.make_step(w, 0)
    mask = np.ones((w.n_qb, w.P), np.uint8)
    g = PT.GpuRun(w)
    g.step(X, mask, want_importance=True)
    rows = np.arange(w.S_q)
    o = PT.OracleRun(w, rows)
    res = o.step(X, mask)
    cmp = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res)
    _log(w.name, cmp)
    assert cmp.ok(), str(cmp)
    # every per-partition lse
    cl = g.cache_lse_rows(rows)
    assert np.abs(cl - o.cache.stored_lse).max() <= PT.LSE_ABS_TOL
    w_gpu = g.sa.importance[0].cpu().numpy().astype(np.float64)
    w_ref = oracle.importance(res.weights, rows, w.q_offsets)
    assert np.abs(w_gpu - w_ref).max() <= PT.IMP_ABS_TOL
    assert np.abs(w_gpu.sum(axis=1) - 1).max() < 1e-4


def test_video720p_reduced_grid():
    run_single_step(W.workload("video720p", grid=(5, 18, 32), H=4))


def test_share32_reduced_grid():
    run_single_step(W.workload("share32", grid=(9, 18, 32), H=4))


def test_video720p_full_size_sampled_rows():
    w = W.workload("video720p")
    rows = W.sample_rows(w, tiles_per_block=2, tile=16)
    run_single_step(w, rows=rows, want_delta=True, want_importance=False)


def test_share32_full_size_sampled_rows():
    w = W.workload("share32")
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(1000, 1016), np.arange(2330, 2363)]))
    run_single_step(w, rows=rows)


def test_longvideo_trajectory_reduced_grid():
    """10 denoising steps, anchor every 5, groups of 4, w*delta planner: per step the C++
    planner (fed by the GPU's importance and delta) and the oracle planner (fed by the
    oracle's) must select the same groups, and outputs must match."""
    w = W.workload("longvideo", grid=(9, 18, 32), H=2)
    rows = np.arange(w.S_q)
    g = PT.GpuRun(w)
    o = PT.OracleRun(w, rows)
    cp = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every, w.recompute_groups, "wdelta")
    rp = oracle.RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every, w.recompute_groups, "wdelta")
    shadow = oracle.RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every, w.recompute_groups, "wdelta")
    for t in range(w.steps):
        X = W.make_step(w, t)
        m_gpu, c_gpu = cp.next(t)
        m_ref, c_ref = rp.next(t)
        m_sh, c_sh = shadow.next(t)
        assert np.array_equal(m_sh, m_gpu) and c_sh == c_gpu, "C++ and oracle planner differ on identical inputs"
        if not (np.array_equal(m_gpu, m_ref) and c_gpu == c_ref):
            e = np.array(rp.scores(t))
            raise AssertionError(f"step {t}: gpu-fed selection {c_gpu} != oracle {c_ref}; scores {e}")
        anchor = t % w.anchor_every == 0
        old_local = o.local_states() if t > 0 else None
        did = g.step(X, m_gpu, want_importance=anchor, want_delta=t > 0)
        res = o.step(X, m_ref)
        cmp = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res)
        _log(f"step {t} anchor={anchor} recomputed={int(m_gpu.sum())}", cmp)
        assert cmp.ok(), str(cmp)
        imp_g = g.sa.importance[0].cpu().numpy() if anchor else None
        imp_r = oracle.importance(res.weights, rows, w.q_offsets) if anchor else None
        if anchor:
            assert np.abs(imp_g - imp_r).max() <= PT.IMP_ABS_TOL
        d_g = g.sa.delta[0].cpu().numpy() if did else None
        d_r = oracle.local_change(o.local_states(), old_local, rows, w.q_offsets) if t > 0 else None
        if did:
            assert np.allclose(d_g, d_r, rtol=PT.DELTA_REL_TOL, atol=0)
        cp.observe(t, imp_g, d_g)
        shadow.observe(t, imp_g, d_g)
        rp.observe(t, None if imp_r is None else imp_r.astype(np.float32),
                   None if d_r is None else d_r.astype(np.float32))
    cp.close()


# ----------------------------------------------------------------------------- edge cases

def _custom(H, D, S_kv, q_offsets, kv_offsets, seed, B=1):
    w = W.Workload(name=f"custom{seed}", H=H, D=D, grid=(S_kv,), P=len(kv_offsets) - 1,
                   q_token_range=(0, q_offsets[-1]), q_offsets=list(q_offsets), local_part=[0] * (len(q_offsets) - 1),
                   group_offsets=[0, len(kv_offsets) - 1], recompute_groups=1, mode="distance", seed=seed,
                   prev_scale=0.05)
    return w


@pytest.mark.parametrize("D", [64, 128])
def test_empty_partition_and_one_row_block(D):
    qo = [0, 1, 130, 300]
    ko = [0, 70, 70, 200, 333]      # partition 1 is empty
    w = _custom(3, D, 333, qo, ko, seed=77)
    local = [0, 2, 3]
    mask = np.array([[1, 1, 0, 1], [0, 1, 1, 0], [1, 0, 0, 1]], np.uint8)
    rows = np.arange(300)
    Xp, X = W.make_step(w, -1), W.make_step(w, 0)
    g = PT.GpuRun(w, q_offsets=qo, kv_offsets=ko, local_part=local)
    o = PT.OracleRun(w, rows, q_offsets=qo, kv_offsets=ko, local_part=local)
    ones = np.ones_like(mask)
    g.step(Xp, ones)
    o.step(Xp, ones)
    old = o.local_states()
    did = g.step(X, mask, want_delta=True, want_importance=True)
    res = o.step(X, mask)
    cmp = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res)
    _log("edge", D, cmp)
    assert cmp.ok(), str(cmp)
    cl = g.cache_lse_rows(rows)
    assert np.isneginf(cl[1]).all()          # empty partition: lse = -inf
    assert (g.cache_o_rows(rows)[1] == 0).all()
    assert did
    d_r = oracle.local_change(o.local_states(), old, rows, qo)
    assert np.allclose(g.sa.delta[0].cpu().numpy(), d_r, rtol=PT.DELTA_REL_TOL)
    imp = g.sa.importance[0].cpu().numpy()
    assert (imp[:, 1] == 0).all()
    assert np.abs(imp - oracle.importance(res.weights, rows, qo)).max() <= PT.IMP_ABS_TOL


def test_all_partitions_empty_gives_zero_output():
    S_q, H, D = 70, 2, 128
    q = torch.randn(1, S_q, H, D, device="cuda").to(torch.bfloat16)
    k = torch.empty(1, 0, H, D, device="cuda", dtype=torch.bfloat16)
    sa = api.SelectiveAttention(1, S_q, 0, H, D, [0, S_q], [0, 0, 0], [0])
    sa.step(q, k, k, np.ones((1, 2), np.uint8))
    torch.cuda.synchronize()
    assert (sa.out.float() == 0).all() and torch.isneginf(sa.lse).all()


def test_batch_of_two_matches_single_batches():
    H, D, S = 2, 128, 400
    qo, ko = [0, 150, 400], [0, 100, 250, 400]
    torch.manual_seed(0)
    q = torch.randn(2, S, H, D, device="cuda").to(torch.bfloat16)
    k = torch.randn(2, S, H, D, device="cuda").to(torch.bfloat16)
    v = torch.randn(2, S, H, D, device="cuda").to(torch.bfloat16)
    mask = np.array([[1, 1, 1], [1, 1, 1]], np.uint8)
    sa2 = api.SelectiveAttention(2, S, S, H, D, qo, ko, [0, 1])
    sa2.step(q, k, v, mask, want_importance=True)
    for b in range(2):
        sa1 = api.SelectiveAttention(1, S, S, H, D, qo, ko, [0, 1])
        sa1.step(q[b:b + 1].contiguous(), k[b:b + 1].contiguous(), v[b:b + 1].contiguous(), mask,
                 want_importance=True)
        torch.cuda.synchronize()
        assert torch.equal(sa1.out[0], sa2.out[b]) and torch.equal(sa1.lse[0], sa2.lse[b])
        assert torch.equal(sa1.importance[0], sa2.importance[b])


def test_explicit_softmax_scale():
    w = W.workload("tiny")
    X = W.make_step(w, 0)
    q, k, v = PT.to_dev(X.q), PT.to_dev(X.k), PT.to_dev(X.v)
    sa = api.SelectiveAttention(1, 256, 256, 2, 64, [0, 256], w.kv_offsets, [0])
    sa.step(q, k, v, np.ones((1, 4), np.uint8), scale=0.05)
    torch.cuda.synchronize()
    rows = np.arange(256)
    qd, kd, vd = W.to_f64(X.q[0]), W.to_f64(X.k[0]), W.to_f64(X.v[0])
    O, lse = oracle.full_attention(qd, kd, vd, 0.05)
    PT.assert_rows_close(PT.bf16_to_f64(sa.out[0]), O, "explicit scale")
    assert np.abs(sa.lse[0].double().cpu().numpy() - lse).max() <= PT.LSE_ABS_TOL


def test_split_entry_points_match_one_call():
    """dit_partition_attention + dit_state_merge + dit_importance + finalize == one call."""
    w = W.workload("video720p", grid=(3, 12, 20), H=3)
    X = W.make_step(w, 0)
    q, k, v = PT.to_dev(X.q), PT.to_dev(X.k), PT.to_dev(X.v)
    m, _, _, _ = PT.masks_from_planners(w)
    ones = np.ones_like(m)
    a = api.SelectiveAttention(1, w.S_q, w.S_kv, w.H, w.D, w.q_offsets, w.kv_offsets, w.local_part)
    a.step(q, k, v, ones)
    cache_o0, cache_lse0 = a.cache_o.clone(), a.cache_lse.clone()
    a.step(q, k, v, m, want_importance=True, want_delta=True)
    co, cl = cache_o0.clone(), cache_lse0.clone()
    out = torch.empty_like(a.out)
    lse = torch.empty_like(a.lse)
    imp = torch.empty_like(a.importance)
    dl = torch.empty_like(a.delta)
    ws = torch.empty_like(a.workspace)
    api.partition_attention(q, k, v, w.q_offsets, w.kv_offsets, m, co, cl, local_part=w.local_part,
                            workspace=ws)
    api.state_merge(co, cl, out, lse, q_offsets=w.q_offsets, importance_out=imp, workspace=ws)
    api.local_change_finalize(ws, 1, w.S_q, w.H, w.D, w.q_offsets, dl)
    torch.cuda.synchronize()
    assert torch.equal(out, a.out) and torch.equal(lse, a.lse)
    assert torch.equal(co, a.cache_o) and torch.equal(cl, a.cache_lse)
    assert torch.equal(imp, a.importance) and torch.equal(dl, a.delta)
    # the second pass over the stored lse planes gives the same importance up to fp32 rounding
    imp2 = torch.empty_like(imp)
    api.importance(cl, lse, w.q_offsets, imp2)
    torch.cuda.synchronize()
    assert (imp2 - imp).abs().max().item() <= 1e-6


def test_tile_sum_bound_and_maximum_jumps():
    """The kernel takes each tile's exponentials against the running maximum first and
    computes the tile maximum only when a lane's tile sum exceeds 2^8.  Three cases in one
    sequence of 20 key tiles: the first tile (no maximum yet), a tile whose 32 scores all sit
    6.5 (base 2) above the running maximum (sum far above 2^8 with no single exponential
    above it: no rescale), and two keys 29 (base 2) above it (a real rescale).  Scores are
    built from one direction u: q = 4u + noise, k = a u (+ noise elsewhere)."""
    rng = np.random.default_rng(11)
    S, H, D = 640, 2, 128
    u = rng.standard_normal(D)
    u /= np.linalg.norm(u)
    q = 4.0 * u + 0.1 * rng.standard_normal((S, H, D))
    k = 0.1 * rng.standard_normal((S, H, D))
    v = rng.standard_normal((S, H, D))
    sq = math.sqrt(D)
    k[160:192] = (4.5 * sq / 4.0) * u          # tile 5: every score ~ 4.5 (natural log units)
    k[400:402] = (20.0 * sq / 4.0) * u         # tile 12: two scores ~ 20
    bits = [W.f32_to_bf16_bits(x[None].astype(np.float32)) for x in (q, k, v)]
    qd, kd, vd = (W.to_f64(b[0]) for b in bits)
    s_chk = np.einsum("hd,khd->hk", qd[0], kd) / sq
    assert s_chk[:, 160:192].min() > 4.0 and s_chk[:, 400:402].min() > 19.0   # the planted scores
    sa = api.SelectiveAttention(1, S, S, H, D, [0, S], [0, S], [0])
    sa.step(*(PT.to_dev(b) for b in bits), np.ones((1, 1), np.uint8))
    torch.cuda.synchronize()
    O, lse = oracle.full_attention(qd, kd, vd, 1.0 / sq)
    PT.assert_rows_close(PT.bf16_to_f64(sa.out[0]), O, "tile-sum bound")
    assert np.abs(sa.lse[0].double().cpu().numpy() - lse).max() <= PT.LSE_ABS_TOL


def _max_layout(D, seed):
    """64 query blocks (1 to 17 rows) and 64 partitions (4 to 16 keys, four of them empty),
    the largest counts the library takes; each block's local partition is a non-empty one."""
    qs = [1 + (i * 7) % 17 for i in range(64)]
    ks = [0 if i % 17 == 0 else 4 + (i * 5) % 13 for i in range(64)]
    qo = [0] + list(np.cumsum(qs))
    ko = [0] + list(np.cumsum(ks))
    S_kv = ko[-1]
    assert qo[-1] <= S_kv
    local = [i if ks[i] > 0 else i + 1 for i in range(64)]
    w = _custom(2, D, S_kv, qo, ko, seed=seed)
    rng = np.random.default_rng(seed)
    mask = (rng.random((64, 64)) < 0.5).astype(np.uint8)
    mask[np.arange(64), local] = 1
    return w, qo, ko, local, mask


@pytest.mark.parametrize("D", [64, 128])
def test_maximum_blocks_and_partitions(D):
    w, qo, ko, local, mask = _max_layout(D, seed=91 + D)
    rows = np.arange(qo[-1])
    Xp, X = W.make_step(w, -1), W.make_step(w, 0)
    g = PT.GpuRun(w, q_offsets=qo, kv_offsets=ko, local_part=local)
    o = PT.OracleRun(w, rows, q_offsets=qo, kv_offsets=ko, local_part=local)
    ones = np.ones_like(mask)
    g.step(Xp, ones)
    o.step(Xp, ones)
    old = o.local_states()
    assert g.step(X, mask, want_delta=True, want_importance=True)
    res = o.step(X, mask)
    cmp = PT.compare_out(g.out_rows(rows), g.lse_rows(rows), res)
    _log("64 blocks x 64 partitions", D, cmp)
    assert cmp.ok(), str(cmp)
    d_r = oracle.local_change(o.local_states(), old, rows, qo)
    assert np.allclose(g.sa.delta[0].cpu().numpy(), d_r, rtol=PT.DELTA_REL_TOL)
    imp = g.sa.importance[0].cpu().numpy()
    assert np.abs(imp - oracle.importance(res.weights, rows, qo)).max() <= PT.IMP_ABS_TOL
    empty = [p for p in range(64) if ko[p + 1] == ko[p]]
    assert len(empty) == 4 and (imp[:, empty] == 0).all()
