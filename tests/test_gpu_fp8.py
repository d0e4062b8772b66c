"""GPU parity of the compressed (fp8 e4m3 + per-row-head scale) state cache.

The codes are rounding decisions taken from the kernel's fp32 states, which differ from
the oracle's fp64 states by the bf16 product error, so codes are not compared one by one.
That difference is bounded per row (one query row and head, over D) by PROD_ROW_TOL times
the row's largest magnitude: each probability is rounded to bf16 (2^-9 relative) before
the P V product, so a state element moves by at most 2^-9 of the row's weighted |V|, and
2^-7 of the row maximum leaves a factor of four.  Instead:
  - every cached slot, decoded by the oracle's bit-field decoder, lies within the e4m3
    rounding bound max(2^-4 |x|, 2^-10 s) of the oracle's exact state x plus that row
    term, and its scale within 2^-7 of max_d |x| / 448;
  - the fp8 merge kernel, fed the kernel's own codes, matches the oracle's fp64 merge of
    the decoded states to bf16 output rounding;
  - a selective step (fresh and reused fp8 states) matches the oracle's exact step within
    the merged rounding bound sum_p w_p [max(2^-4 |O_p|, 2^-10 s_p) + 2^-7 max_d |O_p|]
    plus the bf16 output rounding (2^-8 |O| covers its 2^-9), and its relative Frobenius
    error stays within 2^-4;
  - the local change computed from fp8 states equals the oracle's norm ratio of the
    decoded codes, and differs from the exact one by at most the quantisation error's
    share (triangle inequality).
"""
import math

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle
import workloads as W
import _parity as PT
from partitioned_state_reuse_amd import api

pytestmark = pytest.mark.gpu

# bf16 output rounding (half an ulp is 2^-9 relative) plus fp32 accumulation
MERGE_REL_TOL = 2.0 ** -8
MERGE_LSE_TOL = 2e-5
# kernel fp32 state vs exact fp64 state, per element, relative to the row's maximum
PROD_ROW_TOL = 2.0 ** -7
# e4m3: half an ulp is 2^-4 relative; the subnormal step is 2^-9 of the scale
E4M3_REL = 2.0 ** -4
E4M3_SUB = 2.0 ** -10


def _log(*a):
    print(*a, flush=True)


class Fp8Run(PT.GpuRun):
    def __init__(self, w, B=1, q_offsets=None, kv_offsets=None, local_part=None):
        self.w = w
        self.qo = list(q_offsets if q_offsets is not None else w.q_offsets)
        self.ko = list(kv_offsets if kv_offsets is not None else w.kv_offsets)
        self.local = list(local_part if local_part is not None else w.local_part)
        self.sa = api.SelectiveAttention(B, self.qo[-1], self.ko[-1], w.H, w.D, self.qo, self.ko, self.local,
                                         cache_format="fp8")

    def deq_rows(self, rows):
        """Decoded cache [P, n, H, D] (codes * scale) and the scales [P, H, n]."""
        idx = torch.as_tensor(rows, device="cuda")
        codes = self.sa.cache_o[:, 0][:, idx].cpu().numpy()
        s = self.sa.cache_scale[:, 0][:, idx, :].double().cpu().numpy()     # [P, n, H]
        vals = oracle.decode_fp8_e4m3(codes)
        assert np.isfinite(vals).all(), "NaN code in the cache"
        return vals * s[..., None], np.ascontiguousarray(np.transpose(s, (0, 2, 1)))


def state_bound(O_exact):
    """Per-element bound of a decoded fp8 state against the exact state O_exact
    [..., n, H, D]: e4m3 rounding of the kernel's value (its scale is within the row term of
    the exact one) plus the kernel's own product error, both from the exact row maximum."""
    amax = np.abs(O_exact).max(axis=-1, keepdims=True)
    row = PROD_ROW_TOL * amax
    s_hi = (amax + row) / 448.0
    return np.maximum((np.abs(O_exact) + row) * E4M3_REL, s_hi * E4M3_SUB) + row


def check_states(deq, s, O_exact, what):
    amax = np.abs(O_exact).max(axis=-1)                        # [P, n, H]
    ds = np.abs(448.0 * np.swapaxes(s, -1, -2) - amax)
    assert (ds <= PROD_ROW_TOL * amax + 1e-30).all(), f"{what}: scale off by {(ds / np.maximum(amax, 1e-30)).max()} relative"
    bound = state_bound(O_exact)
    err = np.abs(deq - O_exact)
    rel = np.linalg.norm(deq - O_exact) / max(np.linalg.norm(O_exact), 1e-300)
    # empty partitions: state 0 and bound 0 (their slots must decode to exactly 0)
    ratio = np.divide(err, bound, out=np.zeros_like(err), where=bound > 0)
    _log(f"{what}: max|deq-O|={err.max():.3e} relF={rel:.3e} (max bound ratio {ratio.max():.3f})")
    assert (err <= bound).all(), f"{what}: {(err > bound).sum()} elements beyond the e4m3 bound"
    assert rel <= E4M3_REL


def step_bound(O_exact_planes, weights, O_ref):
    """Bound of a merged fp8 step [n, H, D] against the exact step O_ref: the weighted sum of
    the planes' state bounds (weights [P, H, n] from the exact states) plus the bf16 output
    rounding."""
    Wt = np.transpose(weights, (0, 2, 1))[:, :, :, None]     # [P, n, H, 1]
    return (Wt * state_bound(O_exact_planes)).sum(axis=0) + 2.0 ** -8 * np.abs(O_ref) + 1e-9


def check_merge_of_own_codes(g, rows):
    deq, s = g.deq_rows(rows)
    lse_c = g.cache_lse_rows(rows)
    ref_O, ref_l = oracle.merge_states(list(deq), list(lse_c))
    out, lse = g.out_rows(rows), g.lse_rows(rows)
    fin = np.isfinite(ref_l)
    assert np.array_equal(np.isfinite(lse), fin)
    dl = np.abs(np.where(fin, lse - ref_l, 0.0)).max()
    dO = np.abs(out - ref_O)
    lim = MERGE_REL_TOL * np.abs(ref_O) + 1e-7
    _log(f"fp8 merge of own codes: max|dO|={dO.max():.3e} max|dlse|={dl:.3e}")
    assert dl <= MERGE_LSE_TOL
    assert (dO <= lim).all(), f"{(dO > lim).sum()} merged elements beyond bf16 rounding"


def run_fp8(w, rows, steps=2, layout=None):
    """Anchor step on X_prev (all recompute), then the planner's selective step on X (or, with
    layout = (q_offsets, kv_offsets, local_part, mask), that split and mask)."""
    if layout is None:
        m_cpp, m_ref, _, _ = PT.masks_from_planners(w)
        assert np.array_equal(m_cpp, m_ref)
        q_off, kv_off, local = list(w.q_offsets), list(w.kv_offsets), list(w.local_part)
    else:
        q_off, kv_off, local, m_cpp = layout
    ones = np.ones_like(m_cpp)
    g = Fp8Run(w, q_offsets=q_off, kv_offsets=kv_off, local_part=local)
    o = PT.OracleRun(w, rows, q_offsets=q_off, kv_offsets=kv_off, local_part=local)
    Xp = W.make_step(w, -1)
    g.step(Xp, ones)
    o.step(Xp, ones)
    deq0, s0 = g.deq_rows(rows)
    check_states(deq0, s0, o.cache.exact_O, f"{w.name} anchor states")
    check_merge_of_own_codes(g, rows)
    if steps < 2:
        return g, o
    full = len(rows) == w.S_q
    old_exact_local = o.local_states("exact")
    blk = oracle.block_of_rows(np.asarray(rows), q_off)
    old_deq_local = np.stack([deq0[local[b], j] for j, b in enumerate(blk)])
    X = W.make_step(w, 0)
    did = g.step(X, m_cpp, want_delta=full)
    res = o.step(X, m_cpp)
    deq1, s1 = g.deq_rows(rows)
    check_merge_of_own_codes(g, rows)
    # merged output against the oracle's exact step: weights from the exact states
    bound = step_bound(o.cache.exact_O, res.weights, res.O)
    out = g.out_rows(rows)
    err = np.abs(out - res.O)
    rel = np.linalg.norm(out - res.O) / np.linalg.norm(res.O)
    _log(f"{w.name} fp8 selective step (recomputed {int(m_cpp.sum())}): max|dO|={err.max():.3e} relF={rel:.3e} "
         f"max bound ratio {(err / bound).max():.3f}")
    assert (err <= bound).all()
    assert rel <= E4M3_REL
    lse = g.lse_rows(rows)
    fin = np.isfinite(res.lse)
    assert np.abs(np.where(fin, lse - res.lse, 0.0)).max() <= PT.LSE_ABS_TOL
    if did:
        new_deq_local = np.stack([deq1[local[b], j] for j, b in enumerate(blk)])
        d_gpu = g.sa.delta[0].cpu().numpy().astype(np.float64)
        d_codes = oracle.local_change(new_deq_local, old_deq_local, np.asarray(rows), q_off)
        d_exact = oracle.local_change(o.local_states("exact"), old_exact_local, np.asarray(rows), q_off)
        _log("delta fp8 gpu", d_gpu[:4], "of codes", d_codes[:4], "exact", d_exact[:4])
        assert np.allclose(d_gpu, d_codes, rtol=1e-4, atol=0)
        # |delta_fp8 - delta_exact| <= (||q_new|| + ||q_old||) / ||O_old|| + delta_fp8 ||q_old|| / ||O_old||
        for i in range(len(q_off) - 1):
            sel = blk == i
            on = np.linalg.norm(old_exact_local[sel])
            qn = np.linalg.norm(new_deq_local[sel] - o.local_states("exact")[sel])
            qo = np.linalg.norm(old_deq_local[sel] - old_exact_local[sel])
            lim = (qn + qo) / on + d_gpu[i] * qo / on + PT.DELTA_REL_TOL * d_exact[i]
            assert abs(d_gpu[i] - d_exact[i]) <= lim, (i, d_gpu[i], d_exact[i], lim)
    return g, o


def test_fp8_tiny_d64():
    w = W.workload("tiny")
    run_fp8(w, np.arange(w.S_q))


def test_fp8_video720p_reduced_grid():
    w = W.workload("video720p", grid=(5, 18, 32), H=4)
    run_fp8(w, np.arange(w.S_q))


@pytest.mark.timeout(900)
def test_fp8_video720p_full_size_sampled_rows():
    w = W.workload("video720p")
    rows = W.sample_rows(w, tiles_per_block=2, tile=16)
    run_fp8(w, rows, steps=2)


def test_fp8_cache_bytes_and_bf16_path_unchanged():
    """The fp8 cache has half the O bytes; the bf16 path on the same inputs is unaffected
    by the fp8 instantiation (bitwise repeatable)."""
    w = W.workload("video720p", grid=(3, 12, 20), H=3)
    g8 = Fp8Run(w)
    gb = PT.GpuRun(w)
    assert g8.sa.cache_o.element_size() * 2 == gb.sa.cache_o.element_size()
    ones = np.ones((w.n_qb, w.P), np.uint8)
    X = W.make_step(w, 0)
    gb.step(X, ones)
    a = gb.sa.out.clone()
    g8.step(X, ones)
    gb.step(X, ones)
    assert torch.equal(a, gb.sa.out)


def test_fp8_rejects_invalid_and_unsupported():
    w = W.workload("tiny")
    g = Fp8Run(w)
    X = W.make_step(w, 0)
    with pytest.raises(api.DitError):
        g.step(X, np.zeros((w.n_qb, w.P), np.uint8) | np.eye(1, w.P, w.local_part[0], dtype=np.uint8))
    with pytest.raises(api.DitError):
        g.sa.compose([0, w.P])
    q = PT.to_dev(X.q)
    with pytest.raises(api.DitError):
        api.partition_attention_fp8(q, PT.to_dev(X.k), PT.to_dev(X.v), w.q_offsets, w.kv_offsets,
                                    np.ones((w.n_qb, w.P), np.uint8), g.sa.cache_o, None, g.sa.cache_lse)


def test_fp8_longvideo_trajectory_reduced_grid():
    """10 denoising steps with the compressed cache: anchor every 5, groups of 4, the w*delta
    planner fed by the GPU's own importance and fp8 delta.  Every step's output stays within
    the e4m3 rounding bound of the oracle's exact step under the same masks, and the anchor
    steps' importance (from lse, which is not compressed) matches the oracle's."""
    w = W.workload("longvideo", grid=(9, 18, 32), H=2)
    rows = np.arange(w.S_q)
    g = Fp8Run(w)
    o = PT.OracleRun(w, rows)
    cp = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every, w.recompute_groups, "wdelta")
    worst = 0.0
    for t in range(w.steps):
        X = W.make_step(w, t)
        mask, _ = cp.next(t)
        anchor = t % w.anchor_every == 0
        did = g.step(X, mask, want_importance=anchor, want_delta=t > 0)
        res = o.step(X, mask)
        bound = step_bound(o.cache.exact_O, res.weights, res.O)
        out = g.out_rows(rows)
        err = np.abs(out - res.O)
        rel = np.linalg.norm(out - res.O) / np.linalg.norm(res.O)
        worst = max(worst, float((err / bound).max()))
        _log(f"step {t} anchor={anchor} recomputed={int(mask.sum())} max|dO|={err.max():.3e} relF={rel:.3e} "
             f"bound ratio {(err / bound).max():.3f}")
        assert (err <= bound).all(), t
        assert rel <= E4M3_REL, t
        imp = None
        if anchor:
            imp = g.sa.importance[0].cpu().numpy()
            assert np.abs(imp - oracle.importance(res.weights, rows, w.q_offsets)).max() <= PT.IMP_ABS_TOL
        d = g.sa.delta[0].cpu().numpy() if did else None
        if d is not None:
            assert np.isfinite(d).all() and (d > 0).all()
        cp.observe(t, imp, d)
    cp.close()
    _log("worst bound ratio over the trajectory", worst)


@pytest.mark.parametrize("D", [64, 128])
def test_fp8_maximum_blocks_and_partitions(D):
    """64 query blocks and 64 partitions, four of them empty (their slots hold scale 0 and
    codes 0), D = 64 and 128."""
    from test_gpu_parity import _max_layout
    w, qo, ko, local, mask = _max_layout(D, seed=95 + D)
    run_fp8(w, np.arange(qo[-1]), layout=(qo, ko, local, mask))
