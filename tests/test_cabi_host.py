"""CPU checks of the C-ABI library: it loads, exports every symbol the header declares,
validates arguments on the host (no kernel is launched: every call here fails validation
before reaching the GPU), and its host planner matches the oracle planner bit-exactly."""
import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dit_attn.h")

from partitioned_state_reuse_amd import _lib  # noqa: E402


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_ ]*\**\s*\**(dit_[a-z_0-9]+)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        import partitioned_state_reuse_amd.build as B
        B.build()
    return _lib.lib()


def test_header_symbols_exported(L):
    names = header_functions()
    assert len(names) >= 12, names
    for n in names:
        assert hasattr(L, n), n
        assert n in _lib.SIGNATURES, f"binding lacks {n}"


def test_status_strings(L):
    for code in range(0, -10, -1):
        s = L.dit_status_string(code).decode()
        assert s.startswith("DIT_")
    assert L.dit_status_string(5).decode() == "unknown status"


def test_workspace_bytes(L):
    # local-change partials: (591 + 16) 128-row query tiles x 40 heads x 2 floats, then from the
    # next 256-byte boundary the merge's importance partials: (75,600 x 40 / 16 + 16) merge
    # workgroups x 16 planes x 4 bytes
    delta = (591 + 16) * 40 * 8
    assert L.dit_attn_workspace_bytes(1, 75600, 40, 128, 16, 16) == (delta + 255) // 256 * 256 + (189000 + 16) * 16 * 4
    assert L.dit_attn_workspace_bytes(1, 100, 4, 96, 1, 1) == 0      # unsupported D
    assert L.dit_attn_workspace_bytes(1, 100, 4, 64, 0, 1) == 0      # no blocks
    assert L.dit_attn_workspace_bytes(1, 100, 4, 64, 1, 65) == 0     # too many partitions


def _call(L, *, q=1, k=1, v=1, B=1, S_q=8, S_kv=8, H=1, D=64, qo=(0, 8), ko=(0, 4, 8), local=(0,),
          rec=(1, 0), valid=None, cache_o=1, cache_lse=1, out=1, lse=1, delta=None, ws=None, ws_bytes=0):
    """dit_attn_partitioned with fake (never dereferenced) device pointers."""
    i32 = lambda s: None if s is None else (ctypes.c_int32 * len(s))(*s)
    u8 = lambda s: None if s is None else (ctypes.c_uint8 * len(s))(*s)
    return L.dit_attn_partitioned(q, k, v, B, S_q, S_kv, H, D, i32(qo), len(qo) - 1 if qo else 1, i32(ko),
                                  len(ko) - 1 if ko else 1, i32(local), u8(rec), u8(valid), cache_o, cache_lse,
                                  out, lse, 0.0, None, delta, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), -1), (dict(out=None), -1), (dict(cache_lse=None), -1), (dict(rec=None), -1),
    (dict(qo=None), -1), (dict(ko=None), -1),
    (dict(B=0), -2), (dict(H=0), -2), (dict(S_q=-1), -2),
    (dict(D=96), -7), (dict(D=256), -7),
    (dict(qo=(0, 4, 4, 8)), -3), (dict(qo=(1, 8)), -3), (dict(qo=(0, 7)), -3),
    (dict(ko=(0, 5, 4, 8)), -3), (dict(ko=(0, 4, 9)), -3),
    (dict(rec=(2, 0)), -4), (dict(rec=(0, 1)), -4), (dict(local=(2,)), -4),
    (dict(valid=(1, 0)), -5),
    (dict(delta=1), -6), (dict(delta=1, ws=1, ws_bytes=4), -6),
    (dict(delta=1, ws=1, ws_bytes=1 << 20, valid=(0, 1), rec=(1, 1)), -5),
    (dict(delta=1, ws=1, ws_bytes=1 << 20, local=None), -1),
])
def test_validation_rejects_before_launch(L, kw, code):
    assert _call(L, **kw) == code


def test_binding_refuses_host_and_mismatched_tensors(L):
    """The Python binding hands the library raw device addresses, so it checks device,
    dtype, contiguity and shape first (a host tensor here would be read as device memory)."""
    import torch
    from partitioned_state_reuse_amd import api
    co = torch.zeros((2, 1, 8, 1, 64), dtype=torch.bfloat16)
    cl = torch.zeros((2, 1, 1, 8))
    out = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16)
    lse = torch.zeros((1, 1, 8))
    with pytest.raises(ValueError, match="GPU tensor"):
        api.state_merge(co, cl, out, lse)
    q = torch.zeros((1, 8, 1, 64), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU tensor"):
        api.partition_attention(q, q, q, [0, 8], [0, 4, 8], [[1, 1]], co, cl)
    with pytest.raises(ValueError, match="disagree"):
        api.partition_attention(q, torch.zeros((1, 8, 2, 64), dtype=torch.bfloat16), q, [0, 8], [0, 4, 8],
                                [[1, 1]], co, cl)


def test_attention_grid_beyond_32_bit_work_items(L):
    """2M query rows, 40 heads, 64 recomputed partitions: 1e6 items per head x 256 threads."""
    S_q = 2_000_000
    assert _call(L, S_q=S_q, S_kv=64, H=40, D=128, qo=(0, S_q), ko=tuple(range(65)), rec=(1,) * 64) == -2


def test_importance_needs_the_workspace(L):
    """The one-call step computes the importance inside the merge: importance_out without a
    workspace large enough for the partials is DIT_ERR_WORKSPACE."""
    i32 = lambda s: (ctypes.c_int32 * len(s))(*s)
    u8 = lambda s: (ctypes.c_uint8 * len(s))(*s)
    args = lambda ws, wsb: (1, 1, 1, 1, 8, 8, 1, 64, i32([0, 8]), 1, i32([0, 4, 8]), 2, i32([0]), u8([1, 0]), None,
                           1, 1, 1, 1, 0.0, 1, None, ws, wsb, None)
    assert L.dit_attn_partitioned(*args(None, 0)) == -6
    assert L.dit_attn_partitioned(*args(1, 256)) == -6


def _tile_span_limit(D):
    """Largest H*D whose 32-key tile rows (31 row strides of H*D bf16 plus one row of D)
    fit a 31-bit buffer range, and H*D must be a multiple of D."""
    return ((2 ** 31 - 1) // 2 - D) // 31 // D * D


@pytest.mark.parametrize("D", [64, 128])
def test_head_width_at_the_tile_buffer_range(L, D):
    """The shape check of the attention calls passes at the largest H for D and fails one
    head above it.  An accepted shape is shown by the next check failing instead (delta
    requested without a workspace: DIT_ERR_WORKSPACE), so no kernel is launched."""
    H = _tile_span_limit(D) // D
    assert (31 * H * D + D) * 2 <= 2 ** 31 - 1 < (31 * (H + 1) * D + D) * 2
    assert _call(L, H=H, D=D, delta=1) == -6
    assert _call(L, H=H + 1, D=D, delta=1) == -2
    # 2^25 (accepted) and 2^25 - 64 (accepted); the merge does not build a tile descriptor
    for hd in (1 << 25, (1 << 25) - 64):
        assert _call(L, H=hd // 64, D=64, delta=1) == -6


def test_merge_does_not_apply_the_tile_range_limit(L):
    """Only the attention calls copy K/V tiles: a merge with H*D above the tile limit passes
    the shape check (it fails later, on a NULL output pointer)."""
    H = _tile_span_limit(128) // 128 + 1
    assert L.dit_state_merge(1, 1, 1, 8, H, 128, 2, None, 1, None, 0, None, None, 0, None) == -1


def test_too_many_blocks_or_partitions(L):
    qo = list(range(0, 66))
    assert _call(L, S_q=65, qo=qo, rec=[1, 0] * 65, local=[0] * 65) == -2
    ko = list(range(0, 66))
    assert _call(L, S_kv=65, ko=ko, rec=[1] + [0] * 64) == -2


def _i32(s):
    return None if s is None else (ctypes.c_int32 * len(s))(*s)


def _u8(s):
    return None if s is None else (ctypes.c_uint8 * len(s))(*s)


@pytest.mark.parametrize("call,code", [
    # dit_partition_attention_fp8(q, k, v, B, S_q, S_kv, H, D, qo, n_qb, ko, P, local, rec, valid, q8, scale, lse,
    #                             sm, ws, wsb, st)
    (lambda L: L.dit_partition_attention_fp8(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2, _i32([0]),
                                             _u8([1, 0]), None, 1, None, 1, 0.0, None, 0, None), -1),
    (lambda L: L.dit_partition_attention_fp8(1, 1, 1, 1, 8, 8, 1, 96, _i32([0, 8]), 1, _i32([0, 4, 8]), 2, _i32([0]),
                                             _u8([1, 0]), None, 1, 1, 1, 0.0, None, 0, None), -7),
    (lambda L: L.dit_partition_attention_fp8(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 5, 4]), 2, _i32([0]),
                                             _u8([1, 0]), None, 1, 1, 1, 0.0, None, 0, None), -3),
    (lambda L: L.dit_partition_attention_fp8(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2, _i32([0]),
                                             _u8([0, 1]), None, 1, 1, 1, 0.0, None, 0, None), -4),
    # the compressed cache refuses reuse of a never-computed slot itself
    (lambda L: L.dit_partition_attention_fp8(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2, _i32([0]),
                                             _u8([1, 0]), _u8([1, 0]), 1, 1, 1, 0.0, None, 0, None), -5),
    # ... and a delta against a never-computed local slot
    (lambda L: L.dit_partition_attention_fp8(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2, _i32([0]),
                                             _u8([1, 1]), _u8([0, 1]), 1, 1, 1, 0.0, 1, 1 << 20, None), -5),
    # dit_partition_attention(q, k, v, B, S_q, S_kv, H, D, qo, n_qb, ko, P, local, rec, valid, o, lse, sm, ws, wsb, st)
    (lambda L: L.dit_partition_attention(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2, _i32([0]),
                                         _u8([1, 0]), _u8([1, 0]), 1, 1, 0.0, None, 0, None), -5),
    # dit_partition_attention_premerge(q, k, v, B, S_q, S_kv, H, D, qo, n_qb, ko, P, local, rec, valid, o, lse, sm,
    #                                  pre_o, pre_lse, ws, wsb, st): the partial state's buffers, the workspace
    #                                  (local-change partials and the chunk counter from the first 256-byte
    #                                  boundary past them: 260 bytes here), the mask and the validity bitmap
    (lambda L: L.dit_partition_attention_premerge(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2,
                                                  None, _u8([1, 0]), None, 1, 1, 0.0, None, 1, 1, 1 << 20, None), -1),
    (lambda L: L.dit_partition_attention_premerge(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2,
                                                  None, _u8([1, 0]), None, 1, 1, 0.0, 1, 1, None, 0, None), -6),
    (lambda L: L.dit_partition_attention_premerge(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2,
                                                  _i32([0]), _u8([1, 0]), None, 1, 1, 0.0, 1, 1, 1, 256, None), -6),
    (lambda L: L.dit_partition_attention_premerge(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2,
                                                  None, _u8([1, 0]), _u8([1, 0]), 1, 1, 0.0, 1, 1, 1, 1 << 20, None), -5),
    (lambda L: L.dit_partition_attention_premerge(1, 1, 1, 1, 8, 8, 1, 64, _i32([0, 8]), 1, _i32([0, 4, 8]), 2,
                                                  _i32([0]), _u8([0, 1]), None, 1, 1, 0.0, 1, 1, 1, 1 << 20, None), -4),
    (lambda L: L.dit_partition_attention_premerge(1, 1, 1, 1, 8, 8, 1, 96, _i32([0, 8]), 1, _i32([0, 4, 8]), 2,
                                                  None, _u8([1, 0]), None, 1, 1, 0.0, 1, 1, 1, 1 << 20, None), -7),
    # dit_state_merge_fp8(q8, scale, lse, B, S_q, H, D, P, out, lse_out, qo, n_qb, imp, ws, wsb, st)
    (lambda L: L.dit_state_merge_fp8(1, None, 1, 1, 8, 1, 64, 2, 1, 1, None, 0, None, None, 0, None), -1),
    (lambda L: L.dit_state_merge_fp8(1, 1, 1, 1, 8, 1, 64, 65, 1, 1, None, 0, None, None, 0, None), -2),
    (lambda L: L.dit_state_merge_fp8(1, 1, 1, 1, 8, 1, 48, 2, 1, 1, None, 0, None, None, 0, None), -7),
    # importance in the fp8 merge: offsets, then the workspace
    (lambda L: L.dit_state_merge_fp8(1, 1, 1, 1, 8, 1, 64, 2, 1, 1, _i32([0, 9]), 1, 1, 1, 1 << 20, None), -3),
    (lambda L: L.dit_state_merge_fp8(1, 1, 1, 1, 8, 1, 64, 2, 1, 1, _i32([0, 8]), 1, 1, None, 0, None), -6),
    (lambda L: L.dit_state_merge_fp8(1, 1, 1, 1, 8, 1, 64, 2, 1, 1, _i32([0, 8]), 1, 1, 1, 256, None), -6),
    # dit_state_merge(o, lse, B, S_q, H, D, P, out, lse_out, qo, n_qb, imp, ws, wsb, st)
    (lambda L: L.dit_state_merge(1, 1, 1, 8, 1, 64, 0, 1, 1, None, 0, None, None, 0, None), -2),
    (lambda L: L.dit_state_merge(1, None, 1, 8, 1, 64, 2, 1, 1, None, 0, None, None, 0, None), -1),
    # 8M rows x 40 heads x 16 threads per row-head: more work-items than one dispatch can count
    (lambda L: L.dit_state_merge(1, 1, 1, 8_000_000, 40, 128, 2, 1, 1, None, 0, None, None, 0, None), -2),
    # importance in the merge: offsets checked, workspace required and large enough
    (lambda L: L.dit_state_merge(1, 1, 1, 8, 1, 64, 2, 1, 1, None, 1, 1, 1, 1 << 20, None), -1),
    (lambda L: L.dit_state_merge(1, 1, 1, 8, 1, 64, 2, 1, 1, _i32([0, 4, 4, 8]), 3, 1, 1, 1 << 20, None), -3),
    (lambda L: L.dit_state_merge(1, 1, 1, 8, 1, 64, 2, 1, 1, _i32([0, 8]), 1, 1, None, 0, None), -6),
    (lambda L: L.dit_state_merge(1, 1, 1, 8, 1, 64, 2, 1, 1, _i32([0, 8]), 1, 1, 1, 256, None), -6),
    # dit_state_merge_masked(o, lse, B, S_q, H, D, P, qo, n_qb, sel, extra_o, extra_lse, out, lse_out, st)
    (lambda L: L.dit_state_merge_masked(1, 1, 1, 8, 1, 64, 2, _i32([0, 8]), 1, _u8([1, 2]), None, None, 1, 1, None), -4),
    (lambda L: L.dit_state_merge_masked(1, 1, 1, 8, 1, 64, 2, _i32([0, 9]), 1, _u8([1, 0]), None, None, 1, 1, None), -3),
    (lambda L: L.dit_state_merge_masked(1, 1, 1, 8, 1, 64, 2, _i32([0, 8]), 1, _u8([1, 0]), 1, None, 1, 1, None), -1),
    # dit_state_compose(o, lse, P_in, go, G, B, S_q, H, D, out_o, out_lse, st)
    (lambda L: L.dit_state_compose(1, 1, 4, _i32([0, 2, 2, 4]), 3, 1, 8, 1, 64, 1, 1, None), -3),
    (lambda L: L.dit_state_compose(1, 1, 4, _i32([0, 2, 3]), 2, 1, 8, 1, 64, 1, 1, None), -3),
    (lambda L: L.dit_state_compose(1, 1, 4, _i32([0, 1, 2, 3, 4, 4]), 5, 1, 8, 1, 64, 1, 1, None), -2),
    (lambda L: L.dit_state_compose(1, 1, 4, _i32([0, 4]), 1, 1, 8, 1, 80, 1, 1, None), -7),
    # dit_importance(clse, lse, B, S_q, H, P, qo, n_qb, imp, st) and dit_local_change_finalize
    (lambda L: L.dit_importance(1, 1, 1, 8, 1, 2, _i32([0, 4, 4, 8]), 3, 1, None), -3),
    (lambda L: L.dit_local_change_finalize(1, 4, 1, 8, 1, 64, _i32([0, 8]), 1, 1, None), -6),
], ids=lambda x: "" if callable(x) else str(x))
def test_other_entry_points_validate_before_launch(L, call, code):
    """Each error is caught on the host (fake device pointers are never dereferenced)."""
    assert call(L) == code


# ----------------------------------------------------------------------------- planner

from partitioned_state_reuse_amd.api import Planner, DitError  # noqa: E402
from oracle import RefPlanner  # noqa: E402


def test_planner_rejects_bad_arguments(L):
    with pytest.raises(DitError):
        Planner(1, 4, [0, 2, 2, 4], [0], 5, 1, "wdelta")   # empty group
    with pytest.raises(DitError):
        Planner(1, 4, [0, 2, 4], [4], 5, 1, "wdelta")      # local out of range
    with pytest.raises(DitError):
        Planner(1, 4, [0, 2, 4], [0], 5, 3, "wdelta")      # K > G
    with pytest.raises(DitError):
        Planner(1, 4, [0, 2, 4], [0], 0, 1, "wdelta")      # no anchor period


@pytest.mark.parametrize("seed", range(6))
def test_planner_matches_oracle_planner_bit_exact(L, seed):
    """Same (w, delta) inputs -> identical scores (bitwise) and identical selections."""
    rng = np.random.default_rng(100 + seed)
    P = int(rng.choice([8, 16, 32]))
    gs = int(rng.choice([1, 2, 4]))
    n_qb = int(rng.integers(1, 9))
    go = list(range(0, P + 1, gs))
    G = len(go) - 1
    K = int(rng.integers(1, G + 1))
    local = rng.integers(0, P, size=n_qb).tolist()
    anchor_every = int(rng.integers(2, 6))
    cp = Planner(n_qb, P, go, local, anchor_every, K, "wdelta")
    rp = RefPlanner(n_qb, P, go, local, anchor_every, K, "wdelta")
    for t in range(14):
        sc, sr = cp.scores(t), np.array(rp.scores(t))
        assert np.array_equal(sc, sr), (t, sc, sr)
        m1, c1 = cp.next(t)
        m2, c2 = rp.next(t)
        assert np.array_equal(m1, m2) and c1 == c2, t
        imp = None
        if t % anchor_every == 0:
            imp = rng.random((n_qb, P)).astype(np.float32)
            if seed % 2:  # force exact ties
                imp = np.round(imp * 4).astype(np.float32) / 4
        d = rng.random(n_qb).astype(np.float32) * 0.1 if t > 0 else None
        if d is not None and seed == 3:
            d[0] = np.nan                                # unobserved entry
        cp.observe(t, imp, d)
        rp.observe(t, imp, d)
    cp.close()


@pytest.mark.parametrize("name", ["tiny", "video720p", "share32"])
def test_distance_planner_matches_oracle(L, name):
    import workloads as W
    w = W.workload(name)
    cp = Planner(w.n_qb, w.P, w.group_offsets, w.local_part, 0, w.recompute_groups, "distance")
    rp = RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, 0, w.recompute_groups, "distance")
    m1, c1 = cp.next(0)
    m2, c2 = rp.next(0)
    assert np.array_equal(m1, m2) and c1 == c2


def test_anchor_mode_all_ones(L):
    cp = Planner(8, 8, list(range(9)), list(range(8)), 0, 8, "anchor")
    m, _ = cp.next(3)
    assert m.all()
