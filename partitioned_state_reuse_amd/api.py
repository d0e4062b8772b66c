"""Python binding of the C ABI (include/dit_attn.h): argument marshalling only.

PyTorch supplies device memory and the stream; every step of the path runs in the HIP
library.  Errors from the library raise DitError(code, message).
"""
from __future__ import annotations

import ctypes
from typing import List, Optional, Sequence, Tuple

import numpy as np
import torch

from . import _lib

DIT_PLAN_WDELTA, DIT_PLAN_DISTANCE, DIT_PLAN_ANCHOR = 0, 1, 2
MODES = {"wdelta": DIT_PLAN_WDELTA, "distance": DIT_PLAN_DISTANCE, "anchor": DIT_PLAN_ANCHOR}


class DitError(RuntimeError):
    """A library call returned a non-zero status; `code` is the DIT_ERR_* value."""

    def __init__(self, code: int, message: str):
        super().__init__(f"{message} (status {code})")
        self.code = code


def _check(code: int) -> None:
    if code != 0:
        raise DitError(code, _lib.lib().dit_status_string(code).decode())


def status_string(code: int) -> str:
    """dit_status_string: the name of a status code."""
    return _lib.lib().dit_status_string(code).decode()


def _i32(seq) -> ctypes.Array:
    a = np.ascontiguousarray(np.asarray(seq, dtype=np.int32))
    return (ctypes.c_int32 * len(a))(*a.tolist())


def _u8(arr) -> ctypes.Array:
    a = np.ascontiguousarray(np.asarray(arr, dtype=np.uint8)).reshape(-1)
    return (ctypes.c_uint8 * len(a)).from_buffer_copy(a.tobytes())


def _stream(stream) -> Optional[int]:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _dims(q: torch.Tensor, k: torch.Tensor) -> Tuple[int, int, int, int, int]:
    B, S_q, H, D = q.shape
    Bk, S_kv, Hk, Dk = k.shape
    if (B, H, D) != (Bk, Hk, Dk):
        raise ValueError(f"q {tuple(q.shape)} and k {tuple(k.shape)} disagree")
    return B, S_q, S_kv, H, D


def _dev(t: Optional[torch.Tensor], dtype, shape, name: str) -> Optional[int]:
    """Device address of `t` once it is known to be a contiguous GPU tensor of the expected
    dtype and shape (`shape` None: any).  The library reads every pointer as raw device
    memory of the documented layout, so a host tensor or a strided view must not reach it.
    None passes through (the library reports a missing required pointer itself)."""
    if t is None:
        return None
    if (not isinstance(t, torch.Tensor) or not t.is_cuda or t.dtype != dtype or not t.is_contiguous()
            or (shape is not None and tuple(t.shape) != tuple(shape))):
        got = (f"{t.dtype} {tuple(t.shape)} contiguous={t.is_contiguous()} device={t.device}"
               if isinstance(t, torch.Tensor) else type(t).__name__)
        want = "any shape" if shape is None else f"shape {tuple(shape)}"
        raise ValueError(f"{name}: need a contiguous {dtype} GPU tensor of {want}, got {got}")
    return t.data_ptr()


BF16, F32, U8 = torch.bfloat16, torch.float32, torch.uint8


def _qkv(q, k, v):
    """Shapes of q [B,S_q,H,D] and k, v [B,S_kv,H,D] and their device addresses."""
    if q is None or k is None:
        raise ValueError("q and k are required")
    B, S_q, S_kv, H, D = _dims(q, k)
    return (B, S_q, S_kv, H, D), (_dev(q, BF16, (B, S_q, H, D), "q"), _dev(k, BF16, (B, S_kv, H, D), "k"),
                                  _dev(v, BF16, (B, S_kv, H, D), "v"))


def _ws(t: Optional[torch.Tensor], name: str) -> Tuple[Optional[int], int]:
    """Address and byte size of a float32 workspace (any shape)."""
    if t is None:
        return None, 0
    return _dev(t, F32, None, name), t.numel() * t.element_size()


def workspace_bytes(B: int, S_q: int, H: int, D: int, n_qb: int, P: int) -> int:
    """dit_attn_workspace_bytes: device workspace bytes a step of these sizes needs (0 if the
    sizes are invalid)."""
    return int(_lib.lib().dit_attn_workspace_bytes(B, S_q, H, D, n_qb, P))


def attn_partitioned(q, k, v, q_offsets, kv_offsets, recompute, cache_o, cache_lse, out, lse, *,
                     local_part=None, cache_valid=None, scale: float = 0.0, importance_out=None,
                     delta_out=None, workspace=None, stream=None) -> None:
    """One selective step: dit_attn_partitioned.  Tensors are device tensors in the
    layouts of include/dit_attn.h; offsets, mask, local_part and cache_valid are host
    sequences/arrays."""
    (B, S_q, S_kv, H, D), (qp, kp, vp) = _qkv(q, k, v)
    n_qb, P = len(q_offsets) - 1, len(kv_offsets) - 1
    wp, ws_bytes = _ws(workspace, "workspace")
    _check(_lib.lib().dit_attn_partitioned(
        qp, kp, vp, B, S_q, S_kv, H, D,
        _i32(q_offsets), n_qb, _i32(kv_offsets), P,
        None if local_part is None else _i32(local_part), _u8(recompute),
        None if cache_valid is None else _u8(cache_valid),
        _dev(cache_o, BF16, (P, B, S_q, H, D), "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"),
        _dev(out, BF16, (B, S_q, H, D), "out"), _dev(lse, F32, (B, H, S_q), "lse"), float(scale),
        _dev(importance_out, F32, (B, n_qb, P), "importance_out"), _dev(delta_out, F32, (B, n_qb), "delta_out"),
        wp, ws_bytes, _stream(stream)))


def attn_partitioned_noalloc(q, k, v, q_offsets, kv_offsets, recompute, cache_o, cache_lse, out, lse, *,
                             local_part=None, cache_valid=None, scale: float = 0.0, importance_out=None,
                             delta_out=None, stream=None) -> None:
    """dit_attn_partitioned_noalloc: attn_partitioned with the library's own device scratch
    in place of a workspace (for callers that cannot allocate)."""
    (B, S_q, S_kv, H, D), (qp, kp, vp) = _qkv(q, k, v)
    n_qb, P = len(q_offsets) - 1, len(kv_offsets) - 1
    _check(_lib.lib().dit_attn_partitioned_noalloc(
        qp, kp, vp, B, S_q, S_kv, H, D,
        _i32(q_offsets), n_qb, _i32(kv_offsets), P,
        None if local_part is None else _i32(local_part), _u8(recompute),
        None if cache_valid is None else _u8(cache_valid),
        _dev(cache_o, BF16, (P, B, S_q, H, D), "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"),
        _dev(out, BF16, (B, S_q, H, D), "out"), _dev(lse, F32, (B, H, S_q), "lse"), float(scale),
        _dev(importance_out, F32, (B, n_qb, P), "importance_out"), _dev(delta_out, F32, (B, n_qb), "delta_out"),
        _stream(stream)))


def partition_attention(q, k, v, q_offsets, kv_offsets, recompute, cache_o, cache_lse, *,
                        local_part=None, cache_valid=None, scale: float = 0.0, workspace=None,
                        stream=None) -> None:
    """dit_partition_attention.  With a workspace (and local_part) it also writes the
    local-change partial sums (finish them with local_change_finalize)."""
    (B, S_q, S_kv, H, D), (qp, kp, vp) = _qkv(q, k, v)
    n_qb, P = len(q_offsets) - 1, len(kv_offsets) - 1
    wp, ws_bytes = _ws(workspace, "workspace")
    _check(_lib.lib().dit_partition_attention(
        qp, kp, vp, B, S_q, S_kv, H, D, _i32(q_offsets), n_qb, _i32(kv_offsets), P,
        None if local_part is None else _i32(local_part), _u8(recompute),
        None if cache_valid is None else _u8(cache_valid),
        _dev(cache_o, BF16, (P, B, S_q, H, D), "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"),
        float(scale), wp, ws_bytes, _stream(stream)))


def partition_attention_premerge(q, k, v, q_offsets, kv_offsets, recompute, cache_o, cache_lse, pre_o, pre_lse, *,
                                 workspace, local_part=None, cache_valid=None, scale: float = 0.0,
                                 stream=None) -> None:
    """dit_partition_attention_premerge: partition_attention plus, in the same launch, the
    merge of each block's reused planes into pre_o / pre_lse.  With local_part it also
    writes the local-change partials into the workspace."""
    (B, S_q, S_kv, H, D), (qp, kp, vp) = _qkv(q, k, v)
    n_qb, P = len(q_offsets) - 1, len(kv_offsets) - 1
    wp, ws_bytes = _ws(workspace, "workspace")
    _check(_lib.lib().dit_partition_attention_premerge(
        qp, kp, vp, B, S_q, S_kv, H, D, _i32(q_offsets), n_qb, _i32(kv_offsets), P,
        None if local_part is None else _i32(local_part), _u8(recompute),
        None if cache_valid is None else _u8(cache_valid),
        _dev(cache_o, BF16, (P, B, S_q, H, D), "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"),
        float(scale), _dev(pre_o, BF16, (B, S_q, H, D), "pre_o"), _dev(pre_lse, F32, (B, H, S_q), "pre_lse"),
        wp, ws_bytes, _stream(stream)))


def partition_attention_fp8(q, k, v, q_offsets, kv_offsets, recompute, cache_q8, cache_scale, cache_lse, *,
                            local_part=None, cache_valid=None, scale: float = 0.0, workspace=None,
                            stream=None) -> None:
    """partition_attention into the compressed cache (cache_q8 uint8 e4m3 codes,
    cache_scale one f32 scale per partition, batch, row and head)."""
    (B, S_q, S_kv, H, D), (qp, kp, vp) = _qkv(q, k, v)
    n_qb, P = len(q_offsets) - 1, len(kv_offsets) - 1
    wp, ws_bytes = _ws(workspace, "workspace")
    _check(_lib.lib().dit_partition_attention_fp8(
        qp, kp, vp, B, S_q, S_kv, H, D, _i32(q_offsets), n_qb, _i32(kv_offsets), P,
        None if local_part is None else _i32(local_part), _u8(recompute),
        None if cache_valid is None else _u8(cache_valid),
        _dev(cache_q8, U8, (P, B, S_q, H, D), "cache_q8"), _dev(cache_scale, F32, (P, B, S_q, H), "cache_scale"),
        _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"), float(scale), wp, ws_bytes, _stream(stream)))


def _imp_args(q_offsets, importance_out, workspace, B, P):
    """q_offsets, n_qb, importance address, workspace address and bytes of a merge."""
    if importance_out is None:
        return None, 0, None, None, 0
    n_qb = len(q_offsets) - 1
    wp, ws_bytes = _ws(workspace, "workspace")
    return _i32(q_offsets), n_qb, _dev(importance_out, F32, (B, n_qb, P), "importance_out"), wp, ws_bytes


def state_merge_fp8(cache_q8, cache_scale, cache_lse, out, lse, *, q_offsets=None, importance_out=None,
                    workspace=None, stream=None) -> None:
    """Merge of the compressed cache; with importance_out (and q_offsets, workspace) also the
    partition importance in the same pass."""
    P, B, S_q, H, D = cache_q8.shape
    qo, n_qb, ip, wp, ws_bytes = _imp_args(q_offsets, importance_out, workspace, B, P)
    _check(_lib.lib().dit_state_merge_fp8(
        _dev(cache_q8, U8, None, "cache_q8"), _dev(cache_scale, F32, (P, B, S_q, H), "cache_scale"),
        _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"), B, S_q, H, D, P,
        _dev(out, BF16, (B, S_q, H, D), "out"), _dev(lse, F32, (B, H, S_q), "lse"), qo, n_qb, ip, wp, ws_bytes,
        _stream(stream)))


def state_merge(cache_o, cache_lse, out, lse, *, q_offsets=None, importance_out=None, workspace=None,
                stream=None) -> None:
    """Merge of the P cached states; with importance_out (and q_offsets, workspace) also the
    partition importance in the same pass."""
    P, B, S_q, H, D = cache_o.shape
    qo, n_qb, ip, wp, ws_bytes = _imp_args(q_offsets, importance_out, workspace, B, P)
    _check(_lib.lib().dit_state_merge(
        _dev(cache_o, BF16, None, "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"), B, S_q, H, D, P,
        _dev(out, BF16, (B, S_q, H, D), "out"), _dev(lse, F32, (B, H, S_q), "lse"), qo, n_qb, ip, wp, ws_bytes,
        _stream(stream)))


def state_merge_masked(cache_o, cache_lse, q_offsets, plane_select, out, lse, *, extra_o=None, extra_lse=None,
                       stream=None) -> None:
    """Merge, per query block, only the selected cache planes (plus an optional extra state)."""
    P, B, S_q, H, D = cache_o.shape
    _check(_lib.lib().dit_state_merge_masked(
        _dev(cache_o, BF16, None, "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"), B, S_q, H, D, P,
        _i32(q_offsets), len(q_offsets) - 1, _u8(plane_select),
        _dev(extra_o, BF16, (B, S_q, H, D), "extra_o"), _dev(extra_lse, F32, (B, H, S_q), "extra_lse"),
        _dev(out, BF16, (B, S_q, H, D), "out"), _dev(lse, F32, (B, H, S_q), "lse"), _stream(stream)))


def state_compose(cache_o, cache_lse, group_offsets, out_o, out_lse, *, stream=None) -> None:
    """Compose runs of adjacent cached partition states into coarser group states."""
    P, B, S_q, H, D = cache_o.shape
    G = len(group_offsets) - 1
    _check(_lib.lib().dit_state_compose(
        _dev(cache_o, BF16, None, "cache_o"), _dev(cache_lse, F32, (P, B, S_q, H), "cache_lse"), P,
        _i32(group_offsets), G, B, S_q, H, D,
        _dev(out_o, BF16, (G, B, S_q, H, D), "out_o"), _dev(out_lse, F32, (G, B, S_q, H), "out_lse"),
        _stream(stream)))


def importance(cache_lse, lse, q_offsets, importance_out, *, stream=None) -> None:
    """dit_importance: the partition importance [B, n_qb, P] from the cached lse planes and the
    merged lse, in a second pass (no workspace)."""
    P, B, S_q, H = cache_lse.shape
    n_qb = len(q_offsets) - 1
    _check(_lib.lib().dit_importance(
        _dev(cache_lse, F32, None, "cache_lse"), _dev(lse, F32, (B, H, S_q), "lse"), B, S_q, H, P,
        _i32(q_offsets), n_qb, _dev(importance_out, F32, (B, n_qb, P), "importance_out"), _stream(stream)))


def local_change_finalize(workspace, B, S_q, H, D, q_offsets, delta_out, *, stream=None) -> None:
    """dit_local_change_finalize: the local-state change [B, n_qb] from the partial sums the
    attention kernel left in the workspace."""
    wp, ws_bytes = _ws(workspace, "workspace")
    n_qb = len(q_offsets) - 1
    _check(_lib.lib().dit_local_change_finalize(wp, ws_bytes, B, S_q, H, D, _i32(q_offsets), n_qb,
                                                _dev(delta_out, F32, (B, n_qb), "delta_out"), _stream(stream)))


class Planner:
    """Host group planner (dit_planner_*)."""

    def __init__(self, n_qb: int, P: int, group_offsets: Sequence[int], local_part: Sequence[int],
                 anchor_every: int, recompute_groups: int, mode: str):
        self.n_qb, self.P, self.G = n_qb, P, len(group_offsets) - 1
        h = ctypes.c_void_p()
        _check(_lib.lib().dit_planner_create(n_qb, P, _i32(group_offsets), self.G, _i32(local_part),
                                             int(anchor_every), int(recompute_groups), MODES[mode],
                                             ctypes.byref(h)))
        self._h = h

    def next(self, step: int) -> Tuple[np.ndarray, List[List[int]]]:
        """The recompute mask [n_qb, P] of `step` and each block's chosen groups (local group
        first)."""
        mask = (ctypes.c_uint8 * (self.n_qb * self.P))()
        groups = (ctypes.c_int32 * (self.n_qb * self.G))()
        _check(_lib.lib().dit_planner_next(self._h, int(step), mask, groups))
        m = np.frombuffer(mask, dtype=np.uint8).reshape(self.n_qb, self.P).copy()
        g = np.frombuffer(groups, dtype=np.int32).reshape(self.n_qb, self.G)
        return m, [[int(x) for x in row if x >= 0] for row in g]

    def observe(self, step: int, importance=None, delta=None) -> None:
        """Feed the step's measurements: importance [n_qb, P] (anchor steps) and/or the local
        change [n_qb]."""
        def f32(a):
            if a is None:
                return None
            arr = np.ascontiguousarray(np.asarray(a, dtype=np.float32)).reshape(-1)
            return (ctypes.c_float * len(arr)).from_buffer_copy(arr.tobytes())
        _check(_lib.lib().dit_planner_observe(self._h, int(step), f32(importance), f32(delta)))

    def scores(self, step: int) -> np.ndarray:
        """The predicted reuse error [n_qb, G] that next(step) would rank the groups by."""
        out = (ctypes.c_double * (self.n_qb * self.G))()
        _check(_lib.lib().dit_planner_scores(self._h, int(step), out))
        return np.frombuffer(out, dtype=np.float64).reshape(self.n_qb, self.G).copy()

    def close(self) -> None:
        """Release the native planner (also done on garbage collection)."""
        if getattr(self, "_h", None) is not None and self._h.value:
            _lib.lib().dit_planner_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class SelectiveAttention:
    """Owns one layer's state cache on the GPU and runs selective steps.

    Keeps the per-slot validity bitmap that the C ABI checks (a slot becomes valid once
    its state has been computed) and the local-change workspace."""

    def __init__(self, B: int, S_q: int, S_kv: int, H: int, D: int, q_offsets: Sequence[int],
                 kv_offsets: Sequence[int], local_part: Sequence[int], device="cuda", cache_format="bf16"):
        """cache_format "bf16" keeps O_p in bfloat16; "fp8" keeps e4m3 codes plus one scale
        per (partition, batch, head, row) (about half the bytes; step() only)."""
        if cache_format not in ("bf16", "fp8"):
            raise ValueError(f"cache_format must be 'bf16' or 'fp8', got {cache_format!r}")
        self.B, self.S_q, self.S_kv, self.H, self.D = B, S_q, S_kv, H, D
        self.q_offsets, self.kv_offsets = list(q_offsets), list(kv_offsets)
        self.local_part = list(local_part)
        self.n_qb, self.P = len(q_offsets) - 1, len(kv_offsets) - 1
        self.cache_format = cache_format
        if cache_format == "fp8":
            self.cache_o = torch.empty((self.P, B, S_q, H, D), dtype=torch.uint8, device=device)
            self.cache_scale = torch.empty((self.P, B, S_q, H), dtype=torch.float32, device=device)
        else:
            self.cache_o = torch.empty((self.P, B, S_q, H, D), dtype=torch.bfloat16, device=device)
            self.cache_scale = None
        self.cache_lse = torch.empty((self.P, B, S_q, H), dtype=torch.float32, device=device)
        self.out = torch.empty((B, S_q, H, D), dtype=torch.bfloat16, device=device)
        self.lse = torch.empty((B, H, S_q), dtype=torch.float32, device=device)
        self.importance = torch.empty((B, self.n_qb, self.P), dtype=torch.float32, device=device)
        self.delta = torch.empty((B, self.n_qb), dtype=torch.float32, device=device)
        nb = workspace_bytes(B, S_q, H, D, self.n_qb, self.P)
        self.workspace = torch.empty(max(nb, 4) // 4, dtype=torch.float32, device=device)
        self.valid = np.zeros((self.n_qb, self.P), dtype=np.uint8)

    def step_overlapped(self, q, k, v, recompute, *, side_stream, want_delta=False, scale=0.0):
        """One selective step with the reuse work moved off the critical path: the reused
        states are pre-merged into a partial state on `side_stream` while the attention
        kernel recomputes the others on the current stream (the two touch disjoint cache
        slots); the current stream then merges the fresh states with the partial."""
        self._bf16_only("step_overlapped")
        recompute = np.asarray(recompute, dtype=np.uint8).reshape(self.n_qb, self.P)
        # the pre-merge of the reused planes is enqueued before the attention call validates
        # the mask, so the validity of those planes is checked here first
        if any(not self.valid[i, p] for i in range(self.n_qb) for p in range(self.P) if not recompute[i, p]):
            raise DitError(-5, status_string(-5))
        if not hasattr(self, "partial_o"):
            self.partial_o = torch.empty_like(self.out)
            self.partial_lse = torch.empty_like(self.lse)
        main = torch.cuda.current_stream()
        ready = torch.cuda.Event()
        ready.record(main)
        side_stream.wait_event(ready)
        state_merge_masked(self.cache_o, self.cache_lse, self.q_offsets, 1 - recompute, self.partial_o,
                           self.partial_lse, stream=side_stream)
        do_delta = want_delta and all(self.valid[i, self.local_part[i]] for i in range(self.n_qb))
        partition_attention(q, k, v, self.q_offsets, self.kv_offsets, recompute, self.cache_o, self.cache_lse,
                            local_part=self.local_part, cache_valid=self.valid, scale=scale,
                            workspace=self.workspace if do_delta else None, stream=main)
        done = torch.cuda.Event()
        done.record(side_stream)
        main.wait_event(done)
        state_merge_masked(self.cache_o, self.cache_lse, self.q_offsets, recompute, self.out, self.lse,
                           extra_o=self.partial_o, extra_lse=self.partial_lse, stream=main)
        if do_delta:
            local_change_finalize(self.workspace, self.B, self.S_q, self.H, self.D, self.q_offsets, self.delta,
                                  stream=main)
        self.valid |= recompute
        return do_delta

    def step_premerged(self, q, k, v, recompute, *, want_delta=False, scale=0.0, stream=None):
        """One selective step with the reuse work inside the attention launch: the launch's
        last workgroups pre-merge the reused states into a partial state in the slots that
        the attention work leaves as it drains, then the fresh states and the partial are
        merged (a two-state final combine per row-head, plus the fresh planes)."""
        self._bf16_only("step_premerged")
        recompute = np.asarray(recompute, dtype=np.uint8).reshape(self.n_qb, self.P)
        if not hasattr(self, "partial_o"):
            self.partial_o = torch.empty_like(self.out)
            self.partial_lse = torch.empty_like(self.lse)
        do_delta = want_delta and all(self.valid[i, self.local_part[i]] for i in range(self.n_qb))
        partition_attention_premerge(q, k, v, self.q_offsets, self.kv_offsets, recompute, self.cache_o,
                                     self.cache_lse, self.partial_o, self.partial_lse, workspace=self.workspace,
                                     local_part=self.local_part if do_delta else None, cache_valid=self.valid,
                                     scale=scale, stream=stream)
        state_merge_masked(self.cache_o, self.cache_lse, self.q_offsets, recompute, self.out, self.lse,
                           extra_o=self.partial_o, extra_lse=self.partial_lse, stream=stream)
        if do_delta:
            local_change_finalize(self.workspace, self.B, self.S_q, self.H, self.D, self.q_offsets, self.delta,
                                  stream=stream)
        self.valid |= recompute
        return do_delta

    def compose(self, group_offsets, stream=None) -> "SelectiveAttention":
        """Dynamic group compose: a new SelectiveAttention whose partitions are the groups
        (runs of adjacent partitions given by `group_offsets`) and whose cache holds the
        composed states; validity of a group = every member valid.  This object's cache
        is left unchanged (free it to reclaim the memory)."""
        self._bf16_only("compose")
        go = list(group_offsets)
        kvo = [self.kv_offsets[g] for g in go]
        local = [next(j for j in range(len(go) - 1) if go[j] <= lp < go[j + 1]) for lp in self.local_part]
        out = SelectiveAttention.__new__(SelectiveAttention)
        out.B, out.S_q, out.S_kv, out.H, out.D = self.B, self.S_q, self.S_kv, self.H, self.D
        out.q_offsets, out.kv_offsets, out.local_part = list(self.q_offsets), kvo, local
        out.n_qb, out.P = self.n_qb, len(go) - 1
        out.cache_format, out.cache_scale = "bf16", None
        dev = self.cache_o.device
        out.cache_o = torch.empty((out.P, self.B, self.S_q, self.H, self.D), dtype=torch.bfloat16, device=dev)
        out.cache_lse = torch.empty((out.P, self.B, self.S_q, self.H), dtype=torch.float32, device=dev)
        state_compose(self.cache_o, self.cache_lse, go, out.cache_o, out.cache_lse, stream=stream)
        out.out, out.lse = self.out, self.lse
        out.importance = torch.empty((self.B, out.n_qb, out.P), dtype=torch.float32, device=dev)
        out.delta = self.delta
        out.workspace = self.workspace     # fewer partitions: the workspace bound only shrinks
        out.valid = np.stack([self.valid[:, go[j]:go[j + 1]].all(axis=1) for j in range(out.P)], axis=1).astype(np.uint8)
        return out

    def _bf16_only(self, what: str) -> None:
        if self.cache_format != "bf16":
            raise DitError(-7, f"{what} needs the bf16 state cache")

    def step(self, q, k, v, recompute, *, want_importance=False, want_delta=False, scale=0.0, stream=None):
        """One selective step: the states of the (block, partition) pairs flagged in
        `recompute` are computed and written into the cache, the others are reused, and every
        block's states are merged into `out` / `lse`.  `want_importance` (anchor steps) fills
        `importance`; `want_delta` fills `delta` with the local-state change when every local
        slot already holds a state.  Returns whether `delta` was computed.  With the bf16 cache,
        a step that reuses states and asks for no importance merges the reused states inside
        the attention launch."""
        recompute = np.asarray(recompute, dtype=np.uint8).reshape(self.n_qb, self.P)
        local_valid = all(self.valid[i, self.local_part[i]] for i in range(self.n_qb))
        do_delta = want_delta and local_valid
        if self.cache_format == "fp8":
            partition_attention_fp8(q, k, v, self.q_offsets, self.kv_offsets, recompute, self.cache_o,
                                    self.cache_scale, self.cache_lse, local_part=self.local_part,
                                    cache_valid=self.valid, scale=scale,
                                    workspace=self.workspace if do_delta else None, stream=stream)
            state_merge_fp8(self.cache_o, self.cache_scale, self.cache_lse, self.out, self.lse,
                            q_offsets=self.q_offsets, importance_out=self.importance if want_importance else None,
                            workspace=self.workspace, stream=stream)
            if do_delta:
                local_change_finalize(self.workspace, self.B, self.S_q, self.H, self.D, self.q_offsets, self.delta,
                                      stream=stream)
            self.valid |= recompute
            return do_delta
        # the workspace always goes along: on a reuse step without importance the library merges
        # the reused states inside the attention launch (its chunk counter lives there)
        attn_partitioned(q, k, v, self.q_offsets, self.kv_offsets, recompute, self.cache_o, self.cache_lse,
                         self.out, self.lse, local_part=self.local_part, cache_valid=self.valid, scale=scale,
                         importance_out=self.importance if want_importance else None,
                         delta_out=self.delta if do_delta else None, workspace=self.workspace, stream=stream)
        self.valid |= recompute
        return do_delta
