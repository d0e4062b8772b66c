"""Shared helpers of the GPU parity tests: run one workload through the HIP path (via the
C ABI binding) and through the fp64 oracle on the same seeded inputs, and compare.

Tolerances (fixed by the target of the path): merged bf16 output max |err| <= 1e-2 and
lse max |err| <= 1e-3 (fp32 accumulation); in addition the relative Frobenius error of the
output must stay <= 1e-2, which is the meaningful bound at long sequence lengths where
|O| itself is far below 1e-2, and every output element must lie within 2^-6 of its row's
largest magnitude (row = one query row and head, over D) of the oracle's value.  That bound
is derived from the arithmetic: the output is rounded to bf16 (half an ulp is 2^-9
relative), each cached state to bf16 on both sides, where the two roundings can differ by
one ulp (2^-8 relative) of a state of at most the row's magnitude, and the bf16
probabilities of the P V product add 2^-9 relative per term; 2^-6 leaves a factor of about
two over their sum.  Unlike the absolute 1e-2, it scales with |O| and so bites at every
sequence length: a mis-masked tail or a wrong partition in a few rows fails it.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np
import torch

import oracle
import workloads as W
from partitioned_state_reuse_amd import api

O_ABS_TOL = 1e-2
LSE_ABS_TOL = 1e-3
O_REL_FRO_TOL = 1e-2
O_ROW_REL_TOL = 2.0 ** -6
O_ROW_ABS_FLOOR = 1e-6
# importance is a mean of merge weights in [0, 1]; delta a ratio of norms of bf16 states
IMP_ABS_TOL = 1e-4
DELTA_REL_TOL = 2e-2


def to_dev(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_to_f64(t: torch.Tensor) -> np.ndarray:
    return W.to_f64(t.detach().view(torch.int16).cpu().numpy().view(np.uint16))


def masks_from_planners(w: W.Workload, step: int = 0):
    """Mask of the host C++ planner and of the oracle planner (must agree)."""
    cp = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every or 0, w.recompute_groups, w.mode)
    rp = oracle.RefPlanner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every or 0, w.recompute_groups, w.mode)
    m1, c1 = cp.next(step)
    m2, c2 = rp.next(step)
    cp.close()
    return m1, m2, c1, c2


def row_bound(ref: np.ndarray) -> np.ndarray:
    """Per-element bound 2^-6 max_d |ref[r, h, :]| + 1e-6 for outputs ref [n, H, D]."""
    return O_ROW_REL_TOL * np.abs(ref).max(axis=-1, keepdims=True) + O_ROW_ABS_FLOOR


def assert_rows_close(got: np.ndarray, ref: np.ndarray, what: str = "") -> float:
    """Element-wise O check of states or outputs [..., H, D]: the absolute 1e-2 of the target
    and the row-scaled bound; returns the largest ratio to the row bound."""
    d = np.abs(got - ref)
    ratio = float((d / row_bound(ref)).max()) if d.size else 0.0
    assert d.max() <= O_ABS_TOL, f"{what}: max|dO| {d.max():.3e}"
    assert ratio <= 1.0, f"{what}: {int((d > row_bound(ref)).sum())} elements beyond the row bound (ratio {ratio:.3f})"
    return ratio


@dataclasses.dataclass
class Compare:
    o_abs: float
    o_rel_fro: float
    lse_abs: float
    o_abs_exact: float
    o_row_ratio: float        # max over elements of |dO| / row_bound(O_ref)

    def ok(self) -> bool:
        return (self.o_abs <= O_ABS_TOL and self.lse_abs <= LSE_ABS_TOL and self.o_rel_fro <= O_REL_FRO_TOL
                and self.o_row_ratio <= 1.0)

    def __str__(self):
        return (f"max|dO|={self.o_abs:.3e} (vs exact states {self.o_abs_exact:.3e}) "
                f"relF={self.o_rel_fro:.3e} max|dlse|={self.lse_abs:.3e} row-bound ratio={self.o_row_ratio:.3f}")


def compare_out(gpu_O: np.ndarray, gpu_lse: np.ndarray, res: oracle.StepResult) -> Compare:
    """gpu_O [n, H, D], gpu_lse [H, n] against the oracle's merged result on the same rows."""
    ref = res.O_stored
    fin = np.isfinite(res.lse_stored)
    dl = np.abs(np.where(fin, gpu_lse - res.lse_stored, 0.0))
    assert np.array_equal(np.isfinite(gpu_lse), fin), "lse finiteness differs"
    dO = np.abs(gpu_O - ref)
    return Compare(o_abs=float(dO.max()),
                   o_rel_fro=float(np.linalg.norm(gpu_O - ref) / max(np.linalg.norm(ref), 1e-300)),
                   lse_abs=float(dl.max()) if dl.size else 0.0,
                   o_abs_exact=float(np.abs(gpu_O - res.O).max()),
                   o_row_ratio=float((dO / row_bound(ref)).max()))


class GpuRun:
    """HIP path state for one workload: the SelectiveAttention cache plus helpers."""

    def __init__(self, w: W.Workload, q_offsets=None, kv_offsets=None, local_part=None, B=1):
        self.w = w
        self.qo = list(q_offsets if q_offsets is not None else w.q_offsets)
        self.ko = list(kv_offsets if kv_offsets is not None else w.kv_offsets)
        self.local = list(local_part if local_part is not None else w.local_part)
        self.sa = api.SelectiveAttention(B, self.qo[-1], self.ko[-1], w.H, w.D, self.qo, self.ko, self.local)

    def step(self, X: W.StepInputs, mask, want_importance=False, want_delta=False):
        q, k, v = to_dev(X.q), to_dev(X.k), to_dev(X.v)
        did_delta = self.sa.step(q, k, v, mask, want_importance=want_importance, want_delta=want_delta)
        torch.cuda.synchronize()
        return did_delta

    def out_rows(self, rows) -> np.ndarray:
        return bf16_to_f64(self.sa.out[0, torch.as_tensor(rows, device="cuda")])

    def lse_rows(self, rows) -> np.ndarray:
        return self.sa.lse[0][:, torch.as_tensor(rows, device="cuda")].double().cpu().numpy()

    def cache_lse_rows(self, rows) -> np.ndarray:
        """Cached lse of the rows as [P, H, n] (the oracle's layout; the device keeps [P, B, S_q, H])."""
        a = self.sa.cache_lse[:, 0][:, torch.as_tensor(rows, device="cuda"), :].double().cpu().numpy()
        return np.ascontiguousarray(np.transpose(a, (0, 2, 1)))

    def cache_o_rows(self, rows) -> np.ndarray:
        return bf16_to_f64(self.sa.cache_o[:, 0][:, torch.as_tensor(rows, device="cuda")])


class OracleRun:
    """Oracle state for the same workload on a set of query rows."""

    def __init__(self, w: W.Workload, rows: np.ndarray, q_offsets=None, kv_offsets=None, local_part=None):
        self.w = w
        self.rows = np.asarray(rows)
        self.qo = list(q_offsets if q_offsets is not None else w.q_offsets)
        self.ko = list(kv_offsets if kv_offsets is not None else w.kv_offsets)
        self.local = list(local_part if local_part is not None else w.local_part)
        self.cache = oracle.StateCache.empty(self.rows, len(self.ko) - 1, w.H, w.D, len(self.qo) - 1)
        self.scale = 1.0 / math.sqrt(w.D)

    def local_states(self, which="stored") -> np.ndarray:
        blk = oracle.block_of_rows(self.rows, self.qo)
        O = self.cache.stored_O if which == "stored" else self.cache.exact_O
        return np.stack([O[self.local[b], j] for j, b in enumerate(blk)])

    def step(self, X: W.StepInputs, mask) -> oracle.StepResult:
        q = W.to_f64(X.q[0][self.rows] if X.q.shape[1] != len(self.rows) else X.q[0])
        k, v = W.to_f64(X.k[0]), W.to_f64(X.v[0])
        return oracle.selective_step(q, k, v, self.rows, self.qo, self.ko, np.asarray(mask), self.cache, self.scale)
