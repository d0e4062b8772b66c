"""Reference group planner (pure Python, float64).  TEST INFRASTRUCTURE ONLY.

Follows the Anchor-Guided Selection Planner of the DiTango pages (gist.science
2607.15650, "Methodology §1" / "방법론 §1"):

* Anchor steps: every `anchor_every` steps all partitions are recomputed; this resets the
  accumulated error and refreshes the partition importance w.
* Error model: the error of reusing a state is a function of the partition's importance w
  and the temporal error growth delta.  Reading taken here: the predicted error of reusing
  group g for query block i at step t is
      e_ig = w_ig * sum_{tau = last_ig + 1 .. t} dhat_i(tau),
  with w_ig the sum of the member partitions' importance and last_ig the step at which the
  group was last recomputed.
* Online prediction: delta is observed only for the always-recomputed local state;
  dhat_i(tau) = delta_i(tau) for observed steps; the not-yet-observed current step (or a
  step whose delta was not observed) takes the latest value observed before it, and 1.0
  before any observation.
* Group strategy: decisions are per group of adjacent partitions; the local group is always
  recomputed and the other recomputed groups are the K-1 with the largest e_ig, ties going
  to the smaller partition-index distance, then the lower group index.

Distance mode (fixed selection by distance to the query block) orders the other groups by
(distance, index) only.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np


def group_of(group_offsets: Sequence[int], p: int) -> int:
    for g in range(len(group_offsets) - 1):
        if group_offsets[g] <= p < group_offsets[g + 1]:
            return g
    raise ValueError(f"partition {p} is in no group")


def group_distance(group_offsets: Sequence[int], g: int, local_p: int) -> int:
    """min over member partitions p of |p - local_p|."""
    return min(abs(p - local_p) for p in range(group_offsets[g], group_offsets[g + 1]))


class RefPlanner:
    def __init__(self, n_qb: int, P: int, group_offsets: Sequence[int], local_part: Sequence[int],
                 anchor_every: int, recompute_groups: int, mode: str):
        assert mode in ("wdelta", "distance", "anchor")
        self.n_qb, self.P = n_qb, P
        self.go = list(group_offsets)
        self.G = len(self.go) - 1
        self.local = list(local_part)
        self.anchor_every = anchor_every
        self.K = recompute_groups
        self.mode = mode
        self.w = [[0.0] * self.G for _ in range(n_qb)]        # group importance
        self.last = [[-1] * self.G for _ in range(n_qb)]      # step of last recompute
        self.delta: List[Dict[int, float]] = [dict() for _ in range(n_qb)]

    def is_anchor(self, step: int) -> bool:
        if self.mode == "anchor":
            return True
        if self.mode == "distance":
            return False
        return self.anchor_every > 0 and step % self.anchor_every == 0

    def _dhat(self, i: int, tau: int, step: int) -> float:
        """Observed delta of step tau, else (the current step, or a step whose delta was
        not observed) the latest delta observed before tau, else 1.0."""
        if tau < step and tau in self.delta[i]:
            return self.delta[i][tau]
        prev = [t for t in self.delta[i] if t < tau]
        return self.delta[i][max(prev)] if prev else 1.0

    def scores(self, step: int) -> List[List[float]]:
        """e_ig for every block and group at `step` (fp64)."""
        e = []
        for i in range(self.n_qb):
            row = []
            for g in range(self.G):
                acc = 0.0
                for tau in range(self.last[i][g] + 1, step + 1):
                    acc += self._dhat(i, tau, step)
                row.append(self.w[i][g] * acc)
            e.append(row)
        return e

    def next(self, step: int) -> Tuple[np.ndarray, List[List[int]]]:
        """Recompute mask [n_qb, P] (uint8) and the chosen groups per block
        (local group first, then in rank order)."""
        mask = np.zeros((self.n_qb, self.P), dtype=np.uint8)
        chosen: List[List[int]] = []
        anchor = self.is_anchor(step)
        e = self.scores(step) if (self.mode == "wdelta" and not anchor) else None
        for i in range(self.n_qb):
            lg = group_of(self.go, self.local[i])
            if anchor:
                gs = [lg] + [g for g in range(self.G) if g != lg]
            else:
                others = [g for g in range(self.G) if g != lg]
                if self.mode == "wdelta":
                    key = lambda g: (-e[i][g], group_distance(self.go, g, self.local[i]), g)
                else:
                    key = lambda g: (group_distance(self.go, g, self.local[i]), g)
                others.sort(key=key)
                gs = [lg] + others[:max(0, self.K - 1)]
            for g in gs:
                mask[i, self.go[g]:self.go[g + 1]] = 1
                self.last[i][g] = step
            chosen.append(gs)
        return mask, chosen

    def observe(self, step: int, importance: Optional[np.ndarray] = None,
                delta: Optional[np.ndarray] = None) -> None:
        """Feed the step's partition importance [n_qb, P] (anchor steps) and local change
        delta [n_qb] (float32 values as produced by the device, widened to fp64)."""
        if importance is not None:
            imp = np.asarray(importance, dtype=np.float32)
            for i in range(self.n_qb):
                for g in range(self.G):
                    acc = 0.0
                    for p in range(self.go[g], self.go[g + 1]):
                        acc += float(imp[i, p])
                    self.w[i][g] = acc
        if delta is not None:
            d = np.asarray(delta, dtype=np.float32)
            for i in range(self.n_qb):
                if np.isfinite(d[i]):
                    self.delta[i][step] = float(d[i])
