"""fp64 CPU oracle of partitioned attention with selective state reuse.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package smoke check and the benchmark's
CPU-baseline leg may import this module; the product path never does.

What is computed follows the DiTango pages (gist.science 2607.15650, Portuguese and
Korean technical summaries):

* "Methodology §2, State Composition": attention over a KV partition yields an attention
  state, the pair (output, log-sum-exp); states compose associatively and commutatively,
  and the cache holds composed states instead of raw K/V.  The composition is the
  LSE-weighted combination (`merge_states`): the one associative, commutative rule under
  which the composition of all partition states equals softmax attention over their union.
* "Methodology §1": some partitions are computed from scratch, the others reuse the state
  from an earlier denoising step (`selective_step`); anchor steps recompute everything and
  refresh the partition importance w (`importance`); between anchors the change of the
  always-recomputed local state is the proxy for how states evolve (`local_change`).

Everything is plain numpy in float64 on exactly the bf16-rounded inputs (bf16 -> fp64 is
exact).  A matrix product is used as a library step; there is no tiling, online softmax
or fusion.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional, Sequence, Tuple

import numpy as np


def partition_state(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Attention state of queries q [n, H, D] over one KV partition k, v [m, H, D].

    Per head h and query r: s_j = scale * q_r . k_j; lse = ln sum_j e^{s_j};
    O = sum_j e^{s_j - lse} v_j.  Returns O [n, H, D] and lse [H, n].
    An empty partition has no state: lse = -inf and O = 0."""
    n, H, D = q.shape
    m = k.shape[0]
    O = np.zeros((n, H, D), dtype=np.float64)
    lse = np.full((H, n), -np.inf, dtype=np.float64)
    if m == 0 or n == 0:
        return O, lse
    for h in range(H):
        s = (q[:, h, :] @ k[:, h, :].T) * scale          # [n, m] scores
        mx = s.max(axis=1, keepdims=True)
        e = np.exp(s - mx)
        tot = e.sum(axis=1, keepdims=True)
        lse[h] = mx[:, 0] + np.log(tot[:, 0])
        O[:, h, :] = (e / tot) @ v[:, h, :]
    return O, lse


def full_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of q over all of k, v (one partition holding every key)."""
    return partition_state(q, k, v, scale)


def merge_states(Os: Sequence[np.ndarray], lses: Sequence[np.ndarray]) -> Tuple[np.ndarray, np.ndarray]:
    """Compose attention states by LSE-weighted combination, in the given order.

    Os[p]: [n, H, D]; lses[p]: [H, n].  Per row-head: M = max over finite lse_p,
    lse = M + ln sum_p e^{lse_p - M}, O = sum_p e^{lse_p - lse} O_p.
    States with lse = -inf (empty partitions) carry zero weight; if every state is empty
    the result is O = 0, lse = -inf."""
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])      # [P, H, n]
    fin = np.isfinite(L)
    M = np.where(fin, L, -np.inf).max(axis=0)                          # [H, n]
    any_state = np.isfinite(M)
    Ms = np.where(any_state, M, 0.0)
    W = np.where(fin, np.exp(np.where(fin, L, 0.0) - Ms[None]), 0.0)   # [P, H, n]
    tot = W.sum(axis=0)
    lse = np.where(any_state, Ms + np.log(np.where(any_state, tot, 1.0)), -np.inf)
    O = np.zeros_like(np.asarray(Os[0], dtype=np.float64))
    for p in range(len(Os)):
        coef = np.where(any_state, np.exp(np.where(fin[p], L[p], -np.inf) - np.where(any_state, lse, 0.0)), 0.0)
        O += coef.T[:, :, None] * np.asarray(Os[p], dtype=np.float64)
    return O, lse


def merge_weights(lses: Sequence[np.ndarray], lse: np.ndarray) -> np.ndarray:
    """Weight e^{lse_p - lse} of every state in a merge: [P, H, n]."""
    L = np.stack([np.asarray(x, dtype=np.float64) for x in lses])
    fin = np.isfinite(L) & np.isfinite(lse)[None]
    return np.where(fin, np.exp(np.where(fin, L - np.where(np.isfinite(lse), lse, 0.0)[None], -np.inf)), 0.0)


# --------------------------------------------------------------------------------------
# Rounding of stored states (the cache stores O in bfloat16 and lse in float32)
# --------------------------------------------------------------------------------------

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even), returned as float64.

    Done in two exact-by-construction stages: float64 -> float32 (numpy, round to nearest
    even), then float32 -> bfloat16 on the bit pattern.  The stored O in the state cache is
    bfloat16; this is the oracle's own rounding of it."""
    f = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    r = np.where(np.isfinite(f), r, u >> 16)      # inf stays inf (no rounding carry)
    return (r.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


FP8_MAX = 448.0   # largest finite OCP e4m3 value


def round_fp8_e4m3(x: np.ndarray) -> np.ndarray:
    """Round to the OCP fp8 e4m3 grid (1 sign, 4 exponent bits with bias 7, 3 mantissa bits;
    normals 2^-6 .. 448, subnormals k * 2^-9), nearest with ties to even.  Values above
    464 would round past 448 (the largest finite code) and are rejected.  Returned as
    float64."""
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.abs(x) > 464.0):
        raise ValueError("value beyond the e4m3 range")
    a = np.abs(x)
    # spacing of the grid at |x|: 2^(e-3) for normals (e = floor(log2 a) >= -6), 2^-9 below
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -6.0)
    ulp = np.exp2(e - 3.0)
    q = a / ulp
    r = np.floor(q)
    frac = q - r
    up = (frac > 0.5) | ((frac == 0.5) & (np.fmod(r, 2.0) == 1.0))
    r = r + up
    return np.sign(x) * r * ulp


def decode_fp8_e4m3(codes: np.ndarray) -> np.ndarray:
    """Value of OCP e4m3 codes (uint8) from the bit fields: sign (bit 7), exponent E (bits
    6..3, bias 7), mantissa M (bits 2..0); E = 0 gives M * 2^-9, E = 15 with M = 7 is NaN,
    otherwise (1 + M / 8) * 2^(E - 7).  Returned as float64."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    E = (c >> 3) & 15
    M = (c & 7).astype(np.float64)
    mag = np.where(E == 0, M * 2.0 ** -9, (1.0 + M / 8.0) * np.exp2(E - 7.0))
    mag = np.where((E == 15) & (M == 7), np.nan, mag)
    return sign * mag


def fp8_store(O: np.ndarray) -> np.ndarray:
    """The compressed cache's view of states O [..., D]: per (row, head) scale
    s = max_d |O| / 448 and e4m3 codes of O / s; returns the dequantized s * code."""
    amax = np.abs(O).max(axis=-1, keepdims=True)
    s = amax / FP8_MAX
    safe = np.where(s > 0, s, 1.0)
    return np.where(s > 0, round_fp8_e4m3(np.clip(O / safe, -FP8_MAX, FP8_MAX)) * safe, 0.0)


# --------------------------------------------------------------------------------------
# Selective step with a state cache
# --------------------------------------------------------------------------------------

@dataclasses.dataclass
class StateCache:
    """Cached attention state of every (query row, head, partition).

    O [P, n_rows, H, D] and lse [P, H, n_rows] for the rows the oracle tracks (all query
    rows, or a sample); `exact` holds fp64 states, `stored` the same states rounded the way
    the device cache stores them (O bfloat16, lse float32).  valid[i, p] says whether slot
    (query block i, partition p) has ever been computed."""
    rows: np.ndarray
    exact_O: np.ndarray
    exact_lse: np.ndarray
    stored_O: np.ndarray
    stored_lse: np.ndarray
    valid: np.ndarray

    @staticmethod
    def empty(rows: np.ndarray, P: int, H: int, D: int, n_qb: int) -> "StateCache":
        n = len(rows)
        return StateCache(rows=np.asarray(rows), exact_O=np.zeros((P, n, H, D)),
                          exact_lse=np.full((P, H, n), -np.inf), stored_O=np.zeros((P, n, H, D)),
                          stored_lse=np.full((P, H, n), -np.inf), valid=np.zeros((n_qb, P), dtype=bool))


@dataclasses.dataclass
class StepResult:
    O: np.ndarray            # [n_rows, H, D] merged output from exact states
    lse: np.ndarray          # [H, n_rows]
    O_stored: np.ndarray     # merged output from the stored (rounded) states
    lse_stored: np.ndarray
    weights: np.ndarray      # [P, H, n_rows] merge weights e^{lse_p - lse} (exact states)
    fresh_lse: np.ndarray    # [P, H, n_rows] lse of freshly computed states (-inf where reused)


def block_of_rows(rows: np.ndarray, q_offsets: Sequence[int]) -> np.ndarray:
    """Query block index of every query row."""
    return np.searchsorted(np.asarray(q_offsets), rows, side="right") - 1


def selective_step(q_rows: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray,
                   q_offsets: Sequence[int], kv_offsets: Sequence[int], mask: np.ndarray,
                   cache: StateCache, scale: float) -> StepResult:
    """One selective attention step for the query rows `rows` (q_rows [n, H, D] fp64).

    For every query block i and partition p: if mask[i, p] the state of (i, p) is computed
    from scratch and written into the cache; otherwise the cached state from the earlier
    step is used.  The output is the composition of all P states (DiTango pages,
    "Methodology §1 and §2")."""
    P = len(kv_offsets) - 1
    n, H, D = q_rows.shape
    blk = block_of_rows(rows, q_offsets)
    fresh_lse = np.full((P, H, n), -np.inf)
    for i in np.unique(blk):
        sel = np.nonzero(blk == i)[0]
        for p in range(P):
            if mask[i, p]:
                a, b = kv_offsets[p], kv_offsets[p + 1]
                O_ip, lse_ip = partition_state(q_rows[sel], k[a:b], v[a:b], scale)
                cache.exact_O[p, sel] = O_ip
                cache.exact_lse[p][:, sel] = lse_ip
                cache.stored_O[p, sel] = round_bf16(O_ip)
                cache.stored_lse[p][:, sel] = round_f32(lse_ip)
                fresh_lse[p][:, sel] = lse_ip
            elif not cache.valid[i, p]:
                raise ValueError(f"reuse of never-computed cache slot (block {i}, partition {p})")
    for i in np.unique(blk):
        cache.valid[i] |= mask[i].astype(bool)
    O, lse = merge_states(list(cache.exact_O), list(cache.exact_lse))
    O_s, lse_s = merge_states(list(cache.stored_O), list(cache.stored_lse))
    W = merge_weights(list(cache.exact_lse), lse)
    return StepResult(O=O, lse=lse, O_stored=O_s, lse_stored=lse_s, weights=W, fresh_lse=fresh_lse)


def compose_states(O: np.ndarray, lse: np.ndarray, group_offsets: Sequence[int]) -> Tuple[np.ndarray, np.ndarray]:
    """Dynamic Group Compose (DiTango pages, "Methodology §2, Dynamic Group Compose"): the
    cached states of each run of adjacent partitions [g_j, g_{j+1}) are composed into one
    coarser state, with no recomputation.  O: [P, n, H, D], lse: [P, H, n] ->
    [G, n, H, D], [G, H, n]; each output is `merge_states` of its members, in order."""
    G = len(group_offsets) - 1
    outO, outL = [], []
    for j in range(G):
        a, b = group_offsets[j], group_offsets[j + 1]
        Oj, Lj = merge_states(list(O[a:b]), list(lse[a:b]))
        outO.append(Oj)
        outL.append(Lj)
    return np.stack(outO), np.stack(outL)


def importance(weights: np.ndarray, rows: np.ndarray, q_offsets: Sequence[int]) -> np.ndarray:
    """Partition importance w[i, p] = mean over rows r of block i and heads h of the merge
    weight e^{lse_p - lse} (DiTango pages, "Methodology §1, Error Modeling / Anchor Steps":
    anchor steps refresh the partition importance).  weights: [P, H, n_rows]."""
    blk = block_of_rows(rows, q_offsets)
    n_qb = len(q_offsets) - 1
    P = weights.shape[0]
    w = np.zeros((n_qb, P))
    for i in range(n_qb):
        sel = blk == i
        if sel.any():
            w[i] = weights[:, :, sel].mean(axis=(1, 2))
    return w


def local_change(O_new: np.ndarray, O_old: np.ndarray, rows: np.ndarray, q_offsets: Sequence[int]) -> np.ndarray:
    """delta_i = ||O_new - O_old||_F / ||O_old||_F over block i's rows, all heads and D,
    where O is the block's local-partition state (DiTango pages, "Methodology §1, Online
    Prediction": the change of the always-recomputed local state stands in for how the
    other states evolve).  O_*: [n_rows, H, D]."""
    blk = block_of_rows(rows, q_offsets)
    n_qb = len(q_offsets) - 1
    d = np.full(n_qb, np.nan)
    for i in range(n_qb):
        sel = blk == i
        if sel.any():
            num = np.sqrt(np.sum((O_new[sel] - O_old[sel]) ** 2))
            den = np.sqrt(np.sum(O_old[sel] ** 2))
            d[i] = num / den
    return d
