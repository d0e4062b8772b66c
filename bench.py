"""Benchmark of the selective attention step on one MI355X.

Workload (default): the 720p video layer, S = 75,600 tokens (21x45x80 latent grid, 3D
RoPE), H = 40, D = 128, bf16, P = 16 KV partitions, 16 query blocks, groups of two
adjacent partitions, 4 of 8 groups recomputed per query block by distance.  The state
cache is filled beforehand by an all-recompute step on the previous step's inputs
(X_prev = X - 0.05 N(0,1)).

One step = the whole hot path on one batch: host planner decision and work list, partition
attention with the cache update and the local-change partial sums, state merge, and the
local-change reduction.  Inputs are resident in HBM before the timed region.

Prints one JSON line.  `value` = recomputed-attention FLOP per step / step wall time.
`roofline` = the partition-attention kernel against bf16 dense MFMA peak; `roofline_merge`
= the merge kernel against HBM peak; both from HIP events on the launch stream.
`cpu_baseline` = the fp64 oracle timed on a bounded row sample of the same step.
"""
from __future__ import annotations

import argparse
import json
import re
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as W  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attn_flop(w: W.Workload, mask: np.ndarray) -> float:
    """4 D H sum over recomputed (block i, partition p) of |i| |p|  (QK^T and PV)."""
    qs = np.diff(w.q_offsets)
    ks = np.diff(w.kv_offsets)
    return float(4 * w.D * w.H * np.sum(mask * np.outer(qs, ks)))


def merge_bytes(w: W.Workload) -> float:
    """S_q H [P (2D + 4) + (2D + 4)]: read every state (bf16 O, f32 lse) once, write O and lse."""
    return float(w.S_q * w.H * (w.P * (2 * w.D + 4) + (2 * w.D + 4)))


def kernel_source_sha256() -> str:
    import hashlib
    d = os.path.join(ROOT, "partitioned_state_reuse_amd", "csrc")
    return hashlib.sha256(b"".join(open(os.path.join(d, f), "rb").read() for f in ("kernels.hip", "launch.h"))).hexdigest()


def measured_counters(workload: str, kernel: str) -> dict:
    """Counter-derived figures of an attention launch (clock under load, MFMA busy fraction)
    from the committed rocprofv3 summary of this workload; empty when the kernel sources
    changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_source_sha256():
        return {}
    for key in ("attention_counters", "plain_attention_counters"):
        c = rec.get(key, {})
        if c.get("kernel") == "dit::" + kernel:
            return c
    return {}


def measured_power(workload: str) -> dict:
    """Steady-state socket power and graphics clock of the attention kernel, of the merge and of
    the whole step (one call, plain sequence) from the committed power trace of this workload
    (bench.py --power-trace); empty when the kernel sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"power_{workload}.txt")
    if not os.path.exists(path):
        return {}
    text = open(path).read()
    m = re.search(r"^# source_sha256 ([0-9a-f]+)$", text, flags=re.M)
    if not m or m.group(1) != kernel_source_sha256():
        return {}
    out = {"source": f"profiles/power_{workload}.txt"}
    for name in ("attention", "merge", "one_call", "plain_step"):
        r = re.search(rf"^# {name} steady state \((\d+) samples\): socket power (\d+) W, gfx clock per XCD ([\d ]+) MHz "
                      rf"\(mean (\d+)\)", text, flags=re.M)
        if r:
            out[name] = {"socket_w": int(r.group(2)), "gfx_mhz_per_xcd": [int(x) for x in r.group(3).split()],
                         "gfx_mhz_mean": int(r.group(4))}
    return out


def measured_traffic(workload: str) -> dict:
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE / WRITE_SIZE summary of this
    workload, scaled by the copy-kernel calibration; empty when the kernel sources changed since
    the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return {}
    rec = json.load(open(path))
    if rec.get("source_sha256") != kernel_source_sha256():
        return {}
    return {k: v["traffic_bytes"] for k, v in rec.get("kernels", {}).items()}


def summarize_profile(db_path: str) -> str:
    """Text summary of a rocprofv3 kernel trace (rocpd SQLite output): per kernel and grid
    size, the dispatch count and the mean / min / max duration.  Grouping by grid separates
    the cache-filling all-recompute dispatch from the timed steps' dispatches."""
    import sqlite3
    con = sqlite3.connect(db_path)
    rows = con.execute("select name, grid_x, grid_y, grid_z, workgroup_x, vgpr_count, accum_vgpr_count, "
                       "lds_size, duration from kernels").fetchall()
    groups = {}
    for name, gx, gy, gz, wx, vg, ag, lds, dur in rows:
        short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
        key = (short, gx, gy, gz, wx, vg, ag, lds)
        groups.setdefault(key, []).append(dur)
    lines = [f"{'kernel':<48} {'grid(x,y,z)':>22} {'wg':>4} {'vgpr':>5} {'agpr':>5} {'lds':>6} {'calls':>5} "
             f"{'mean_us':>11} {'min_us':>11} {'max_us':>11}"]
    for key, durs in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        short, gx, gy, gz, wx, vg, ag, lds = key
        d = np.array(durs, dtype=np.float64) / 1e3
        lines.append(f"{short[:48]:<48} {f'{gx},{gy},{gz}':>22} {wx:>4} {vg:>5} {ag:>5} {lds:>6} {len(d):>5} "
                     f"{d.mean():>11.2f} {d.min():>11.2f} {d.max():>11.2f}")
    # two-stream steps: how long each masked merge ran alongside an attention dispatch
    try:
        disp = con.execute("select name, start, end from kernels order by start").fetchall()
    except Exception:
        disp = []
    attn = [(a, b) for n, a, b in disp if "partition_attention" in n]
    masked = [(a, b) for n, a, b in disp if "state_merge_masked_kernel" in n]
    if attn and masked:
        lines.append("")
        lines.append("# masked merges (two-stream and pre-merged steps) against the attention dispatches they overlap (us):")
        lines.append(f"{'merge start':>12} {'merge dur':>10} {'overlap':>10} {'attn start':>12} {'attn dur':>10}")
        t0 = min(a for a, _ in attn + masked)
        for a, b in masked:
            best = max(attn, key=lambda ab: max(0, min(b, ab[1]) - max(a, ab[0])))
            ov = max(0, min(b, best[1]) - max(a, best[0]))
            if ov == 0:   # no overlap: the attention dispatch this merge follows
                best = max((ab for ab in attn if ab[1] <= a), key=lambda ab: ab[1], default=best)
            lines.append(f"{(a - t0) / 1e3:>12.1f} {(b - a) / 1e3:>10.1f} {ov / 1e3:>10.1f} {(best[0] - t0) / 1e3:>12.1f} "
                         f"{(best[1] - best[0]) / 1e3:>10.1f}")
    return "\n".join(lines)


def read_pmc(dirpath: str) -> dict:
    """Per (kernel, grid size) from a rocprofv3 --pmc CSV run: {counter: [value per dispatch]}
    and the dispatch durations in ns."""
    import csv
    import glob
    files = glob.glob(os.path.join(dirpath, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise FileNotFoundError(f"no *counter_collection.csv under {dirpath}")
    out = {}
    for fn in files:
        with open(fn) as f:
            for row in csv.DictReader(f):
                name = row["Kernel_Name"].replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
                key = (name, int(row["Grid_Size"]))
                d = out.setdefault(key, {"dispatch": {}})
                disp = d["dispatch"].setdefault(row["Dispatch_Id"], {})
                disp[row["Counter_Name"]] = disp.get(row["Counter_Name"], 0.0) + float(row["Counter_Value"])
                disp["_ns"] = float(row["End_Timestamp"]) - float(row["Start_Timestamp"])
    return out


def pmc_mean(rec: dict, counter: str) -> float:
    vals = [d[counter] for d in rec["dispatch"].values() if counter in d]
    return float(np.mean(vals)) if vals else float("nan")


def summarize_pmc(workload: str, out_json: str, fetch_dir: str, write_dir: str, sq_dirs: list) -> str:
    """HBM traffic per launch of every kernel of one workload's steps from FETCH_SIZE and
    WRITE_SIZE runs, scaled by the same counters' reading for the 4 GiB device copy of the
    bench (bytes known), plus the attention kernel's SQ-counter figures; writes the record the
    bench reads (profiles/traffic_<workload>.json) and returns a text summary."""
    from partitioned_state_reuse_amd import api
    w = W.workload(workload)
    mode = "anchor" if w.mode == "anchor" else "distance"
    pl = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every or 0, w.recompute_groups, mode)
    mask, _ = pl.next(1)
    pl.close()
    qt = [math.ceil(n / 128) for n in np.diff(w.q_offsets)]
    attn_grid = w.H * int(sum(qt[i] for i in range(w.n_qb) for p in range(w.P) if mask[i, p])) * 256
    merge_grid = math.ceil(w.S_q * w.H / 16) * 256
    # grids (threads) of this workload's launches: merges (bf16 16 and fp8 32 row-heads per
    # workgroup, per-block placement with importance partials), the reductions
    qb_sizes = np.diff(w.q_offsets)
    grids = {merge_grid, math.ceil(w.S_q * w.H / 32) * 256,
             int(sum(math.ceil(n * w.H / 16) for n in qb_sizes)) * 256,
             int(sum(math.ceil(n * w.H / 32) for n in qb_sizes)) * 256,
             w.n_qb * w.P * 1024, w.n_qb * w.P * 256, w.n_qb * 256}
    fetch, write = read_pmc(fetch_dir), read_pmc(write_dir)
    copy_bytes = 1 << 32

    def copy_reading(runs, counter):
        # the bench's 4 GiB device copy runs four times with identical readings; the other
        # copies of a run (cache clones, uploads, sampled-row gathers) are smaller: take the
        # largest value that occurs at least three times (within 0.1%)
        vals = sorted(d[counter] for (n, _), r in runs.items() if "copyBuffer" in n
                      for d in r["dispatch"].values() if counter in d)
        groups = []
        for x in vals:
            if groups and abs(x - groups[-1][0]) <= 1e-3 * groups[-1][0]:
                groups[-1].append(x)
            else:
                groups.append([x])
        best = max((g for g in groups if len(g) >= 3), key=lambda g: g[0])
        return float(np.mean(best)), len(best)

    (fetch_copy, nf), (write_copy, nw) = copy_reading(fetch, "FETCH_SIZE"), copy_reading(write, "WRITE_SIZE")
    rf, wf = copy_bytes / (fetch_copy * 1024), copy_bytes / (write_copy * 1024)
    kernels = {}
    for (name, grid), rec in fetch.items():
        if "copyBuffer" in name or (name, grid) not in write:
            continue
        # the attention launch, the one with the reuse pre-merge in its tail (at most 4,096
        # more workgroups), the merges and reductions
        if not ((name.startswith("dit::partition_attention_kernel") and grid == attn_grid) or
                (name.startswith("dit::partition_attention_premerge") and attn_grid < grid <= attn_grid + (1 << 20)) or
                (not name.startswith("dit::partition_attention") and grid in grids)):
            continue
        fk, wk = pmc_mean(rec, "FETCH_SIZE"), pmc_mean(write[(name, grid)], "WRITE_SIZE")
        kernels[name if name not in kernels else f"{name} grid {grid}"] = {"grid_threads": grid, "fetch_kib": fk, "write_kib": wk,
                              "hbm_read_bytes": fk * 1024 * rf, "hbm_write_bytes": wk * 1024 * wf,
                              "traffic_bytes": fk * 1024 * rf + wk * 1024 * wf,
                              "dispatches": len(rec["dispatch"])}
    rec = {"workload": workload, "source_sha256": kernel_source_sha256(),
           "command": f"rocprofv3 --pmc FETCH_SIZE -d {fetch_dir} -o run --output-format csv -- python3 -u bench.py "
                      f"--steps 2 --warmup 0 --no-cpu-baseline (then the same with WRITE_SIZE)",
           "calibration": {"kernel": "__amd_rocclr_copyBuffer (the 4 GiB device copy in bench.py)",
                           "bytes_read": copy_bytes, "bytes_written": copy_bytes, "fetch_kib": fetch_copy,
                           "write_kib": write_copy, "read_factor": rf, "write_factor": wf},
           "kernels": kernels}
    lines = [f"# HBM traffic per launch, {workload} (attention grid {attn_grid} threads, merge grid {merge_grid})",
             f"# calibration: the 4 GiB device copy ({nf} and {nw} dispatches) reads FETCH_SIZE {fetch_copy:.0f} KiB and "
             f"WRITE_SIZE {write_copy:.0f} KiB -> read factor {rf:.4f}, write factor {wf:.4f}"]
    for n, k in kernels.items():
        lines.append(f"#   {n:<46} FETCH {k['fetch_kib']:>12.0f} KiB x {rf:.4f} = {k['hbm_read_bytes'] / 1e9:8.3f} GB read, "
                     f"WRITE {k['write_kib']:>12.0f} KiB x {wf:.4f} = {k['hbm_write_bytes'] / 1e9:8.3f} GB written")
    if sq_dirs:
        def sq_of(match):
            sq = {}
            for dpath in sq_dirs:
                for key, r in read_pmc(dpath).items():
                    if match(*key):
                        for c in {c for d in r["dispatch"].values() for c in d if not c.startswith("_")}:
                            sq[c] = pmc_mean(r, c)
                        sq["_ns"] = pmc_mean(r, "_ns")
            return sq

        def figures(kernel, sq):
            clocks = sq["GRBM_GUI_ACTIVE"] / 8
            ghz = clocks / sq["_ns"]
            busy = sq["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * clocks)
            counters = {"kernel": kernel, "clock_ghz_under_load": round(ghz, 3),
                        "mfma_busy_frac": round(busy, 4), "peak_tflops_at_that_clock": round(PEAK_BF16_TFLOPS * ghz / 2.4, 1),
                        "commands": "rocprofv3 --pmc <SQ counters> -- python3 -u bench.py --steps 2 --warmup 0 "
                                    "--no-cpu-baseline (two passes)"}
            if "SQ_WAIT_ANY" in sq:
                counters["waves_waiting_frac"] = round(sq["SQ_WAIT_ANY"] / sq["SQ_WAVE_CYCLES"], 4)
            if "SQ_LDS_IDX_ACTIVE" in sq:
                counters["lds_indexed_active_frac"] = round(sq["SQ_LDS_IDX_ACTIVE"] / (256 * clocks), 4)
            if "SQ_VALU_MFMA_COEXEC_CYCLES" in sq:
                counters["mfma_valu_coexec_frac"] = round(sq["SQ_VALU_MFMA_COEXEC_CYCLES"] / (1024 * clocks), 4)
            if "SQ_INSTS_VALU" in sq:
                counters["valu_instructions_per_mfma"] = round(sq["SQ_INSTS_VALU"] / sq["SQ_INSTS_MFMA"], 3)
            if "TCC_HIT_sum" in sq:
                counters["l2_hit_frac"] = round(sq["TCC_HIT_sum"] / (sq["TCC_HIT_sum"] + sq["TCC_MISS_sum"]), 4)
            lines.append(f"# SQ counters of {kernel} (mean over its dispatches of this workload):")
            for c in sorted(k for k in sq if not k.startswith("_")):
                lines.append(f"#   {c:<28} {sq[c]:.4e}")
            lines.append(f"#   dispatch duration under the counters {sq['_ns'] / 1e6:.2f} ms; GRBM_GUI_ACTIVE / 8 XCDs = "
                         f"{clocks:.4e} clocks -> {ghz:.2f} GHz; MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x clocks)"
                         f" = {busy:.1%}")
            for k, v in counters.items():
                if k.endswith("_frac") or k.endswith("_per_mfma") or k.endswith("_ghz_under_load"):
                    lines.append(f"#   {k} {v}")
            return counters

        plain_name = "dit::partition_attention_kernel<128, false>"
        pre_name = "dit::partition_attention_premerge_kernel<128>"
        sq_plain = sq_of(lambda n, g: n == plain_name and g == attn_grid)
        sq_pre = sq_of(lambda n, g: n == pre_name and attn_grid < g <= attn_grid + (1 << 20))
        # the bench step's attention launch: the one with the reuse pre-merge when the step reuses
        if sq_pre:
            rec["attention_counters"] = figures(pre_name, sq_pre)
            if sq_plain:
                rec["plain_attention_counters"] = figures(plain_name, sq_plain)
        elif sq_plain:
            rec["attention_counters"] = figures(plain_name, sq_plain)
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    return "\n".join(lines)


def run_trajectory(args, w: "W.Workload") -> dict:
    """The long-video trajectory: every step planned by the host w*delta planner from the
    previous steps' importance (anchor steps) and local change, with the device-to-host copy
    of those measurements inside each step.  Inputs of all steps are resident in HBM before
    the timed region; every step is timed."""
    import torch
    from partitioned_state_reuse_amd import api
    dev = torch.device("cuda:0")
    t0 = time.time()
    steps = []
    for t, X in W.trajectory(w):
        steps.append(tuple(torch.from_numpy(np.ascontiguousarray(b).view(np.int16)).view(torch.bfloat16).to(dev)
                           for b in (X.q, X.k, X.v)))
        log(f"[bench] step {t} inputs ready ({time.time() - t0:.1f}s)")
    sa = api.SelectiveAttention(1, w.S_q, w.S_kv, w.H, w.D, w.q_offsets, w.kv_offsets, w.local_part)
    planner = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every, w.recompute_groups, "wdelta")
    stream = torch.cuda.current_stream()

    def run(t, record=None):
        mask, groups = planner.next(t)
        anchor = bool(mask.all())
        q, k, v = steps[t]
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        ev[0].record(stream)
        # (a reuse step merges the reused states inside the attention launch; an anchor step,
        # which computes the importance, merges all states after it)
        did_delta = sa.step(q, k, v, mask, want_importance=anchor, want_delta=t > 0, stream=stream)
        ev[1].record(stream)
        imp = sa.importance[0].cpu().numpy() if anchor else None
        dl = sa.delta[0].cpu().numpy() if did_delta else None
        ev[2].record(stream)
        planner.observe(t, imp, dl)
        if record is not None:
            record.append((t, anchor, mask, ev))
        return mask

    # warm-up: one anchor-shaped pass on step 0 (a fresh planner is used for the timed run)
    for _ in range(args.warmup):
        sa.step(*steps[0], np.ones((w.n_qb, w.P), np.uint8), want_importance=True)
    torch.cuda.synchronize()
    sa.valid[:] = 0
    planner.close()
    planner = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every, w.recompute_groups, "wdelta")
    rec = []
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(w.steps):
        run(t, rec)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    qs, ks = np.diff(w.q_offsets), np.diff(w.kv_offsets)
    flops = [float(4 * w.D * w.H * np.sum(m * np.outer(qs, ks))) for _, _, m, _ in rec]
    step_ms = [e[0].elapsed_time(e[2]) for _, _, _, e in rec]
    dev_ms = [e[0].elapsed_time(e[1]) for _, _, _, e in rec]
    planner.close()
    per_step = [{"step": t, "anchor": a, "recomputed_pairs": int(m.sum()), "ms": round(ms, 3), "device_ms": round(dm, 3),
                 "tflops": round(f / (dm * 1e-3) / 1e12, 1)} for (t, a, m, _), ms, dm, f in zip(rec, step_ms, dev_ms, flops)]
    for r in per_step:
        log(f"[bench] {r}")
    return {
        "metric": "recomputed-attn TFLOP/s over the 10-step trajectory (147.6k tokens)",
        "value": round(sum(flops) / wall / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": w.steps, "warmup": args.warmup,
        "ms_per_step": round(wall / w.steps * 1e3, 3),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V with 3D RoPE and per-step drift 0.02 N(0,1), bf16",
        "config": {"workload": w.name, "tokens": w.S_kv, "heads": w.H, "head_dim": w.D, "partitions": w.P,
                   "query_blocks": w.n_qb, "group_size": int(np.diff(w.group_offsets)[0]),
                   "recomputed_groups_per_block": w.recompute_groups, "anchor_every": w.anchor_every,
                   "parallelism": "single GPU"},
        "per_step": per_step,
    }


def cold_ms(launch, copies, reps: int) -> float:
    """Median duration (HIP events on the launch stream) of `launch(copy)` over `reps` launches
    that rotate over several copies of the same state cache: each launch reads planes last
    touched one or more whole merges earlier (at least 0.8 GB of other traffic, beyond the
    256 MB Infinity Cache, the MALL), and no overwrite is needed to empty the MALL, which
    would leave dirty lines to be written back during the timed launch."""
    import torch
    stream = torch.cuda.current_stream()
    for c in copies:
        launch(c)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        launch(copies[i % len(copies)])
        e1.record(stream)
    torch.cuda.synchronize()
    return float(np.median([e0.elapsed_time(e1) for e0, e1 in ev]))


def cache_copies(tensors, n: int):
    """The cache tensors plus n - 1 clones (for cold_ms)."""
    return [tuple(tensors)] + [tuple(t.clone() for t in tensors) for _ in range(n - 1)]


def oracle_leg(w: W.Workload, X: "W.StepInputs", Xp: "W.StepInputs", mask: np.ndarray, rows: np.ndarray,
               gpu_out: np.ndarray, gpu_lse: np.ndarray) -> dict:
    """The oracle beside the GPU step: its reused slots hold the previous step's states for the
    sampled rows (computed first, not timed), then its step work (states of the recomputed
    partitions and the merge of all P states) is timed; the GPU output on the same rows is
    checked against it to the tolerances of the tests."""
    import oracle
    try:
        affinity = len(os.sched_getaffinity(0))
    except AttributeError:
        affinity = os.cpu_count() or 1
    # the oracle's parallel work is its BLAS matrix products: report that pool's thread count
    threads = affinity
    try:
        from threadpoolctl import threadpool_info
        blas = [d["num_threads"] for d in threadpool_info() if d.get("user_api") == "blas"]
        if blas:
            threads = min(max(blas), affinity)
    except Exception:
        pass
    scale = 1.0 / math.sqrt(w.D)
    cache = oracle.StateCache.empty(rows, w.P, w.H, w.D, w.n_qb)
    cache.valid[:] = True          # slots not computed yet hold empty states (weight 0)
    t0 = time.perf_counter()
    oracle.selective_step(W.to_f64(Xp.q[0][rows]), W.to_f64(Xp.k[0]), W.to_f64(Xp.v[0]), rows, w.q_offsets,
                          w.kv_offsets, 1 - mask, cache, scale)
    prep = time.perf_counter() - t0
    t0 = time.perf_counter()
    res = oracle.selective_step(W.to_f64(X.q[0][rows]), W.to_f64(X.k[0]), W.to_f64(X.v[0]), rows, w.q_offsets,
                                w.kv_offsets, mask, cache, scale)
    dt = time.perf_counter() - t0
    blk = oracle.block_of_rows(rows, w.q_offsets)
    sizes = np.diff(w.kv_offsets)
    flop = float(4 * w.D * w.H * sum(int(mask[b].astype(np.int64) @ sizes) for b in blk))
    ref, fin = res.O_stored, np.isfinite(res.lse_stored)
    dO = np.abs(gpu_out - ref)
    row_bound = 2.0 ** -6 * np.abs(ref).max(axis=-1, keepdims=True) + 1e-6
    parity = {"rows": int(len(rows)),
              "max_abs_O": float(dO.max()),
              "rel_fro_O": float(np.linalg.norm(gpu_out - ref) / np.linalg.norm(ref)),
              "max_abs_lse": float(np.abs(np.where(fin, gpu_lse - res.lse_stored, 0.0)).max()),
              "row_bound_ratio": float((dO / row_bound).max())}
    parity["ok"] = bool(parity["max_abs_O"] <= 1e-2 and parity["rel_fro_O"] <= 1e-2 and
                        parity["max_abs_lse"] <= 1e-3 and parity["row_bound_ratio"] <= 1.0 and
                        np.array_equal(np.isfinite(gpu_lse), fin))
    full = len(rows) == w.S_q
    out = {"value": flop / dt / 1e12, "unit": "TFLOP/s", "cores": threads, "host_cpus_available": affinity,
           "kind": "oracle", "seconds": round(dt, 3), "prep_seconds": round(prep, 3)}
    if full:
        out["sample"] = (f"all {w.S_q} query rows, all {w.H} heads (the whole step): fp64 states of the "
                         f"{int(mask.sum())} recomputed (block, partition) pairs and the {w.P}-state merge; "
                         f"reused slots hold the previous step's states (computed before the timing)")
    else:
        out["sample"] = (f"{len(rows)} of {w.S_q} query rows (the first and the last 128-row tile of each of "
                         f"the {w.n_qb} query blocks), all {w.H} heads: fp64 states of the recomputed "
                         f"partitions and the {w.P}-state merge; reused slots hold the previous step's states "
                         f"(computed before the timing)")
        out["extrapolated_step_s"] = round(dt * w.S_q / len(rows), 2)
    return out, parity


def layer_bench(w: W.Workload, args, dev, extras: bool) -> dict:
    """Time the selective step of one single-step layer and its two kernels."""
    import torch
    from partitioned_state_reuse_amd import api
    log(f"[bench] workload {w.name}: S_q={w.S_q} S_kv={w.S_kv} H={w.H} D={w.D} P={w.P} n_qb={w.n_qb}")
    t0 = time.time()
    X = W.make_step(w, 0)
    Xp = W.make_step(w, -1) if w.prev_scale else X
    log(f"[bench] inputs generated in {time.time() - t0:.1f}s")

    def dev_t(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = dev_t(X.q), dev_t(X.k), dev_t(X.v)
    sa = api.SelectiveAttention(1, w.S_q, w.S_kv, w.H, w.D, w.q_offsets, w.kv_offsets, w.local_part)
    mode = "anchor" if w.mode == "anchor" else "distance"
    planner = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every or 0,
                          w.recompute_groups, mode)
    # fill the cache with the previous step's states (not timed)
    qp, kp, vp = dev_t(Xp.q), dev_t(Xp.k), dev_t(Xp.v)
    sa.step(qp, kp, vp, np.ones((w.n_qb, w.P), np.uint8))
    torch.cuda.synchronize()
    del qp, kp, vp
    stream = torch.cuda.current_stream()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    valid = np.ones((w.n_qb, w.P), np.uint8)

    def one_step(t, events=None, plain=False):
        """One step.  By default the library's one call (dit_attn_partitioned with the local
        change): on a step that reuses states it merges them inside the attention launch and
        finishes with the final combine.  With plain: the split calls of the plain sequence (the
        attention kernel, the merge of all P states, the local-change finish), each between
        events."""
        mask, _ = planner.next(t)
        pre = not mask.all()
        if events:
            events[0].record(stream)
        if not plain:
            api.attn_partitioned(q, k, v, w.q_offsets, w.kv_offsets, mask, sa.cache_o, sa.cache_lse, sa.out, sa.lse,
                                 local_part=w.local_part, cache_valid=valid, delta_out=sa.delta,
                                 workspace=sa.workspace, stream=stream)
            if events:
                for e in events[1:]:
                    e.record(stream)
            return mask, pre
        api.partition_attention(q, k, v, w.q_offsets, w.kv_offsets, mask, sa.cache_o, sa.cache_lse,
                                local_part=w.local_part, cache_valid=valid, workspace=sa.workspace, stream=stream)
        if events:
            events[1].record(stream)
        api.state_merge(sa.cache_o, sa.cache_lse, sa.out, sa.lse, stream=stream)
        if events:
            events[2].record(stream)
        api.local_change_finalize(sa.workspace, 1, w.S_q, w.H, w.D, w.q_offsets, sa.delta, stream=stream)
        if events:
            events[3].record(stream)
        return mask, pre

    def timed(plain):
        """The warm-up steps, then the timed steps with nothing else on the stream (wall time
        per step), then the same steps again with HIP events around each call and kernel (the
        device times): the events' own packets stay out of the wall-time figure."""
        for t in range(args.warmup):
            one_step(t + 1, plain=plain)
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for t in range(args.steps):
            mask, pre = one_step(t + 1, plain=plain)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t_start
        for t in range(args.steps):
            one_step(t + 1, ev[t], plain=plain)
        torch.cuda.synchronize()
        return (mask, pre, wall / max(args.steps, 1) * 1e3, float(np.mean([e[0].elapsed_time(e[1]) for e in ev])),
                float(np.mean([e[1].elapsed_time(e[2]) for e in ev])),
                float(np.mean([e[2].elapsed_time(e[3]) for e in ev])))

    # the step as the library runs it (device time of the one call between events), then the
    # plain sequence with an event between its kernels (the attention kernel's roofline)
    mask, pre, ms_step, step_dev_ms, _, _ = timed(False)
    # the GPU's output of the step, for the parity check beside the oracle
    rows = np.arange(w.S_q) if w.S_q <= 4096 else W.sample_rows(w, tiles_per_block=2, tile=128)
    ridx = torch.as_tensor(rows, device=dev)
    gpu_out = W.to_f64(sa.out[0, ridx].view(torch.int16).cpu().numpy().view(np.uint16))
    gpu_lse = sa.lse[0][:, ridx].double().cpu().numpy()
    # the same steps with the plain sequence (attention launch, then the merge of all P states)
    _, _, p_ms, attn_ms, merge_in_step_ms, fin_ms = timed(True)
    p_out = W.to_f64(sa.out[0, ridx].view(torch.int16).cpu().numpy().view(np.uint16))
    plain = {"ms_per_step": round(p_ms, 4), "attention_ms": round(attn_ms, 4),
             "merge_in_step_ms": round(merge_in_step_ms, 4), "kernel": "partition_attention_kernel<128, false>",
             "max_abs_diff_vs_step_out": float(np.abs(p_out - gpu_out).max())}

    # the merge alone on a cold cache (rotating over copies of the cache); the importance
    # variant of anchor steps on the same copies
    copies = cache_copies((sa.cache_o, sa.cache_lse), 2 if w.S_q * w.H * w.P * 260 > 4e9 else 3)
    merge_ms = cold_ms(lambda c: api.state_merge(c[0], c[1], sa.out, sa.lse, stream=stream), copies,
                       max(args.steps, 6))
    imp = torch.empty((1, w.n_qb, w.P), dtype=torch.float32, device=dev)
    anchor_merge_ms = cold_ms(lambda c: api.state_merge(c[0], c[1], sa.out, sa.lse, q_offsets=w.q_offsets,
                                                        importance_out=imp, workspace=sa.workspace, stream=stream),
                              copies, max(args.steps, 6))
    del copies

    flop = attn_flop(w, mask)
    mbytes = merge_bytes(w)
    attn_tflops = flop / (attn_ms * 1e-3) / 1e12
    merge_gbs = mbytes / (merge_ms * 1e-3) / 1e9
    plain["value"] = round(flop / (plain["ms_per_step"] * 1e-3) / 1e12, 2)
    how = ", the reused states merged in the attention launch" if pre else ""
    log(f"[bench] {w.name}: step {ms_step:.3f} ms (device {step_dev_ms:.3f} ms{how})  plain step "
        f"{plain['ms_per_step']:.3f} ms: attention {attn_ms:.3f} ms ({attn_tflops:.1f} TFLOP/s), merge "
        f"{merge_in_step_ms:.3f} ms, finalize {fin_ms:.4f} ms  merge cold {merge_ms:.3f} ms ({merge_gbs:.0f} GB/s; "
        f"with importance {anchor_merge_ms:.3f} ms)")
    traffic = measured_traffic(w.name)
    merge_kernel = f"state_merge_kernel<128, {16 if w.P <= 16 else 32 if w.P <= 32 else 64}, false>"
    # roofline: the partition-attention kernel (a2) itself, from the plain steps of the same run
    # (on a reuse step the step's own launch also carries the pre-merge of the reused states)
    plain_kernel = "partition_attention_kernel<128, false>"
    counters = measured_counters(w.name, plain_kernel)
    roof = {"bound": "mfma", "achieved": round(attn_tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(attn_tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic.get("dit::" + plain_kernel),
            "kernel": plain_kernel, "ms": round(attn_ms, 4), "algorithmic_flop": flop,
            "timed_in": "the plain steps of the same run (attention kernel, merge of all P states, finish)",
            "counters": counters or None,
            "frac_of_clock_peak": (round(attn_tflops / counters["peak_tflops_at_that_clock"], 4)
                                   if counters else None),
            "power": measured_power(w.name) or None}
    res = {
        "ms_per_step": round(ms_step, 4),
        "value": round(flop / (ms_step * 1e-3) / 1e12, 2),
        "step_device_ms": round(step_dev_ms, 4),
        "step": ("dit_attn_partitioned: the reused states merged inside the attention launch, then the final "
                 "combine, then the local-change finish" if pre else
                 "dit_attn_partitioned: attention launch, merge of all states, local-change finish"),
        "config": {"workload": w.name, "tokens": w.S_kv, "query_tokens": w.S_q, "heads": w.H, "head_dim": w.D,
                   "partitions": w.P, "query_blocks": w.n_qb, "group_size": int(np.diff(w.group_offsets)[0]),
                   "recomputed_groups_per_block": w.recompute_groups,
                   "recomputed_pairs": int(mask.sum()), "reused_pairs": int(mask.size - mask.sum()),
                   "parallelism": "single GPU"},
        "roofline": roof,
        "roofline_merge": {"bound": "hbm", "achieved": round(merge_gbs, 1), "peak": PEAK_HBM_GBS,
                           "unit": "GB/s", "frac": round(merge_gbs / PEAK_HBM_GBS, 4),
                           "traffic": traffic.get("dit::" + merge_kernel),
                           "kernel": merge_kernel, "ms": round(merge_ms, 4),
                           "ms_in_plain_step": round(merge_in_step_ms, 4),
                           "algorithmic_bytes": mbytes,
                           "timing": "median over launches rotating over copies of the cache (cold MALL)",
                           "anchor_ms": round(anchor_merge_ms, 4),
                           "anchor_what": "the same merge with the importance partials and their fixed-order finish"},
        "local_change_finalize_ms": round(fin_ms, 5),
        "plain_step": plain,
    }
    plain_ms = plain["ms_per_step"]
    ctx = {"X": X, "Xp": Xp, "mask": mask, "rows": rows, "gpu_out": gpu_out, "gpu_lse": gpu_lse,
           "q": q, "k": k, "v": v, "sa": sa, "planner": planner, "flop": flop, "ms_step": ms_step,
           "plain_ms_step": plain_ms, "merge_ms": merge_ms}
    if extras:
        res.update(layer_extras(w, args, dev, ctx))
    elif pre:
        ov_ms = overlapped_step_ms(args, ctx)
        log(f"[bench] {w.name}: two-stream step {ov_ms:.3f} ms (plain {plain_ms:.3f})")
        res["overlap_two_streams"] = {"ms_per_step": round(ov_ms, 4), "plain_ms_per_step": round(plain_ms, 4),
                                      "value": round(flop / (ov_ms * 1e-3) / 1e12, 2)}
    planner.close()
    return res, ctx


def overlapped_step_ms(args, ctx) -> float:
    """Wall time per step of the two-stream step: the reused states are pre-merged on a second
    stream during the attention kernel, then merged with the fresh states."""
    import torch
    q, k, v, sa, planner, mask = ctx["q"], ctx["k"], ctx["v"], ctx["sa"], ctx["planner"], ctx["mask"]
    side = torch.cuda.Stream()
    for _ in range(args.warmup):
        sa.step_overlapped(q, k, v, mask, side_stream=side, want_delta=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.steps):
        m_t, _ = planner.next(t + 1)
        sa.step_overlapped(q, k, v, m_t, side_stream=side, want_delta=True)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / max(args.steps, 1) * 1e3


def layer_extras(w: W.Workload, args, dev, ctx) -> dict:
    """Importance, planner and enqueue costs, the two-stream step, group compose and the
    compressed cache on the same layer."""
    import torch
    from partitioned_state_reuse_amd import api
    q, k, v, sa, planner, flop, mask = ctx["q"], ctx["k"], ctx["v"], ctx["sa"], ctx["planner"], ctx["flop"], ctx["mask"]
    stream = torch.cuda.current_stream()
    # a5 importance by the second pass over the stored lse planes (callers without a
    # workspace; anchor steps otherwise take it inside the merge, timed with the merge)
    imp = torch.empty((1, w.n_qb, w.P), dtype=torch.float32, device=dev)
    api.importance(sa.cache_lse, sa.lse, w.q_offsets, imp, stream=stream)
    i0, i1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    i0.record(stream)
    for _ in range(5):
        api.importance(sa.cache_lse, sa.lse, w.q_offsets, imp, stream=stream)
    i1.record(stream)
    torch.cuda.synchronize()
    imp_ms = i0.elapsed_time(i1) / 5
    # a7 planner decision and a1 host enqueue cost (validation + work description + launch)
    t0 = time.perf_counter()
    for t in range(200):
        planner.next(t + 100)
    planner_us = (time.perf_counter() - t0) / 200 * 1e6
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(3):
        api.partition_attention(q, k, v, w.q_offsets, w.kv_offsets, mask, sa.cache_o, sa.cache_lse,
                                local_part=w.local_part, stream=stream)
    enqueue_us = (time.perf_counter() - t0) / 3 * 1e6
    torch.cuda.synchronize()
    log(f"[bench] second-pass importance {imp_ms:.3f} ms, planner {planner_us:.1f} us/call, attention enqueue "
        f"{enqueue_us:.1f} us")

    ov_ms = overlapped_step_ms(args, ctx)
    # dynamic group compose of the P cached states into the groups
    go = w.group_offsets
    G = len(go) - 1
    comp_o = torch.empty((G, 1, w.S_q, w.H, w.D), dtype=torch.bfloat16, device=dev)
    comp_l = torch.empty((G, 1, w.S_q, w.H), dtype=torch.float32, device=dev)
    api.state_compose(sa.cache_o, sa.cache_lse, go, comp_o, comp_l, stream=stream)
    c0_, c1_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0_.record(stream)
    for _ in range(5):
        api.state_compose(sa.cache_o, sa.cache_lse, go, comp_o, comp_l, stream=stream)
    c1_.record(stream)
    torch.cuda.synchronize()
    comp_ms = c0_.elapsed_time(c1_) / 5
    comp_bytes = float(w.S_q * w.H * (w.P + G) * (2 * w.D + 4))
    del comp_o, comp_l
    log(f"[bench] two-stream step {ov_ms:.3f} ms (plain {ctx['plain_ms_step']:.3f}); group compose {comp_ms:.3f} ms "
        f"({comp_bytes / (comp_ms * 1e-3) / 1e9:.0f} GB/s)")

    # compressed (fp8 e4m3 + per-row-head scale) state cache: same step on its own cache
    sa8 = api.SelectiveAttention(1, w.S_q, w.S_kv, w.H, w.D, w.q_offsets, w.kv_offsets, w.local_part,
                                 cache_format="fp8")
    sa8.step(q, k, v, np.ones((w.n_qb, w.P), np.uint8))
    ev8 = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    valid = np.ones((w.n_qb, w.P), np.uint8)

    def fp8_step(t, e=None):
        m_t, _ = planner.next(t)
        if e:
            e[0].record(stream)
        api.partition_attention_fp8(q, k, v, w.q_offsets, w.kv_offsets, m_t, sa8.cache_o, sa8.cache_scale,
                                    sa8.cache_lse, local_part=w.local_part, cache_valid=valid,
                                    workspace=sa8.workspace, stream=stream)
        if e:
            e[1].record(stream)
        api.state_merge_fp8(sa8.cache_o, sa8.cache_scale, sa8.cache_lse, sa8.out, sa8.lse, stream=stream)
        if e:
            e[2].record(stream)
        api.local_change_finalize(sa8.workspace, 1, w.S_q, w.H, w.D, w.q_offsets, sa8.delta, stream=stream)

    for t in range(args.warmup):
        fp8_step(t + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for t in range(args.steps):
        fp8_step(t + 1)
    torch.cuda.synchronize()
    fp8_ms = (time.perf_counter() - t0) / max(args.steps, 1) * 1e3
    for t in range(args.steps):   # again with events, for the attention kernel's device time
        fp8_step(t + 1, ev8[t])
    torch.cuda.synchronize()
    fp8_attn_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev8]))
    copies = cache_copies((sa8.cache_o, sa8.cache_scale, sa8.cache_lse), 2)
    fp8_merge_ms = cold_ms(lambda c: api.state_merge_fp8(c[0], c[1], c[2], sa8.out, sa8.lse, stream=stream), copies,
                           max(args.steps, 6))
    del copies
    # per row-head: P planes of D code bytes + scale + lse read, bf16 output + lse written
    fp8_bytes = float(w.S_q * w.H * (w.P * (w.D + 8) + 2 * w.D + 4))
    del sa8
    log(f"[bench] fp8 cache step {fp8_ms:.3f} ms: attention {fp8_attn_ms:.3f} ms, merge {fp8_merge_ms:.3f} ms "
        f"({fp8_bytes / (fp8_merge_ms * 1e-3) / 1e9:.0f} GB/s)")
    return {
        "overlap_two_streams": {"ms_per_step": round(ov_ms, 4), "plain_ms_per_step": round(ctx["plain_ms_step"], 4),
                                "value": round(flop / (ov_ms * 1e-3) / 1e12, 2)},
        "group_compose": {"ms": round(comp_ms, 4), "gbs": round(comp_bytes / (comp_ms * 1e-3) / 1e9, 1),
                          "frac": round(comp_bytes / (comp_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                          "algorithmic_bytes": comp_bytes, "planes": f"{w.P} -> {len(w.group_offsets) - 1}"},
        "fp8_cache": {"ms_per_step": round(fp8_ms, 4), "attention_ms": round(fp8_attn_ms, 4),
                      "attention_tflops": round(flop / (fp8_attn_ms * 1e-3) / 1e12, 1),
                      "merge_ms": round(fp8_merge_ms, 4),
                      "merge_gbs": round(fp8_bytes / (fp8_merge_ms * 1e-3) / 1e9, 1),
                      "merge_frac": round(fp8_bytes / (fp8_merge_ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
                      "merge_algorithmic_bytes": fp8_bytes,
                      "value": round(flop / (fp8_ms * 1e-3) / 1e12, 2)},
        "importance_second_pass_ms": round(imp_ms, 4),
        "planner_us_per_step": round(planner_us, 2),
        "attention_enqueue_us": round(enqueue_us, 2),
    }


def power_trace(w: W.Workload) -> str:
    """Socket power, per-XCD graphics clock and temperatures (amd-smi, sampled about every
    0.3 s by a child process) while the selective step's attention kernel runs back to back
    for 10 s, then the merge for 6 s, then the whole step for 8 s each way (the library's one
    call, with the reused states merged inside the attention launch, and the plain sequence of
    attention, merge of all states and local-change finish), with idle gaps between: whether a
    kernel runs at the clock ceiling or the power ceiling, and what the in-launch merge does to
    the power and clock of the step."""
    import subprocess
    import threading
    import torch
    from partitioned_state_reuse_amd import api
    X = W.make_step(w, 0)
    dev = torch.device("cuda:0")

    def dev_t(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    q, k, v = dev_t(X.q), dev_t(X.k), dev_t(X.v)
    sa = api.SelectiveAttention(1, w.S_q, w.S_kv, w.H, w.D, w.q_offsets, w.kv_offsets, w.local_part)
    sa.step(q, k, v, np.ones((w.n_qb, w.P), np.uint8))
    mode = "anchor" if w.mode == "anchor" else "distance"
    planner = api.Planner(w.n_qb, w.P, w.group_offsets, w.local_part, w.anchor_every or 0, w.recompute_groups, mode)
    mask, _ = planner.next(1)
    planner.close()
    valid = np.ones((w.n_qb, w.P), np.uint8)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    samples, phase, done = [], ["idle"], threading.Event()

    def sample():
        while not done.is_set():
            t = time.time()
            try:
                r = subprocess.run(["amd-smi", "metric", "-p", "-c", "-t", "--json"], capture_output=True, text=True,
                                   timeout=10)
                d = json.loads(r.stdout)
                g = (d["gpu_data"] if isinstance(d, dict) else d)[0]
                clk = [g["clock"][f"gfx_{i}"]["clk"]["value"] for i in range(8) if f"gfx_{i}" in g["clock"]]
                temp = g.get("temperature", {})
                hot = temp.get("hotspot", {}).get("value") if isinstance(temp.get("hotspot"), dict) else None
                mem = temp.get("mem", {}).get("value") if isinstance(temp.get("mem"), dict) else None
                samples.append((t, phase[0], g["power"]["socket_power"]["value"], clk, hot, mem))
            except Exception as e:  # no amd-smi or an unexpected format: report and stop sampling
                samples.append((t, phase[0], None, [], None, repr(e)[:200]))
                return
            time.sleep(0.2)

    th = threading.Thread(target=sample, daemon=True)
    th.start()

    def run_for(name, seconds, fn, batch):
        phase[0] = name
        t0, n = time.time(), 0
        while time.time() - t0 < seconds:
            for _ in range(batch):
                fn()
            torch.cuda.synchronize()
            n += batch
        return (time.time() - t0) / n * 1e3

    time.sleep(2)
    att_ms = run_for("attention", 10, lambda: api.partition_attention(
        q, k, v, w.q_offsets, w.kv_offsets, mask, sa.cache_o, sa.cache_lse, cache_valid=valid, stream=stream), 5)
    phase[0] = "idle"
    time.sleep(3)
    mer_ms = run_for("merge", 6, lambda: api.state_merge(sa.cache_o, sa.cache_lse, sa.out, sa.lse, stream=stream), 50)
    phase[0] = "idle"
    time.sleep(3)

    def one_call():
        api.attn_partitioned(q, k, v, w.q_offsets, w.kv_offsets, mask, sa.cache_o, sa.cache_lse, sa.out, sa.lse,
                             local_part=w.local_part, cache_valid=valid, delta_out=sa.delta, workspace=sa.workspace,
                             stream=stream)

    def plain():
        api.partition_attention(q, k, v, w.q_offsets, w.kv_offsets, mask, sa.cache_o, sa.cache_lse,
                                local_part=w.local_part, cache_valid=valid, workspace=sa.workspace, stream=stream)
        api.state_merge(sa.cache_o, sa.cache_lse, sa.out, sa.lse, stream=stream)
        api.local_change_finalize(sa.workspace, 1, w.S_q, w.H, w.D, w.q_offsets, sa.delta, stream=stream)

    one_ms = run_for("one_call", 8, one_call, 5)
    phase[0] = "idle"
    time.sleep(3)
    pl_ms = run_for("plain_step", 8, plain, 5)
    phase[0] = "idle"
    time.sleep(2)
    done.set()
    th.join()
    lines = [f"# source_sha256 {kernel_source_sha256()}",
             f"# {w.name}: attention kernel {att_ms:.2f} ms per launch back to back, merge {mer_ms:.3f} ms, "
             f"step {one_ms:.3f} ms as one call, {pl_ms:.3f} ms as the plain sequence",
             "# time_s  phase       socket_W  gfx_MHz per XCD                                  hotspot_C mem_C"]
    t_first = samples[0][0] if samples else 0.0
    prev = None
    for t, ph, pw, clk, hot, mem in samples:
        if (ph, pw, clk, hot, mem) == prev:   # amd-smi refreshes about once a second: repeats dropped
            continue
        prev = (ph, pw, clk, hot, mem)
        lines.append(f"{t - t_first:7.2f}  {ph:<10} {str(pw):>8}  {' '.join(f'{c:>5}' for c in clk):<48} {str(hot):>8} {str(mem):>5}")
    # the sampler refreshes about once a second; steady state: samples at least 1.5 s into a phase
    for name in ("attention", "merge", "one_call", "plain_step"):
        t_start = min((t for t, ph, *_ in samples if ph == name), default=None)
        sel = [s for s in samples if s[1] == name and t_start is not None and s[0] - t_start >= 1.5 and s[2] is not None]
        if sel:
            clk = np.array([s[3] for s in sel], dtype=np.float64)
            lines.append(f"# {name} steady state ({len(sel)} samples): socket power {np.mean([s[2] for s in sel]):.0f} W, "
                         f"gfx clock per XCD {' '.join(f'{c:.0f}' for c in clk.mean(axis=0))} MHz "
                         f"(mean {clk.mean():.0f}), hotspot up to {max(s[4] or 0 for s in sel)} C")
    return "\n".join(lines)


def main() -> int:
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-profile":
        print(summarize_profile(sys.argv[2]))
        return 0
    if len(sys.argv) in (2, 3) and sys.argv[1] == "--power-trace":
        # --power-trace [workload]
        print(power_trace(W.workload(sys.argv[2] if len(sys.argv) == 3 else "video720p")), flush=True)
        return 0
    if len(sys.argv) >= 6 and sys.argv[1] == "--summarize-pmc":
        # --summarize-pmc <workload> <out.json> <FETCH_SIZE dir> <WRITE_SIZE dir> [<SQ dir> ...]
        print(summarize_pmc(sys.argv[2], sys.argv[3], sys.argv[4], sys.argv[5], sys.argv[6:]))
        return 0
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 10; 100 for the short share32 and image_anchor steps)")
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 2; 20 for share32 and image_anchor)")
    ap.add_argument("--workload", default="video720p", choices=["video720p", "share32", "image_anchor", "longvideo"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-share32", action="store_true", help="with the 720p layer: skip the 32-way-share object")
    args = ap.parse_args()
    if args.gpus != 1:
        print(json.dumps({"error": "this library runs on one GPU only; --gpus must be 1 "
                                   "(the path would shard by query block across GPUs; that exchange is not implemented)"}))
        return 2

    import torch

    if not torch.cuda.is_available():
        log("no GPU visible")
        return 1
    dev = torch.device("cuda:0")
    w = W.workload(args.workload)
    # a step of the short layouts takes ~1 ms or less: ten times the steps by default, so that
    # the timing covers a steady clock as the 720p one does
    short = w.name in ("share32", "image_anchor")
    if args.steps is None:
        args.steps = 100 if short else 10
    if args.warmup is None:
        args.warmup = 20 if short else 2
    if w.mode == "wdelta":
        print(json.dumps(run_trajectory(args, w)), flush=True)
        return 0
    layer, ctx = layer_bench(w, args, dev, extras=(w.name == "video720p"))

    # plain device copy of 4 GiB as the achievable-bandwidth reference (and PMC calibration)
    stream = torch.cuda.current_stream()
    src = torch.empty(1 << 31, dtype=torch.int16, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(3):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * src.numel() * 2 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst
    log(f"[bench] device copy {copy_gbs:.0f} GB/s")
    layer["roofline_merge"]["device_copy_gbs"] = round(copy_gbs, 1)

    share = None
    if w.name == "video720p" and not args.no_share32:
        # a 32-way-share step takes ~1.2 ms: ten times the steps (and warm-up steps) of the
        # 720p layer, so that the timing covers a steady clock as the 720p one does
        ws = W.workload("share32")
        sargs = argparse.Namespace(**vars(args))
        sargs.steps, sargs.warmup = 10 * args.steps, 10 * args.warmup
        share, sctx = layer_bench(ws, sargs, dev, extras=False)
        share["steps"], share["warmup"] = sargs.steps, sargs.warmup
        share["metric"] = "recomputed-attn TFLOP/s + merge GB/s, one GPU's share of a 32-way split of 75.6k tokens"
        share["unit"] = "TFLOP/s"
    result = {
        "metric": "recomputed-attn TFLOP/s + merge GB/s at 75.6k tokens, % of MFMA/HBM peak",
        "value": layer["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": layer["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded N(0,1) Q/K/V with 3D RoPE, bf16",
    }
    result.update({k: v for k, v in layer.items() if k not in ("value", "ms_per_step")})
    if not args.no_cpu_baseline:
        log(f"[bench] timing the oracle on {len(ctx['rows'])} rows of {w.name} ...")
        result["cpu_baseline"], result["parity"] = oracle_leg(w, ctx["X"], ctx["Xp"], ctx["mask"], ctx["rows"],
                                                              ctx["gpu_out"], ctx["gpu_lse"])
        log(f"[bench] oracle {result['cpu_baseline']['seconds']} s (prep {result['cpu_baseline']['prep_seconds']} s), "
            f"parity {result['parity']}")
    if share is not None:
        if not args.no_cpu_baseline:
            log(f"[bench] timing the oracle on the whole 32-way-share step ...")
            share["cpu_baseline"], share["parity"] = oracle_leg(ws, sctx["X"], sctx["Xp"], sctx["mask"], sctx["rows"],
                                                                sctx["gpu_out"], sctx["gpu_lse"])
            log(f"[bench] oracle {share['cpu_baseline']['seconds']} s (prep {share['cpu_baseline']['prep_seconds']} s), "
                f"parity {share['parity']}")
        result["share32"] = share
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
