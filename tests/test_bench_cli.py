"""CPU checks of bench.py's command-line contract (nothing here touches a GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_record_matches_kernel_sources_or_is_ignored():
    """The committed HBM-traffic record is used only while its source hash matches."""
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_video720p.json")))
    got = bench.measured_traffic("video720p")
    if rec["source_sha256"] == bench.kernel_source_sha256():
        assert got and all(v > 0 for v in got.values())
    else:
        assert got == {}


def test_counter_record_follows_the_same_source_hash():
    """The attention kernel's counter figures are reported under the same hash guard, and are
    self-consistent: the clock-scaled peak follows from the nominal peak at 2.4 GHz."""
    sys.path.insert(0, ROOT)
    import bench
    rec = json.load(open(os.path.join(ROOT, "profiles", "traffic_video720p.json")))
    for kernel in ("partition_attention_kernel<128, false>", "partition_attention_premerge_kernel<128>"):
        got = bench.measured_counters("video720p", kernel)
        if rec["source_sha256"] != bench.kernel_source_sha256():
            assert got == {}
            continue
        assert got["kernel"] == "dit::" + kernel
        assert 0.5 < got["clock_ghz_under_load"] <= 2.4
        assert 0.0 < got["mfma_busy_frac"] <= 1.0
        assert abs(got["peak_tflops_at_that_clock"] - 2500.0 * got["clock_ghz_under_load"] / 2.4) < 1.0


def test_power_record_follows_the_same_source_hash(monkeypatch):
    """The committed power trace is parsed (attention, merge and both step phases) while its
    source hash matches the kernel sources, and ignored once it does not."""
    sys.path.insert(0, ROOT)
    import bench
    text = open(os.path.join(ROOT, "profiles", "power_video720p.txt")).read()
    got = bench.measured_power("video720p")
    if f"# source_sha256 {bench.kernel_source_sha256()}" in text:
        for phase in ("attention", "merge", "one_call", "plain_step"):
            assert 500 < got[phase]["socket_w"] < 2000
            assert len(got[phase]["gfx_mhz_per_xcd"]) == 8
            assert min(got[phase]["gfx_mhz_per_xcd"]) <= got[phase]["gfx_mhz_mean"] <= max(got[phase]["gfx_mhz_per_xcd"])
    else:
        assert got == {}
    # once the kernel sources differ from those the trace was taken on, it is not used
    monkeypatch.setattr(bench, "kernel_source_sha256", lambda: "0" * 64)
    assert bench.measured_power("video720p") == {}
