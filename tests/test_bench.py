"""CPU checks of bench.py's host logic: the one-GPU guard, the CPU baseline
leg (the oracle on whole heads over a pool of host processes) and the
traffic record it reports next to the roofline."""
import json
import os
import subprocess
import sys

import bench
import fa_inputs as fi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_cpu_baseline_runs_whole_heads_on_host_processes():
    cfg = fi.Config("tiny", 1, 3, 96, 80, 64, fi.F16, True, seed=5)
    inp = fi.make_inputs(cfg)
    r = bench.cpu_baseline(cfg, inp, 30.0)
    assert r["kind"] == "oracle" and r["unit"] == "TFLOP/s" and r["value"] > 0
    assert 1 <= r["cores"] <= 16 and r["cores"] <= len(os.sched_getaffinity(0))
    assert r["sample"].startswith("3 of 3 heads of tiny")


def test_cpu_baseline_of_the_backward():
    cfg = fi.Config("tinyb", 1, 2, 64, 64, 64, fi.BF16, False, seed=6)
    inp = fi.make_inputs(cfg)
    dout = fi.make_cotangent(tuple(inp.q.shape), cfg.dtype, 7)
    r = bench.cpu_baseline_bwd(cfg, inp, dout, 30.0)
    assert r["value"] > 0 and r["sample"].startswith("backward of 2 of 2 heads")


def test_traffic_records():
    """The committed HBM-byte records: one per workload, each the copy-
    calibrated counter readings; bench.py reports a workload's bytes only
    while the kernel sources still hash to the recorded value (else null)."""
    d = json.load(open(bench.TRAFFIC_FILE))
    recs = d["workloads"]
    assert set(recs) == {c.name for c in fi.CONFIGS}
    for name, r in recs.items():
        assert r["bytes_per_launch"] == r["fetch_bytes"] + r["write_bytes"]
        assert abs(r["fetch_bytes"] - r["fetch_size_kib_raw"] * 1024 * d["copy_factor_fetch"]) < 1e6
        assert abs(r["write_bytes"] - r["write_size_kib_raw"] * 1024 * d["copy_factor_write"]) < 1e6
        # no kernel moves fewer bytes than Q, K, V once and O, lse once
        assert r["bytes_per_launch"] >= 0.99 * r["algorithmic_bytes"]
        got = bench.measured_traffic(name)
        if d["kernel_source_sha256_16"] == bench.kernel_source_hash():
            assert got == r["bytes_per_launch"]
        else:
            assert got is None
    assert bench.measured_traffic("no such workload") is None
