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


def test_traffic_record_belongs_to_the_headline_kernel():
    """The committed HBM-byte record names the headline kernel and workload;
    bench.py reports its bytes only while the kernel sources still hash to
    the recorded value (else null), and the record's bytes are the copy-
    calibrated counter readings."""
    d = json.load(open(bench.TRAFFIC_FILE))
    assert d["workload"] == fi.HEADLINE.name
    assert d["bytes_per_launch"] == d["fetch_bytes"] + d["write_bytes"]
    assert abs(d["fetch_bytes"] - d["fetch_size_kib_raw"] * 1024 * d["copy_factor_fetch"]) < 1e6
    assert abs(d["write_bytes"] - d["write_size_kib_raw"] * 1024 * d["copy_factor_write"]) < 1e6
    got = bench.measured_traffic(fi.HEADLINE.name)
    if d["kernel_source_sha256_16"] == bench.kernel_source_hash():
        assert got == d["bytes_per_launch"]
    else:
        assert got is None
    # another workload's line carries no traffic figure (it was not measured)
    for cfg in fi.CONFIGS:
        if cfg.name != fi.HEADLINE.name:
            assert bench.measured_traffic(cfg.name) is None
