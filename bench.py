"""Benchmark: attention forward TFLOP/s and fraction of the MI355X dense fp16
MFMA peak on B4 H32 Sq=Sk=4096 D128 fp16, BNSD, non-causal, one GPU.

One step = one fa_fwd call over the whole batch (inputs resident in HBM).
With --pass bwd one step is one fa_bwd call (dQ, dK, dV from the forward's
O and lse, which are computed before the timed region) on the same
workload, counted at 2.5 times the forward's flop. Prints one JSON line.
Options:
  --gpus N      only N=1 is supported (one process, one GPU)
  --steps K     timed steps (default 50)
  --warmup W    untimed steps first (default 30: the clocks settle under load)
  --workload I  index into the workload list (default: the headline, 2)
  --pass P      fwd (default) or bwd
  --keep-prob K with dropout (keep probability K < 1, seed 0), forward or
                backward
  --no-cpu      skip the CPU-oracle baseline leg
  --cpu-seconds approximate CPU budget for the oracle leg (default 15)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "fp8_e4m3": 5033.2}   # dense MFMA, MI355X
HBM_GBPS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fa_fwd_traffic.json")
KERNEL_SRCS = [os.path.join(ROOT, "attention_fa_fwd_07_amd", "csrc", f)
               for f in ("fa_fwd.hip", "fa_device.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SRCS:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def device_info():
    import ctypes
    import torch
    props = torch.cuda.get_device_properties(0)
    info = {"name": props.name, "cus": props.multi_processor_count,
            "arch": getattr(props, "gcnArchName", "")}
    try:
        hip = ctypes.CDLL("libamdhip64.so")
        v = ctypes.c_int(0)
        # hipDeviceAttributeClockRate = 5 (kHz)
        if hip.hipDeviceGetAttribute(ctypes.byref(v), 5, 0) == 0:
            info["sclk_mhz"] = v.value / 1000.0
    except OSError:
        pass
    return info


def measured_traffic(workload: str):
    """HBM bytes per launch of the forward kernel on this workload, from the
    committed rocprofv3 counter summary (one record per workload), valid only
    for the kernel source it was measured on."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    d = json.load(open(TRAFFIC_FILE))
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    rec = d.get("workloads", {}).get(workload)
    return None if rec is None else rec.get("bytes_per_launch")


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _single_thread():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _oracle_fwd_head(args):
    from oracle import head_forward
    q, k, v, scale, causal = args
    head_forward(q, k, v, scale, causal)
    return 1


def _oracle_bwd_head(args):
    from oracle import attention_bwd_fp64
    q, k, v, g, scale, causal = args
    attention_bwd_fp64(q, k, v, g, scale, causal)
    return 1


def _host_workers() -> int:
    # the host cores this process may use, at most 16 (one GPU's share of a box)
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _timed_pool(fn, items, budget_s: float):
    """Run fn over items on a pool of single-threaded worker processes (one
    per host core), one wave of len(pool) items at a time, until the items
    or the budget run out; returns (items done, wall seconds, workers).
    The pool is forked before this process touches the GPU."""
    import multiprocessing as mp
    workers = _host_workers()
    with mp.get_context("fork").Pool(workers, initializer=_single_thread) as pool:
        pool.map(int, range(workers))            # start the workers before timing
        done = 0
        t0 = time.perf_counter()
        while done < len(items) and time.perf_counter() - t0 < budget_s:
            batch = [items[i]() for i in range(done, min(done + workers, len(items)))]
            pool.map(fn, batch)
            done += len(batch)
        dt = time.perf_counter() - t0
    return done, dt, workers


def cpu_baseline(cfg, inp, budget_s: float):
    """The oracle, as it stands, on a bounded sample of whole heads, one head
    per host core at a time."""
    import fa_inputs as fi
    items = [(lambda b=b, h=h: (fi.as_float64(inp.q[b, h], inp.descale_q),
                                fi.as_float64(inp.k[b, h], inp.descale_k),
                                fi.as_float64(inp.v[b, h], inp.descale_v), cfg.scale, cfg.causal))
             for b in range(cfg.B) for h in range(cfg.H)]
    heads, dt, workers = _timed_pool(_oracle_fwd_head, items, budget_s)
    flops = cfg.flops() * heads / (cfg.B * cfg.H)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": f"{heads} of {cfg.B * cfg.H} heads of {cfg.name}, fp64 numpy, "
                      f"{workers} processes of one BLAS thread, one head each at a time, "
                      f"{dt:.1f} s; value = algorithmic FLOP of the sample / wall time",
            "cpu": cpu_model()}


def cpu_baseline_bwd(cfg, inp, dout, budget_s: float):
    """The oracle's backward, as it stands, on a bounded sample of whole heads."""
    import fa_inputs as fi

    def head(b, h):
        sl = (slice(b, b + 1), slice(h, h + 1))
        return (fi.as_float64(inp.q[sl], inp.descale_q), fi.as_float64(inp.k[sl], inp.descale_k),
                fi.as_float64(inp.v[sl], inp.descale_v), dout[sl].double().numpy(), cfg.scale,
                cfg.causal)
    items = [(lambda b=b, h=h: head(b, h)) for b in range(cfg.B) for h in range(cfg.H)]
    heads, dt, workers = _timed_pool(_oracle_bwd_head, items, budget_s)
    flops = 2.5 * cfg.flops() * heads / (cfg.B * cfg.H)
    return {"value": round(flops / dt / 1e12, 6), "unit": "TFLOP/s", "cores": workers,
            "kind": "oracle",
            "sample": f"backward of {heads} of {cfg.B * cfg.H} heads of {cfg.name}, fp64 numpy, "
                      f"{workers} processes of one BLAS thread, {dt:.1f} s; value = 2.5 x "
                      f"forward flop of the sample / wall time",
            "cpu": cpu_model()}


def gemm_ceiling(torch, steps, warmup):
    """torch.matmul (hipBLASLt) on 8192^3 fp16 and bf16 operands: one JSON
    line per type with the mean time per product (HIP events)."""
    n = 8192
    g = torch.Generator(device="cuda:0").manual_seed(7)
    for dt in (torch.float16, torch.bfloat16):
        a = torch.randn(n, n, device="cuda:0", generator=g).to(dt)
        b = torch.randn(n, n, device="cuda:0", generator=g).to(dt)
        for _ in range(warmup):
            c = a @ b
        torch.cuda.synchronize()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        for _ in range(steps):
            c = a @ b
        e.record()
        torch.cuda.synchronize()
        ms = s.elapsed_time(e) / steps
        print(json.dumps({"gemm": f"{n}^3", "dtype": str(dt).replace("torch.", ""),
                          "ms": round(ms, 4), "tflops": round(2 * n ** 3 / ms / 1e9, 1),
                          "frac_of_dense_peak": round(2 * n ** 3 / ms / 1e9 / PEAK_TFLOPS["f16"], 4)}))
        del a, b, c


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", type=int, default=2)
    ap.add_argument("--pass", dest="which", choices=("fwd", "bwd"), default="fwd")
    ap.add_argument("--keep-prob", type=float, default=1.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 512 MiB device-to-device copy (reference kernel "
                         "of known traffic for the HBM byte counters)")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only time the library GEMM (torch.matmul, hipBLASLt) at 8192^3 "
                         "in fp16 and bf16: the dense MFMA rate a tuned GEMM reaches on "
                         "this GPU, context for the attention kernel's fraction")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on one GPU only: the attention forward here is a "
              "single-GPU kernel (heads shard across GPUs without communication; "
              "no multi-GPU path is built)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = 512 << 20
        a = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_read": n, "copy_bytes_written": n, "launches": 3}))
        return
    if args.gemm_ceiling:
        gemm_ceiling(torch, args.steps, args.warmup)
        return
    import attention_fa_fwd_07_amd as fa
    import fa_inputs as fi

    cfg = fi.CONFIGS[args.workload]
    inp = fi.make_inputs(cfg)
    bwd = args.which == "bwd"
    if bwd and cfg.dtype not in (fi.F16, fi.BF16):
        print("the backward takes fp16 or bf16 inputs", file=sys.stderr)
        sys.exit(2)
    dout_cpu = fi.make_cotangent(tuple(inp.q.shape), cfg.dtype, cfg.seed + 5000) if bwd else None
    # the CPU leg first: its worker processes are forked before this process
    # initialises the GPU
    baseline = None
    if not args.no_cpu and args.keep_prob == 1.0:
        baseline = (cpu_baseline_bwd(cfg, inp, dout_cpu, args.cpu_seconds) if bwd
                    else cpu_baseline(cfg, inp, args.cpu_seconds))
    dev = torch.device("cuda:0")
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    kw = {}
    if cfg.dtype == fi.FP8:
        kw = {n: torch.tensor([d], dtype=torch.float32, device=dev) for n, d in
              (("descale_q", inp.descale_q), ("descale_k", inp.descale_k),
               ("descale_v", inp.descale_v))}
    o = torch.empty(tuple(q.shape), dtype=fi.TORCH_DTYPE[cfg.o_dtype], device=dev)
    lse = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device=dev)
    if bwd:
        dout = dout_cpu.to(dev)
        dkw = {} if args.keep_prob == 1.0 else dict(keep_prob=args.keep_prob, seed=0)
        fa.fa_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, out=o, lse=lse, **dkw)
        grads = tuple(torch.empty_like(t) for t in (q, k, v))
        ws = torch.empty(fa.bwd_workspace_size(cfg.B, cfg.H, cfg.Sq) + 256, dtype=torch.uint8,
                         device=dev)

    def step():
        if bwd:
            fa.fa_bwd(q, k, v, o, dout, lse, scale=cfg.scale, causal=cfg.causal, dq=grads[0],
                      dk=grads[1], dv=grads[2], workspace=ws, **dkw)
        elif args.keep_prob != 1.0:
            fa.fa_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, out=o, lse=lse,
                      keep_prob=args.keep_prob, seed=0, **kw)
        else:
            fa.fa_fwd(q, k, v, scale=cfg.scale, causal=cfg.causal, out=o, lse=lse, **kw)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        starts[i].record(stream)
        step()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_launch_ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    avg_ms = statistics.fmean(per_launch_ms)
    med_ms = statistics.median(per_launch_ms)
    ms_per_step = wall / args.steps * 1e3

    flops = cfg.flops() * (2.5 if bwd else 1.0)
    value = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[cfg.dtype]
    achieved = flops / (avg_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak,
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": None if (bwd or args.keep_prob != 1.0) else measured_traffic(cfg.name),
                "kernel": "fa_bwd (row pass, dK/dV and dQ kernels; one call)" if bwd
                else "fa_fwd_kernel", "avg_launch_ms": round(avg_ms, 4),
                "median_launch_ms": round(med_ms, 4), "min_launch_ms": round(min(per_launch_ms), 4)}

    out = {
        "metric": ("attn bwd TFLOP/s (2.5x forward flop) + % fp16 MFMA peak, "
                   f"{cfg.name} (1 GPU)") if bwd else
                  "attn fwd TFLOP/s + % fp16 MFMA peak, B4 H32 S4096 D128 fp16 (1 GPU)",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "pct_peak": round(100 * value / peak, 2),
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1), BNSD)",
        "config": {"workload": cfg.name, "B": cfg.B, "H": cfg.H, "Sq": cfg.Sq, "Sk": cfg.Sk,
                   "D": cfg.D, "causal": cfg.causal, "in_dtype": cfg.dtype,
                   "o_dtype": cfg.o_dtype, "layout": "BNSD", "flop_per_step": flops,
                   "pass": args.which, "keep_prob": args.keep_prob},
        "roofline": roofline,
        "device": device_info(),
    }
    if args.keep_prob != 1.0:
        out["metric"] += f", dropout keep_prob {args.keep_prob}"
        if not bwd:
            out["roofline"]["kernel"] = "fa_fwd_drop_kernel"
    if baseline is not None:
        out["cpu_baseline"] = baseline
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
