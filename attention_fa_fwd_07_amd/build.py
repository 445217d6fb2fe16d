"""Build libfa_mi355x.so in place (hipcc, gfx950).

Usage: python -m attention_fa_fwd_07_amd.build
"""
from __future__ import annotations

import hashlib
import json
import os
import re
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("fa_fwd.hip", "fa_bwd.hip")]
LIB = os.path.join(HERE, "libfa_mi355x.so")
USAGE = os.path.join(HERE, "resource_usage.json")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # keep IEEE infinities and NaNs: the causal mask is -inf
    "-fno-finite-math-only",
    "-fno-fast-math",
    # no packed fp32 arithmetic (v_pk_{add,mul,fma}_f32) in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: no AGPR copies around the O rescale
    "-mllvm", "-amdgpu-mfma-vgpr-form=1",
    "-Rpass-analysis=kernel-resource-usage",
]


def sources_hash() -> str:
    """sha256 of the HIP sources, headers and build flags."""
    h = hashlib.sha256(" ".join(FLAGS).encode())
    files = SRCS + [os.path.join(HERE, "csrc", f) for f in sorted(os.listdir(os.path.join(HERE, "csrc")))
                    if f.endswith(".h")] + [os.path.join(ROOT, "include", "fa_mi355x.h")]
    for f in files:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse_usage(log: str) -> dict:
    """Per-kernel resource usage from the compiler's kernel-resource-usage
    remarks: {mangled name: {"vgprs", "agprs", "scratch", "occupancy"}}."""
    out, cur = {}, None
    keys = {"VGPRs": "vgprs", "AGPRs": "agprs", "ScratchSize [bytes/lane]": "scratch",
            "Occupancy [waves/SIMD]": "occupancy"}
    for line in log.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]|Occupancy \[waves/SIMD\]): (\d+)", line)
        if m and cur is not None:
            cur[keys[m.group(1)]] = int(m.group(2))
    return out


def write_usage(log: str) -> dict:
    usage = {"sources_sha256_16": sources_hash(), "kernels": parse_usage(log)}
    with open(USAGE, "w") as f:
        json.dump(usage, f, indent=1, sort_keys=True)
    return usage


def device_usage() -> dict:
    """Compile the sources for the device only (no library) and return the
    usage record; for checks where no current build record exists."""
    inc = os.path.join(ROOT, "include")
    flags = [f for f in FLAGS if f not in ("-shared", "-fPIC")]
    logs = []
    with tempfile.TemporaryDirectory() as tmp:
        procs = [subprocess.Popen([HIPCC, *flags, "--cuda-device-only", "-c", "-I", inc, src, "-o",
                                   os.path.join(tmp, os.path.basename(src) + ".o")],
                                  stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
                 for src in SRCS]
        for pr in procs:
            out, _ = pr.communicate()
            if pr.returncode != 0:
                raise RuntimeError("hipcc failed:\n" + out[-4000:])
            logs.append(out)
    return {"sources_sha256_16": sources_hash(), "kernels": parse_usage("\n".join(logs))}


def current_usage() -> dict:
    """The build's usage record when it matches the sources, else a fresh
    device-only compile."""
    if os.path.exists(USAGE):
        with open(USAGE) as f:
            u = json.load(f)
        if u.get("sources_sha256_16") == sources_hash() and u.get("kernels"):
            return u
    return device_usage()


def build(verbose: bool = False) -> str:
    """Compile the HIP library; returns the path of the .so. Always rebuilds."""
    inc = os.path.join(ROOT, "include")
    tmp = LIB + ".tmp"
    srcs = [f for f in SRCS if os.path.exists(f)]
    cmd = [HIPCC, *FLAGS, "-I", inc, *srcs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    log = os.path.join(HERE, "build.log")
    with open(log, "w") as f:
        f.write(" ".join(cmd) + "\n" + r.stdout + r.stderr)
    if r.returncode != 0:
        sys.stderr.write(r.stderr[-4000:])
        raise RuntimeError(f"hipcc failed (exit {r.returncode}); see {log}")
    os.replace(tmp, LIB)
    usage = write_usage(r.stdout + r.stderr)
    if verbose:
        spills = {k: v["scratch"] for k, v in usage["kernels"].items() if v.get("scratch")}
        print(f"built {LIB} ({len(usage['kernels'])} kernels, "
              f"{len(spills)} with scratch{': ' + str(spills) if spills else ''})")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
