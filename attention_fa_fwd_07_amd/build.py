"""Build libfa_mi355x.so in place (hipcc, gfx950).

Usage: python -m attention_fa_fwd_07_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRCS = [os.path.join(HERE, "csrc", f) for f in ("fa_fwd.hip", "fa_bwd.hip")]
LIB = os.path.join(HERE, "libfa_mi355x.so")
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
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
