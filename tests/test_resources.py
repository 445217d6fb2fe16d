"""Every kernel the library builds runs without scratch memory: no register
spills (the static-register-indexing lesson of "Hygon FlashAttention:
fixed-defect review", item 6, checked with the compiler's
kernel-resource-usage report). Uses the build's record when it matches the
sources, else compiles the sources for the device (about a minute)."""
from attention_fa_fwd_07_amd.build import current_usage


def test_no_kernel_uses_scratch():
    usage = current_usage()
    kernels = usage["kernels"]
    assert len(kernels) > 50, "expected the full set of kernel instances"
    spills = {k: v.get("scratch") for k, v in kernels.items() if v.get("scratch", 0) != 0}
    assert not spills, f"kernels with scratch (bytes per lane): {spills}"
    missing = [k for k, v in kernels.items() if "scratch" not in v]
    assert not missing, f"no scratch figure for {missing[:3]}"
