"""GPU parity of the split-KV entry point (keys of each query block split
into ranges that run as separate workgroups, merged by logsumexp) against
the fp64 oracle on the same seeded inputs, through the C ABI."""
import functools

import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from parity_util import compare, oracle_full, oracle_rows, run_gpu, sample_rows

pytestmark = pytest.mark.gpu

LENGTHS = [(1, 1), (65, 65), (129, 513), (300, 100), (257, 1000)]


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16, fi.FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_splitkv_edges(dtype, D, causal):
    """Several range counts, including more ranges than key tiles (empty
    ranges) and the automatic choice."""
    native = fi.BF16 if dtype == fi.BF16 else fi.F16
    for i, (Sq, Sk) in enumerate(LENGTHS):
        cfg = fi.Config("split", 1, 3, Sq, Sk, D, dtype, causal, seed=700 + i)
        inp = fi.make_inputs(cfg)
        ref_o, ref_l = oracle_full(cfg, inp)
        for ns in (0, 2, 7, 40):
            fwd = functools.partial(fa.fa_fwd_splitkv, num_splits=ns)
            for od in (fi.F32, native):
                o, lse = run_gpu(cfg, inp, od, fwd=fwd)
                compare(cfg, od, o, lse, ref_o, ref_l,
                        what=f"{dtype} D{D} c{causal} {Sq}x{Sk} splits {ns} {od}")


@pytest.mark.parametrize("idx", range(len(fi.CONFIGS)), ids=[c.name for c in fi.CONFIGS])
def test_splitkv_workloads(idx):
    """The five workloads at full size, automatic range count and three
    ranges: whole first head and sampled rows of two more."""
    cfg = fi.CONFIGS[idx]
    inp = fi.make_inputs(cfg)
    rng = np.random.default_rng(100 + idx)
    for ns in (0, 3):
        fwd = functools.partial(fa.fa_fwd_splitkv, num_splits=ns)
        o, lse = run_gpu(cfg, inp, fi.F32, fwd=fwd)
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
        ro, rl = oracle_rows(cfg, inp, 0, 0, np.arange(cfg.Sq))
        compare(cfg, fi.F32, o[0, 0], lse[0, 0], ro, rl, what=f"{cfg.name} splits {ns} head 0,0")
        for _ in range(2):
            b, h = int(rng.integers(cfg.B)), int(rng.integers(cfg.H))
            rows = sample_rows(cfg.Sq, rng)
            ro, rl = oracle_rows(cfg, inp, b, h, rows)
            compare(cfg, fi.F32, o[b, h, rows], lse[b, h, rows], ro, rl,
                    what=f"{cfg.name} splits {ns} rows of {b},{h}")


def test_splitkv_reuses_a_dirty_workspace():
    """The workspace's previous contents do not matter (NaN-filled here)."""
    cfg = fi.Config("ws", 2, 2, 200, 700, 128, fi.F16, True, seed=790)
    inp = fi.make_inputs(cfg)
    ref_o, ref_l = oracle_full(cfg, inp)
    need = fa.splitkv_workspace_size(2, 2, 200, 700, 128, True, 5)
    ws = torch.full((need // 4 + 64,), float("nan"), device="cuda").view(torch.uint8)
    fwd = functools.partial(fa.fa_fwd_splitkv, num_splits=5, workspace=ws)
    o, lse = run_gpu(cfg, inp, fi.F32, fwd=fwd)
    compare(cfg, fi.F32, o, lse, ref_o, ref_l, what="dirty workspace")
