"""fa_fwd_splitkv_noalloc (through the C ABI) against fa_fwd_splitkv with a
caller-owned workspace: the same kernels, so the outputs must be equal bit
for bit, on two calls in a row, the second with a smaller problem (the
static workspace keeps the first call's partial results, which the second
must not see), and against the oracle's tolerances."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from parity_util import compare, oracle_full

pytestmark = pytest.mark.gpu


def noalloc(q, k, v, cfg, num_splits, o_dtype):
    o = torch.full(tuple(q.shape), float("nan"), dtype=o_dtype, device="cuda")
    lse = torch.full(tuple(q.shape[:3]), float("nan"), dtype=torch.float32, device="cuda")
    code = fa.fa_fwd_splitkv_noalloc_raw(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), cfg.B, cfg.H,
        cfg.Sq, cfg.Sk, cfg.D, fa.FA_LAYOUT_BNSD, cfg.scale, 1 if cfg.causal else 0, 1.0,
        fa._dtype_code(q.dtype), fa._dtype_code(o_dtype), None, None, None, num_splits,
        torch.cuda.current_stream().cuda_stream)
    assert code == fa.FA_OK, fa.status_str(code)
    return o, lse


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
def test_noalloc_equals_splitkv_twice(dtype):
    cases = [
        (fi.Config("big", 2, 8, 1000, 1500, 128, dtype, True, seed=501), 5),
        (fi.Config("small", 1, 3, 130, 200, 64, dtype, False, seed=502), 3),
    ]
    for cfg, ns in cases:
        inp = fi.make_inputs(cfg)
        q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
        ref_o, ref_l = fa.fa_fwd_splitkv(q, k, v, num_splits=ns, scale=cfg.scale,
                                         causal=cfg.causal, o_dtype=torch.float32)
        o, lse = noalloc(q, k, v, cfg, ns, torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), cfg.name
        oo, ol = oracle_full(cfg, inp)
        compare(cfg, fi.F32, o.double().cpu().numpy(), lse.double().cpu().numpy(), oo, ol,
                what=f"noalloc {cfg.name}")


def test_noalloc_automatic_split_count_and_fp8():
    cfg = fi.Config("fp8", 1, 4, 300, 2000, 128, fi.FP8, True, seed=503)
    inp = fi.make_inputs(cfg)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    ds = [torch.tensor([d], dtype=torch.float32, device="cuda")
          for d in (inp.descale_q, inp.descale_k, inp.descale_v)]
    ref_o, ref_l = fa.fa_fwd_splitkv(q, k, v, num_splits=0, scale=cfg.scale, causal=True,
                                     o_dtype=torch.float16, descale_q=ds[0], descale_k=ds[1], descale_v=ds[2])
    o = torch.empty(tuple(q.shape), dtype=torch.float16, device="cuda")
    lse = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device="cuda")
    code = fa.fa_fwd_splitkv_noalloc_raw(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 4, 300, 2000,
        128, fa.FA_LAYOUT_BNSD, cfg.scale, 1, 1.0, fa.FA_FP8_E4M3, fa.FA_F16, ds[0].data_ptr(),
        ds[1].data_ptr(), ds[2].data_ptr(), 0, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert code == fa.FA_OK
    assert torch.equal(o, ref_o) and torch.equal(lse, ref_l)


def test_noalloc_rejects_a_problem_over_its_workspace():
    q = torch.zeros(1, 64, 1017, 128, dtype=torch.float16, device="cuda")
    o = torch.empty_like(q)
    lse = torch.empty(1, 64, 1017, dtype=torch.float32, device="cuda")
    code = fa.fa_fwd_splitkv_noalloc_raw(
        q.data_ptr(), q.data_ptr(), q.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 64, 1017, 1017,
        128, fa.FA_LAYOUT_BNSD, 0.1, 0, 1.0, fa.FA_F16, fa.FA_F16, None, None, None, 2,
        torch.cuda.current_stream().cuda_stream)
    assert code == fa.FA_ERR_SCRATCH
