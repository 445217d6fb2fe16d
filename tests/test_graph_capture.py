"""The forward under HIP graph capture: fa_fwd (one kernel) and
fa_fwd_splitkv_noalloc (split kernels plus merge, its workspace in the
library's static array: the entry point meant for callers that capture
graphs and cannot allocate) captured once, replayed several times with new
inputs copied into the captured buffers and eager work in between; every
replay must equal the eager call on the same inputs bit for bit."""
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi

pytestmark = pytest.mark.gpu


def _inputs(seed, B, H, S, D, dtype):
    cfg = fi.Config("graph", B, H, S, S, D, dtype, True, seed=seed)
    inp = fi.make_inputs(cfg)
    return cfg, [t.cuda() for t in (inp.q, inp.k, inp.v)]


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                      # warm-up outside the graph
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def test_fa_fwd_replays_equal_eager():
    cfg, (q, k, v) = _inputs(901, 2, 4, 700, 128, fi.F16)
    o = torch.empty_like(q)
    lse = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device="cuda")
    g = _capture(lambda: fa.fa_fwd(q, k, v, scale=cfg.scale, causal=True, out=o, lse=lse))
    for rep in range(4):
        _, (q2, k2, v2) = _inputs(910 + rep, 2, 4, 700, 128, fi.F16)
        q.copy_(q2); k.copy_(k2); v.copy_(v2)
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = fa.fa_fwd(q2, k2, v2, scale=cfg.scale, causal=True)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        _ = (q2.float() @ k2.float().transpose(-1, -2).contiguous()).sum()   # eager work between


def test_noalloc_splitkv_replays_equal_eager():
    cfg, (q, k, v) = _inputs(920, 1, 2, 1500, 64, fi.BF16)
    o = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
    lse = torch.empty(tuple(q.shape[:3]), dtype=torch.float32, device="cuda")
    ns = 4
    assert fa.splitkv_workspace_size(1, 2, 1500, 1500, 64, True, ns) > 0

    def call():
        code = fa.fa_fwd_splitkv_noalloc_raw(
            q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), 1, 2, 1500,
            1500, 64, fa.FA_LAYOUT_BNSD, cfg.scale, 1, 1.0, fa.FA_BF16, fa.FA_F32, None, None, None,
            ns, torch.cuda.current_stream().cuda_stream)
        assert code == fa.FA_OK, fa.status_str(code)

    g = _capture(call)
    for rep in range(4):
        _, (q2, k2, v2) = _inputs(930 + rep, 1, 2, 1500, 64, fi.BF16)
        q.copy_(q2); k.copy_(k2); v.copy_(v2)
        g.replay()
        torch.cuda.synchronize()
        ref_o, ref_l = fa.fa_fwd_splitkv(q2, k2, v2, num_splits=ns, scale=cfg.scale, causal=True,
                                         o_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(o, ref_o) and torch.equal(lse, ref_l), f"replay {rep}"
        _ = torch.zeros(1 << 20, device="cuda").add_(1).sum()
