"""GPU guard tests: NaN canaries around every tensor, offsets past 4 GiB,
bitwise determinism, outputs pre-filled with NaN, a non-default stream."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from parity_util import check_grads, compare, grad_bounds, oracle_full

pytestmark = pytest.mark.gpu

NAN16 = 0x7E00


def embed(t: torch.Tensor, pad: int, fill_bits: int):
    """Copy t into the middle of a larger buffer whose padding holds the
    given 16-bit pattern; returns (view, whole buffer)."""
    n = t.numel()
    buf = torch.empty(n + 2 * pad, dtype=torch.int16, device="cuda")
    buf.fill_(fill_bits - 65536 if fill_bits > 32767 else fill_bits)
    view = buf[pad:pad + n].view(t.dtype).view(t.shape)
    view.copy_(t)
    return view, buf


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_nan_canaries_and_untouched_padding(causal, D):
    cfg = fi.Config("canary", 2, 3, 130, 197, D, fi.F16, causal, seed=77)
    inp = fi.make_inputs(cfg)
    ref_o, ref_l = oracle_full(cfg, inp)
    pad = 4096   # elements of NaN on each side
    q, _ = embed(inp.q.cuda(), pad, NAN16)
    k, _ = embed(inp.k.cuda(), pad, NAN16)
    v, _ = embed(inp.v.cuda(), pad, NAN16)
    o_template = torch.empty(cfg.B, cfg.H, cfg.Sq, D, dtype=torch.float16, device="cuda")
    o, obuf = embed(o_template, pad, NAN16)
    lbuf = torch.full((cfg.B * cfg.H * cfg.Sq + 2 * pad,), float("nan"), device="cuda")
    lse = lbuf[pad:pad + cfg.B * cfg.H * cfg.Sq].view(cfg.B, cfg.H, cfg.Sq)
    fa.fa_fwd(q, k, v, scale=cfg.scale, causal=causal, out=o, lse=lse)
    torch.cuda.synchronize()
    compare(cfg, fi.F16, o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l,
            what="canary")
    ob = obuf.cpu().numpy()
    assert np.all(ob[:pad] == np.int16(NAN16 - 65536 if NAN16 > 32767 else NAN16))
    assert np.all(ob[-pad:] == ob[0])
    lb = lbuf.cpu().numpy()
    assert np.all(np.isnan(lb[:pad])) and np.all(np.isnan(lb[-pad:]))


def test_offsets_past_4gib():
    """All five tensors start beyond 4 GiB inside one 5 GiB allocation."""
    cfg = fi.Config("far", 1, 2, 200, 200, 128, fi.BF16, True, seed=78)
    inp = fi.make_inputs(cfg)
    ref_o, ref_l = oracle_full(cfg, inp)
    big = torch.empty(5 << 30, dtype=torch.uint8, device="cuda")
    base = (4 << 30) + 4096
    nq = inp.q.numel() * 2

    def place(off, t_or_shape, dtype):
        n = int(np.prod(t_or_shape)) * torch.tensor([], dtype=dtype).element_size()
        return big[off:off + n].view(dtype).view(t_or_shape), off + ((n + 4095) // 4096) * 4096

    q, off = place(base, tuple(inp.q.shape), torch.bfloat16)
    k, off = place(off, tuple(inp.k.shape), torch.bfloat16)
    v, off = place(off, tuple(inp.v.shape), torch.bfloat16)
    o, off = place(off, tuple(inp.q.shape), torch.float32)
    lse, off = place(off, (cfg.B, cfg.H, cfg.Sq), torch.float32)
    assert q.data_ptr() - big.data_ptr() > (4 << 30) and nq > 0
    q.copy_(inp.q.cuda()); k.copy_(inp.k.cuda()); v.copy_(inp.v.cuda())
    fa.fa_fwd(q, k, v, scale=cfg.scale, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    compare(cfg, fi.F32, o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l,
            what="past 4 GiB")
    del big


def test_deterministic_and_nan_prefilled_output():
    cfg = fi.Config("det", 2, 4, 333, 333, 128, fi.F16, False, seed=79)
    inp = fi.make_inputs(cfg)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o1 = torch.full((2, 4, 333, 128), float("nan"), dtype=torch.float16, device="cuda")
    l1 = torch.full((2, 4, 333), float("nan"), device="cuda")
    fa.fa_fwd(q, k, v, out=o1, lse=l1)
    o2, l2 = fa.fa_fwd(q, k, v)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def test_non_default_stream():
    cfg = fi.Config("stream", 1, 2, 257, 257, 64, fi.F16, True, seed=80)
    inp = fi.make_inputs(cfg)
    ref_o, ref_l = oracle_full(cfg, inp)
    s = torch.cuda.Stream()
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=True, o_dtype=torch.float32)
    s.synchronize()
    compare(cfg, fi.F32, o.double().cpu().numpy(), lse.double().cpu().numpy(), ref_o, ref_l,
            what="stream")


def test_large_logits_stay_finite():
    """Scores far beyond the fp16 exp-overflow point of the pages (a scaled
    logit of ~11.09) give finite outputs equal to the oracle's."""
    cfg = fi.Config("hot", 1, 2, 300, 300, 64, fi.F16, True, amp=6.0, seed=81)
    inp = fi.make_inputs(cfg)
    inp.v = fi.make_inputs(cfg.replace(amp=1.0)).v   # large scores, unit-size values
    ref_o, ref_l = oracle_full(cfg, inp)
    from parity_util import run_gpu
    o, lse = run_gpu(cfg, inp, fi.F32)
    compare(cfg, fi.F32, o, lse, ref_o, ref_l, what="large logits")
    assert ref_l.max() > 100


def test_backward_offsets_past_4gib_and_side_stream():
    """Every backward tensor and the workspace start beyond 4 GiB inside one
    5 GiB allocation, launched on a non-default stream."""
    from oracle import attention_bwd_fp64
    cfg = fi.Config("far_bwd", 1, 4, 150, 170, 128, fi.F16, True, seed=82)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :2].contiguous()
    inp.v = inp.v[:, :2].contiguous()
    do = fi.make_cotangent((1, 4, 150, 128), fi.F16, 83)
    qq, kk, vv = fi.values(inp)
    ref = attention_bwd_fp64(qq, kk, vv, do.double().numpy(), cfg.scale, True)
    big = torch.empty(5 << 30, dtype=torch.uint8, device="cuda")
    off = [(4 << 30) + 4096]

    def place(shape, dtype):
        n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
        t = big[off[0]:off[0] + n].view(dtype).view(shape)
        off[0] += ((n + 4095) // 4096) * 4096
        return t

    q = place(tuple(inp.q.shape), torch.float16)
    k = place(tuple(inp.k.shape), torch.float16)
    v = place(tuple(inp.v.shape), torch.float16)
    o = place(tuple(inp.q.shape), torch.float16)
    dout = place(tuple(inp.q.shape), torch.float16)
    lse = place((1, 4, 150), torch.float32)
    dq = place(tuple(inp.q.shape), torch.float32)
    dk = place(tuple(inp.k.shape), torch.float32)
    dv = place(tuple(inp.v.shape), torch.float32)
    ws = place((fa.bwd_workspace_size(1, 4, 150),), torch.uint8)
    assert q.data_ptr() - big.data_ptr() > (4 << 30)
    q.copy_(inp.q.cuda()); k.copy_(inp.k.cuda()); v.copy_(inp.v.cuda()); dout.copy_(do.cuda())
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        fa.fa_fwd(q, k, v, scale=cfg.scale, causal=True, out=o, lse=lse)
        fa.fa_bwd(q, k, v, o, dout, lse, scale=cfg.scale, causal=True, dq=dq, dk=dk, dv=dv,
                  workspace=ws)
    s.synchronize()
    bnd = grad_bounds(qq, kk, vv, do.double().numpy(), cfg.scale, True, 0,
                      o_used=o.double().cpu().numpy(), lse_used=lse.double().cpu().numpy())
    check_grads(fi.F16, tuple(t.double().cpu().numpy() for t in (dq, dk, dv)), ref, bnd,
                "tensors past 4 GiB")
    del big


def test_varlen_on_side_stream():
    from oracle import attention_varlen_fp64
    vi = fi.make_varlen_inputs([70, 1, 130], [90, 40, 130], 4, 2, 64, fi.F16, seed=84)
    q, k, v = (t.cuda() for t in (vi.inp.q, vi.inp.k, vi.inp.v))
    cq, ck = vi.cu_q.cuda(), vi.cu_k.cuda()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        o, lse = fa.fa_fwd_varlen(q, k, v, cq, ck, vi.max_q, causal="bottom_right",
                                  o_dtype=torch.float32)
    s.synchronize()
    q64, k64, v64 = fi.values(vi.inp)
    ro, rl = attention_varlen_fp64(q64, k64, v64, vi.cu_q.numpy(), vi.cu_k.numpy(), 0.125, True,
                                   True)
    assert np.abs(o.double().cpu().numpy() - ro).max() <= 2e-3
    assert np.abs(lse.double().cpu().numpy() - rl).max() <= 1e-3
