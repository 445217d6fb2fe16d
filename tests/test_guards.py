"""GPU guard tests: NaN canaries around every tensor, offsets past 4 GiB,
bitwise determinism, outputs pre-filled with NaN, a non-default stream."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from parity_util import compare, oracle_full

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
