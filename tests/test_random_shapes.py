"""Seeded random sweep of the whole call surface against the fp64 oracle:
forward (dtype, head dim, grouped heads, lengths, mask, layout, split count,
output type), variable-length batches and the backward. Every case prints
its parameters first, so a failure names it."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from oracle import attention_bwd_fp64, attention_fp64, attention_varlen_fp64
from parity_util import TOL_LSE, TOL_O, as_used, check_grads, grad_bounds, to_device, ulp

pytestmark = pytest.mark.gpu

MASKS = ["none", "top_left", "bottom_right"]


def draw_case(rng):
    dtype = [fi.F16, fi.BF16, fi.FP8][rng.integers(3)]
    D = [64, 128][rng.integers(2)]
    Hkv = int(rng.integers(1, 4))
    H = Hkv * int(rng.integers(1, 4))
    B = int(rng.integers(1, 4))
    Sq = int(rng.integers(1, 600))
    Sk = int(rng.integers(1, 600))
    mask = MASKS[rng.integers(3)]
    layout = ["BNSD", "BSHD"][rng.integers(2)]
    splits = [None, None, 0, 3][rng.integers(4)]
    od = [fi.F32, "native"][rng.integers(2)]
    return dtype, D, B, H, Hkv, Sq, Sk, mask, layout, splits, od


@pytest.mark.parametrize("case", range(40))
def test_random_forward(case):
    rng = np.random.default_rng(9000 + case)
    dtype, D, B, H, Hkv, Sq, Sk, mask, layout, splits, od = draw_case(rng)
    if od == "native":
        od = fi.BF16 if dtype == fi.BF16 else fi.F16
    what = f"case {case}: {dtype} D{D} B{B} H{H}/{Hkv} {Sq}x{Sk} {mask} {layout} splits {splits} {od}"
    print(what, flush=True)
    cfg = fi.Config("rand", B, H, Sq, Sk, D, dtype, mask != "none", seed=9100 + case)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    q64, k64, v64 = fi.values(inp)
    off = (Sk - Sq) if mask == "bottom_right" else 0
    ref_o, ref_l = attention_fp64(q64, k64, v64, cfg.scale, mask != "none", off)
    q, k, v, ds = to_device(inp)
    kw = {} if ds is None else dict(descale_q=ds[0], descale_k=ds[1], descale_v=ds[2])
    if layout == "BSHD":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    causal = False if mask == "none" else mask
    if splits is None:
        o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=causal, o_dtype=fi.TORCH_DTYPE[od],
                           layout=layout, **kw)
    else:
        o, lse = fa.fa_fwd_splitkv(q, k, v, num_splits=splits, scale=cfg.scale, causal=causal,
                                   o_dtype=fi.TORCH_DTYPE[od], layout=layout, **kw)
    torch.cuda.synchronize()
    if layout == "BSHD":
        o = o.transpose(1, 2)
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0.0), what
    bound = TOL_O[dtype] + (0.0 if od == fi.F32 else ulp(ref_o[~empty], od))
    err = np.abs(o[~empty] - ref_o[~empty])
    assert np.all(err <= bound), f"{what}: max |dO| {err.max():.3e}"
    assert np.abs(lse[~empty] - ref_l[~empty]).max(initial=0.0) <= TOL_LSE, what


@pytest.mark.parametrize("case", range(24))
def test_random_causal_many_heads(case):
    """Causal grids with 4..16 key/value head groups, the range where the
    launch order deals whole groups to the XCDs and orders blocks by length
    (groups beyond a multiple of 8 first; long and short blocks paired when
    the grid is resident): the forward and, for 16-bit inputs, the backward
    chained on it, against the oracle."""
    rng = np.random.default_rng(9700 + case)
    dtype = [fi.F16, fi.BF16, fi.FP8][rng.integers(3)]
    D = [64, 128][rng.integers(2)]
    B = int(rng.integers(2, 5))
    Hkv = int(rng.integers(2, 5))
    H = Hkv * int(rng.integers(1, 3))
    Sq = int(rng.integers(1, 700))
    Sk = int(rng.integers(1, 700))
    mask = ["top_left", "bottom_right"][rng.integers(2)]
    what = f"case {case}: {dtype} D{D} B{B} H{H}/{Hkv} {Sq}x{Sk} {mask}"
    print(what, flush=True)
    cfg = fi.Config("rcausal", B, H, Sq, Sk, D, dtype, True, seed=9800 + case)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    q64, k64, v64 = fi.values(inp)
    off = (Sk - Sq) if mask == "bottom_right" else 0
    ref_o, ref_l = attention_fp64(q64, k64, v64, cfg.scale, True, off)
    q, k, v, ds = to_device(inp)
    kw = {} if ds is None else dict(descale_q=ds[0], descale_k=ds[1], descale_v=ds[2])
    o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=mask, o_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0.0), what
    err = np.abs(o[~empty] - ref_o[~empty])
    assert np.all(err <= TOL_O[dtype]), f"{what}: max |dO| {err.max(initial=0.0):.3e}"
    assert np.abs(lse[~empty] - ref_l[~empty]).max(initial=0.0) <= TOL_LSE, what
    if dtype == fi.FP8:
        return
    g = fi.make_cotangent((B, H, Sq, D), dtype, 9900 + case)
    td = fi.TORCH_DTYPE[dtype]
    o16 = torch.from_numpy(ref_o).to(torch.float32).to(td).cuda()
    l32 = torch.from_numpy(ref_l).to(torch.float32).cuda()
    dq, dk, dv = fa.fa_bwd(q, k, v, o16, g.cuda(), l32, scale=cfg.scale, causal=mask,
                           grad_dtype=torch.float32)
    torch.cuda.synchronize()
    refs = attention_bwd_fp64(q64, k64, v64, g.double().numpy(), cfg.scale, True, off)
    bounds = grad_bounds(q64, k64, v64, g.double().numpy(), cfg.scale, True, off,
                         o_used=as_used(ref_o, dtype), lse_used=as_used(ref_l, fi.F32))
    check_grads(dtype, tuple(t.double().cpu().numpy() for t in (dq, dk, dv)), refs, bounds, what)


@pytest.mark.parametrize("case", range(12))
def test_random_varlen(case):
    rng = np.random.default_rng(9200 + case)
    dtype = [fi.F16, fi.BF16, fi.FP8][rng.integers(3)]
    D = [64, 128][rng.integers(2)]
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.integers(1, 4))
    nseq = int(rng.integers(1, 9))
    lq = [int(x) for x in rng.integers(0, 400, nseq)]
    lk = [int(x) for x in rng.integers(0, 400, nseq)]
    if sum(lq) == 0:
        lq[0] = 1
    if sum(lk) == 0:
        lk[0] = 1
    mask = MASKS[rng.integers(3)]
    what = f"case {case}: {dtype} D{D} H{H}/{Hkv} lq {lq} lk {lk} {mask}"
    print(what, flush=True)
    vi = fi.make_varlen_inputs(lq, lk, H, Hkv, D, dtype, seed=9300 + case)
    q64, k64, v64 = fi.values(vi.inp)
    scale = D ** -0.5
    ref_o, ref_l = attention_varlen_fp64(q64, k64, v64, vi.cu_q.numpy(), vi.cu_k.numpy(), scale,
                                         mask != "none", mask == "bottom_right")
    q, k, v = (t.cuda() for t in (vi.inp.q, vi.inp.k, vi.inp.v))
    kw = {}
    if dtype == fi.FP8:
        kw = {n: torch.tensor([d], dtype=torch.float32, device="cuda") for n, d in
              (("descale_q", vi.inp.descale_q), ("descale_k", vi.inp.descale_k),
               ("descale_v", vi.inp.descale_v))}
    o, lse = fa.fa_fwd_varlen(q, k, v, vi.cu_q.cuda(), vi.cu_k.cuda(), vi.max_q, scale=scale,
                              causal=False if mask == "none" else mask,
                              o_dtype=torch.float32, **kw)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    empty = np.isneginf(ref_l)
    assert np.all(np.isneginf(lse[empty])), what
    assert np.all(o.transpose(1, 0, 2)[empty] == 0.0), what
    assert np.abs(o - ref_o).max(initial=0.0) <= TOL_O[dtype], what
    assert np.abs(lse[~empty] - ref_l[~empty]).max(initial=0.0) <= TOL_LSE, what


@pytest.mark.parametrize("case", range(12))
def test_random_backward(case):
    rng = np.random.default_rng(9400 + case)
    dtype = [fi.F16, fi.BF16][rng.integers(2)]
    D = [64, 128][rng.integers(2)]
    Hkv = int(rng.integers(1, 3))
    H = Hkv * int(rng.integers(1, 4))
    B = int(rng.integers(1, 3))
    Sq = int(rng.integers(1, 400))
    Sk = int(rng.integers(1, 400))
    mask = MASKS[rng.integers(3)]
    what = f"case {case}: {dtype} D{D} B{B} H{H}/{Hkv} {Sq}x{Sk} {mask}"
    print(what, flush=True)
    cfg = fi.Config("rbwd", B, H, Sq, Sk, D, dtype, mask != "none", seed=9500 + case)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    do = fi.make_cotangent((B, H, Sq, D), dtype, 9600 + case)
    q64, k64, v64 = fi.values(inp)
    off = (Sk - Sq) if mask == "bottom_right" else 0
    o_ref, lse_ref = attention_fp64(q64, k64, v64, cfg.scale, mask != "none", off)
    ref = attention_bwd_fp64(q64, k64, v64, do.double().numpy(), cfg.scale, mask != "none", off)
    td = fi.TORCH_DTYPE[dtype]
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o = torch.from_numpy(o_ref).to(torch.float32).to(td).cuda()
    lse = torch.from_numpy(lse_ref).to(torch.float32).cuda()
    grads = fa.fa_bwd(q, k, v, o, do.cuda(), lse, scale=cfg.scale,
                      causal=False if mask == "none" else mask, grad_dtype=torch.float32)
    torch.cuda.synchronize()
    bnd = grad_bounds(q64, k64, v64, do.double().numpy(), cfg.scale, mask != "none", off,
                      o_used=as_used(o_ref, dtype), lse_used=as_used(lse_ref, fi.F32))
    check_grads(dtype, tuple(t.double().cpu().numpy() for t in grads), ref, bnd, what)
