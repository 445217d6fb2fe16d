"""GPU parity of grouped key/value heads (k, v with H_kv heads) and the
bottom-right causal alignment against the fp64 oracle, through the C ABI
(fa_fwd_ex; the plain and the split-KV paths)."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from oracle import attention_fp64, attention_rows_fp64
from parity_util import compare

pytestmark = pytest.mark.gpu

MASKS = {"none": (False, 0), "top_left": (True, 0), "bottom_right": (True, None)}


def run_case(dtype, D, H, Hkv, Sq, Sk, mask, num_splits, seed):
    cfg = fi.Config("gqa", 2, H, Sq, Sk, D, dtype, MASKS[mask][0], seed=seed)
    inp = fi.make_inputs(cfg)
    # the first H_kv heads of the drawn k, v are the grouped key/value heads
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    q64, k64, v64 = fi.values(inp)
    offset = (Sk - Sq) if mask == "bottom_right" else 0
    ref_o, ref_l = attention_fp64(q64, k64, v64, cfg.scale, MASKS[mask][0], offset)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    kw = {}
    if dtype == fi.FP8:
        kw = {n: torch.tensor([d], dtype=torch.float32, device="cuda") for n, d in
              (("descale_q", inp.descale_q), ("descale_k", inp.descale_k),
               ("descale_v", inp.descale_v))}
    causal = False if mask == "none" else mask
    native = fi.BF16 if dtype == fi.BF16 else fi.F16
    for od in (fi.F32, native):
        if num_splits is None:
            o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=causal,
                               o_dtype=fi.TORCH_DTYPE[od], **kw)
        else:
            o, lse = fa.fa_fwd_splitkv(q, k, v, num_splits=num_splits, scale=cfg.scale,
                                       causal=causal, o_dtype=fi.TORCH_DTYPE[od], **kw)
        torch.cuda.synchronize()
        o = o.double().cpu().numpy()
        lse = lse.double().cpu().numpy()
        what = f"{dtype} D{D} H{H}/{Hkv} {Sq}x{Sk} {mask} splits {num_splits} {od}"
        empty = np.isneginf(ref_l)
        # rows without a visible key: O = 0 and lse = -inf exactly
        assert np.all(np.isneginf(lse[empty])), what
        assert np.all(o[empty] == 0.0), what
        assert not np.any(np.isneginf(lse[~empty])), what
        compare(cfg, od, o[~empty], lse[~empty], ref_o[~empty], ref_l[~empty], what=what)


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16, fi.FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
def test_grouped_heads_and_masks(dtype, D, mask):
    for i, (H, Hkv, Sq, Sk) in enumerate([(4, 1, 65, 130), (6, 2, 130, 65), (4, 4, 1, 200),
                                          (4, 2, 200, 1), (2, 1, 257, 300)]):
        for ns in (None, 3):
            run_case(dtype, D, H, Hkv, Sq, Sk, mask, ns, seed=900 + 10 * i)


def test_bottom_right_long_tail_of_empty_rows():
    """Sq far above Sk: all but the last Sk rows see no key (whole blocks of
    empty rows, and blocks whose waves are partly empty)."""
    run_case(fi.F16, 128, 4, 2, 1000, 70, "bottom_right", None, seed=990)
    run_case(fi.F16, 64, 4, 2, 1000, 70, "bottom_right", 4, seed=991)


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16, fi.FP8])
@pytest.mark.parametrize("D", [64, 128])
def test_bshd_layout(dtype, D):
    """q, o [B,Sq,H,D] and k, v [B,Sk,H_kv,D]: the BNSD inputs, transposed;
    the result transposed back must match the oracle."""
    for i, (H, Hkv, Sq, Sk, mask, ns) in enumerate([
            (4, 2, 100, 300, "none", None), (6, 3, 257, 257, "top_left", None),
            (4, 1, 300, 100, "bottom_right", None), (4, 4, 129, 700, "top_left", 3)]):
        cfg = fi.Config("bshd", 2, H, Sq, Sk, D, dtype, mask != "none", seed=960 + i)
        inp = fi.make_inputs(cfg)
        inp.k = inp.k[:, :Hkv].contiguous()
        inp.v = inp.v[:, :Hkv].contiguous()
        q64, k64, v64 = fi.values(inp)
        offset = (Sk - Sq) if mask == "bottom_right" else 0
        ref_o, ref_l = attention_fp64(q64, k64, v64, cfg.scale, mask != "none", offset)
        q, k, v = (t.transpose(1, 2).contiguous().cuda() for t in (inp.q, inp.k, inp.v))
        kw = {}
        if dtype == fi.FP8:
            kw = {n: torch.tensor([d], dtype=torch.float32, device="cuda") for n, d in
                  (("descale_q", inp.descale_q), ("descale_k", inp.descale_k),
                   ("descale_v", inp.descale_v))}
        causal = False if mask == "none" else mask
        if ns is None:
            o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=causal, layout="BSHD",
                               o_dtype=torch.float32, **kw)
        else:
            o, lse = fa.fa_fwd_splitkv(q, k, v, num_splits=ns, scale=cfg.scale, causal=causal,
                                       layout="BSHD", o_dtype=torch.float32, **kw)
        torch.cuda.synchronize()
        assert tuple(o.shape) == (2, Sq, H, D) and tuple(lse.shape) == (2, H, Sq)
        o = o.transpose(1, 2).double().cpu().numpy()
        lse = lse.double().cpu().numpy()
        empty = np.isneginf(ref_l)
        assert np.all(o[empty] == 0.0) and np.all(np.isneginf(lse[empty]))
        compare(cfg, fi.F32, o[~empty], lse[~empty], ref_o[~empty], ref_l[~empty],
                what=f"BSHD {dtype} D{D} H{H}/{Hkv} {Sq}x{Sk} {mask} splits {ns}")


def _block_rows(Sq: int, bm: int):
    """First, middle and last row of every block of bm query rows."""
    rows = set()
    for s in range(0, Sq, bm):
        rows.update((s, min(s + bm // 2, Sq - 1), min(s + bm - 1, Sq - 1)))
    return np.array(sorted(rows))


@pytest.mark.parametrize("D,B,H,Hkv,Sq,Sk,full", [
    (128, 2, 8, 4, 700, 700, True),      # 96 workgroups: resident at once, long and short paired
    (128, 2, 8, 4, 600, 700, True),      # the same with the diagonal shifted (bottom-right)
    (128, 2, 16, 4, 3200, 3200, False),  # 800 workgroups of 4 waves: several rounds, longest first
    (64, 2, 8, 4, 2000, 2000, True),     # D = 64 (64-key tiles), resident at once
    (64, 2, 8, 4, 7000, 7000, False),    # D = 64, 880 workgroups: several rounds
    (128, 3, 12, 12, 700, 700, True),    # 36 head groups: the 4 beyond a multiple of 8 go first
    (64, 3, 6, 3, 2900, 3000, False),    # 9 groups of 2 heads, one beyond a multiple of 8
])
def test_causal_launch_orders(D, B, H, Hkv, Sq, Sk, full):
    """Causal grids with at least 8 groups of query heads sharing a
    key/value head run in q-block-major order inside each XCD (long and
    short blocks paired when the whole grid is resident and the groups
    divide evenly over the XCDs, longest first otherwise; groups beyond a
    multiple of 8 first). Every (head, block) must still compute its own
    rows: checked against the oracle on every row (full) or on the first,
    middle and last row of every query block of every head."""
    mask = "bottom_right" if Sq != Sk else "top_left"
    cfg = fi.Config("order", B, H, Sq, Sk, D, fi.F16, True, seed=1200 + Sq + D)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    q64, k64, v64 = fi.values(inp)
    offset = Sk - Sq
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=mask, o_dtype=torch.float32)
    torch.cuda.synchronize()
    o = o.double().cpu().numpy()
    lse = lse.double().cpu().numpy()
    what = f"D{D} B{B} H{H}/{Hkv} {Sq}x{Sk} {mask}"
    if full:
        ref_o, ref_l = attention_fp64(q64, k64, v64, cfg.scale, True, offset)
        compare(cfg, fi.F32, o, lse, ref_o, ref_l, what=what)
        return
    rows = _block_rows(Sq, 128)
    for b in range(B):
        for h in range(H):
            ro, rl = attention_rows_fp64(q64, k64, v64, cfg.scale, True, b, h, rows, offset)
            compare(cfg, fi.F32, o[b, h, rows], lse[b, h, rows], ro, rl, what=f"{what} b{b} h{h}")
