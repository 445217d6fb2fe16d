"""GPU parity of the backward pass (fa_bwd, through the C ABI) against the
fp64 oracle's gradients.

The kernels take O and lse as inputs. Here they are the oracle's forward
results stored as the library stores them (O in the input type, lse fp32),
so that the comparison measures the backward's own arithmetic; one test
chains the library's forward instead.

Tolerance, element by element: every product rounds one operand per term
to the input type (P, and dS = P (dP - Delta), in the MFMA inputs) and sums
in fp32, so the error of a gradient element is a small multiple of the unit
roundoff u times the sum T of the absolute values of its terms:
  dQ: scale * (P * (|dP| + |Delta|)) |K|,  dK: scale * (P * (|dP| + |Delta|))^T |Q|,
  dV: P^T |dO|.
Each element must satisfy |g - g_ref| <= 2u T + E (fp16 u = 2^-11, bf16
2^-8), where E is the exact propagation of the O and lse the kernels are
given (the oracle's, rounded as the library stores them, or the library's
own forward output) through Delta = rowsum(dO * O) and P = exp(S - lse);
16-bit gradients may in addition be off by one unit in the last place.
"""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from parity_util import as_used, check_grads, grad_bounds
from oracle import attention_bwd_fp64, attention_dropout_fp64, attention_fp64

pytestmark = pytest.mark.gpu

MASKS = {"none": (False, 0), "top_left": (True, 0), "bottom_right": (True, None)}


def case_inputs(dtype, B, H, Hkv, Sq, Sk, D, seed, amp=1.0):
    cfg = fi.Config("bwd", B, H, Sq, Sk, D, dtype, False, seed=seed, amp=amp)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    do = fi.make_cotangent((B, H, Sq, D), dtype, seed + 5000)
    return cfg, inp, do


def oracle_all(cfg, inp, do, causal, off):
    q, k, v = fi.values(inp)
    g = do.double().numpy()
    o, lse = attention_fp64(q, k, v, cfg.scale, causal, off)
    dq, dk, dv = attention_bwd_fp64(q, k, v, g, cfg.scale, causal, off)
    bounds = grad_bounds(q, k, v, g, cfg.scale, causal, off, o_used=as_used(o, cfg.dtype),
                         lse_used=as_used(lse, fi.F32))
    return o, lse, (dq, dk, dv), bounds


def run_bwd(cfg, inp, do, o, lse, causal, grad_dtype, drop=None):
    td = fi.TORCH_DTYPE[cfg.dtype]
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    ot = torch.from_numpy(o).to(torch.float32).to(td).cuda()
    lt = torch.from_numpy(lse).to(torch.float32).cuda()
    gd = fi.TORCH_DTYPE[grad_dtype]
    dq = torch.full(tuple(q.shape), float("nan"), dtype=gd, device="cuda")
    dk = torch.full(tuple(k.shape), float("nan"), dtype=gd, device="cuda")
    dv = torch.full(tuple(v.shape), float("nan"), dtype=gd, device="cuda")
    ws = torch.full((fa.bwd_workspace_size(cfg.B, cfg.H, cfg.Sq) + 256,), 255, dtype=torch.uint8,
                    device="cuda")
    kw = {} if drop is None else dict(keep_prob=drop[0], seed=drop[1], rng_offset=drop[2])
    fa.fa_bwd(q, k, v, ot, do.cuda(), lt, scale=cfg.scale, causal=causal, dq=dq, dk=dk, dv=dv,
              workspace=ws, **kw)
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in (dq, dk, dv))


def check(dtype, got, ref, bounds, what, grad_dtype=fi.F32):
    return check_grads(dtype, got, ref, bounds, what, grad_dtype)


LENGTHS = [(1, 1), (33, 65), (64, 64), (65, 130), (130, 65), (200, 200), (257, 129)]


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
def test_bwd_edge_sweep(dtype, D, mask):
    worst = [0.0, 0.0, 0.0]
    for i, (Sq, Sk) in enumerate(LENGTHS):
        H, Hkv = ((2, 2), (4, 2), (3, 1))[i % 3]
        causal = MASKS[mask][0]
        off = (Sk - Sq) if mask == "bottom_right" else 0
        cfg, inp, do = case_inputs(dtype, 1, H, Hkv, Sq, Sk, D, seed=1400 + 13 * i + D)
        o, lse, ref, bnd = oracle_all(cfg, inp, do, causal, off)
        causal_arg = False if mask == "none" else mask
        for gd in (fi.F32, dtype):
            got = run_bwd(cfg, inp, do, o, lse, causal_arg, gd)
            e = check(dtype, got, ref, bnd, f"{dtype} D{D} {mask} {Sq}x{Sk} H{H}/{Hkv} {gd}", gd)
            if gd == fi.F32:
                worst = [max(a, b) for a, b in zip(worst, e)]
    print(f"{dtype} D{D} {mask}: worst rel err dq/dk/dv {worst}")


@pytest.mark.parametrize("dtype,D,mask,H,Hkv,S", [
    (fi.F16, 128, "none", 4, 4, 4096),
    (fi.BF16, 128, "top_left", 4, 2, 2048),
    (fi.F16, 64, "bottom_right", 3, 1, 1500),
])
def test_bwd_long_sequences(dtype, D, mask, H, Hkv, S):
    """Long rows: whole heads of 1500..4096 tokens against the oracle."""
    causal = MASKS[mask][0]
    Sk = S if mask != "bottom_right" else S + 300
    cfg, inp, do = case_inputs(dtype, 1, H, Hkv, S, Sk, D, seed=1450 + D + H)
    off = (Sk - S) if mask == "bottom_right" else 0
    o, lse, ref, bnd = oracle_all(cfg, inp, do, causal, off)
    got = run_bwd(cfg, inp, do, o, lse, False if mask == "none" else mask, fi.F32)
    e = check(dtype, got, ref, bnd, f"long {dtype} D{D} {mask} S{S}")
    print(f"long {dtype} D{D} {mask} S{S}: rel err dq/dk/dv {e}")


def test_bwd_chained_with_library_forward():
    """fa_fwd's own O and lse feed fa_bwd (the training-step order)."""
    for dtype in (fi.F16, fi.BF16):
        cfg, inp, do = case_inputs(dtype, 2, 4, 2, 300, 300, 128, seed=1470)
        q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
        o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=True)
        dq, dk, dv = fa.fa_bwd(q, k, v, o, do.cuda(), lse, scale=cfg.scale, causal=True,
                               grad_dtype=torch.float32)
        torch.cuda.synchronize()
        qq, kk, vv = fi.values(inp)
        g = do.double().numpy()
        ref = attention_bwd_fp64(qq, kk, vv, g, cfg.scale, True, 0)
        bnd = grad_bounds(qq, kk, vv, g, cfg.scale, True, 0, o_used=o.double().cpu().numpy(),
                          lse_used=lse.double().cpu().numpy())
        check(dtype, tuple(t.double().cpu().numpy() for t in (dq, dk, dv)), ref, bnd,
              f"chained {dtype}")


def test_bwd_deterministic():
    cfg, inp, do = case_inputs(fi.F16, 2, 8, 2, 700, 700, 128, seed=1480)
    o, lse, _, _ = oracle_all(cfg, inp, do, True, 0)
    a = run_bwd(cfg, inp, do, o, lse, True, fi.F16)
    b = run_bwd(cfg, inp, do, o, lse, True, fi.F16)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_bwd_large_logits():
    """Scores far past the fp16 exp-overflow point (amplitude 3 at D=64)."""
    cfg, inp, do = case_inputs(fi.F16, 1, 2, 2, 300, 300, 64, seed=1490, amp=3.0)
    o, lse, ref, bnd = oracle_all(cfg, inp, do, True, 0)
    got = run_bwd(cfg, inp, do, o, lse, True, fi.F32)
    e = check(fi.F16, got, ref, bnd, "large logits")
    print(f"large logits: rel err dq/dk/dv {e}")


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
def test_bwd_dropout(dtype, D, mask):
    """The backward of the dropout forward: O and lse from the oracle's
    dropout forward, gradients against the oracle's (same mask)."""
    worst = [0.0, 0.0, 0.0]
    for i, (Sq, Sk, keep) in enumerate([(1, 1, 0.9), (65, 130, 0.5), (130, 65, 0.7),
                                        (200, 200, 0.8)]):
        H, Hkv = ((2, 2), (4, 2), (3, 1), (2, 1))[i]
        causal = MASKS[mask][0]
        off = (Sk - Sq) if mask == "bottom_right" else 0
        cfg, inp, do = case_inputs(dtype, 1, H, Hkv, Sq, Sk, D, seed=1700 + 13 * i + D)
        drop = (keep, 77 + i, 5 * i)
        q, k, v = fi.values(inp)
        g = do.double().numpy()
        o, lse = attention_dropout_fp64(q, k, v, cfg.scale, causal, off, *drop)
        ref = attention_bwd_fp64(q, k, v, g, cfg.scale, causal, off, *drop)
        bnd = grad_bounds(q, k, v, g, cfg.scale, causal, off, drop, o_used=as_used(o, dtype),
                          lse_used=as_used(lse, fi.F32))
        got = run_bwd(cfg, inp, do, o, lse, False if mask == "none" else mask, fi.F32, drop)
        e = check(dtype, got, ref, bnd, f"dropout {dtype} D{D} {mask} {Sq}x{Sk} keep {keep}")
        worst = [max(a, b) for a, b in zip(worst, e)]
    print(f"dropout bwd {dtype} D{D} {mask}: worst rel err dq/dk/dv {worst}")


def test_bwd_dropout_chained_with_library_forward():
    """fa_fwd with dropout, then fa_bwd with the same seed and offset."""
    cfg, inp, do = case_inputs(fi.F16, 2, 4, 2, 300, 333, 128, seed=1750)
    q, k, v = (t.cuda() for t in (inp.q, inp.k, inp.v))
    o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal="bottom_right", keep_prob=0.75,
                       seed=99, rng_offset=4)
    dq, dk, dv = fa.fa_bwd(q, k, v, o, do.cuda(), lse, scale=cfg.scale, causal="bottom_right",
                           grad_dtype=torch.float32, keep_prob=0.75, seed=99, rng_offset=4)
    torch.cuda.synchronize()
    qq, kk, vv = fi.values(inp)
    g = do.double().numpy()
    ref = attention_bwd_fp64(qq, kk, vv, g, cfg.scale, True, 33, 0.75, 99, 4)
    bnd = grad_bounds(qq, kk, vv, g, cfg.scale, True, 33, (0.75, 99, 4),
                      o_used=o.double().cpu().numpy(), lse_used=lse.double().cpu().numpy())
    check(fi.F16, tuple(t.double().cpu().numpy() for t in (dq, dk, dv)), ref, bnd,
          "dropout chained")


def test_bwd_scale_variants():
    """Negative, zero and large scales (a negative scale negates the
    register-resident operand of S; zero gives uniform P and dQ = dK = 0)."""
    for scale in (-0.3, 0.0, 0.6):
        for mask in ("none", "top_left"):
            cfg, inp, do = case_inputs(fi.F16, 1, 4, 2, 130, 97, 64, seed=1800)
            cfg = cfg.replace(scale=scale) if scale != 0.0 else cfg.replace(scale=1e-30)
            causal = MASKS[mask][0]
            o, lse, ref, bnd = oracle_all(cfg, inp, do, causal, 0)
            got = run_bwd(cfg, inp, do, o, lse, False if mask == "none" else mask, fi.F32)
            check(fi.F16, got, ref, bnd, f"scale {scale} {mask}")


@pytest.mark.parametrize("D,B,H,Hkv,Sq,Sk,mask", [
    (128, 2, 8, 4, 700, 700, "top_left"),       # 8 groups: resident grids, long and short paired
    (64, 2, 8, 8, 600, 800, "bottom_right"),    # 16 key/value heads, diagonal shifted
    (128, 3, 6, 3, 1000, 1000, "top_left"),     # 9 groups: the one beyond a multiple of 8 first
    (64, 2, 16, 8, 2200, 2200, "top_left"),     # dQ: 544 workgroups, several rounds
])
def test_bwd_causal_launch_orders(D, B, H, Hkv, Sq, Sk, mask):
    """Causal backward grids with at least 8 key/value heads order the
    key blocks (dK/dV kernel) and query blocks (dQ kernel) by work across
    each XCD's heads; every gradient must still land on its own rows."""
    cfg, inp, do = case_inputs(fi.F16, B, H, Hkv, Sq, Sk, D, seed=1300 + Sq + D)
    off = (Sk - Sq) if mask == "bottom_right" else 0
    o, lse, ref, bounds = oracle_all(cfg, inp, do, True, off)
    got = run_bwd(cfg, inp, do, o, lse, mask, fi.F32)
    check(fi.F16, got, ref, bounds, f"D{D} B{B} H{H}/{Hkv} {Sq}x{Sk} {mask}")
