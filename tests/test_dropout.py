"""GPU parity of the forward with dropout (fa_fwd_dropout, through the C ABI)
against the fp64 oracle with the same Philox4x64-10 keep mask.

Tolerance: the kernel's O error without dropout (2e-3 fp16/bf16, 6e-2 fp8)
comes from the rounding of P; with dropout the kept terms are the same
products scaled by 1/keep_prob, so the bound is the forward's divided by
keep_prob. lse is the undropped one (1e-3). A single wrong keep bit moves
O by about P_ij |V_j| / keep_prob, far outside these bounds for the
workloads' P.
"""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from oracle import attention_dropout_fp64
from parity_util import TOL_LSE, TOL_O, to_device, ulp

pytestmark = pytest.mark.gpu

MASKS = {"none": (False, 0), "top_left": (True, 0), "bottom_right": (True, None)}


def run(cfg, inp, mask, keep, seed, rng_offset, od, Hkv=None, layout="BNSD"):
    q, k, v, ds = to_device(inp)
    kw = {}
    if ds is not None:
        kw = dict(descale_q=ds[0], descale_k=ds[1], descale_v=ds[2])
    if layout == "BSHD":
        q, k, v = (t.transpose(1, 2).contiguous() for t in (q, k, v))
    o, lse = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=False if mask == "none" else mask,
                       keep_prob=keep, seed=seed, rng_offset=rng_offset,
                       o_dtype=fi.TORCH_DTYPE[od], layout=layout, **kw)
    torch.cuda.synchronize()
    if layout == "BSHD":
        o = o.transpose(1, 2)
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(cfg, od, keep, o, lse, ref_o, ref_l, what):
    tol = TOL_O[cfg.dtype] / keep
    bound = tol + (0.0 if od == fi.F32 else ulp(ref_o, od) / keep)
    err = np.abs(o - ref_o)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), what
    assert not np.any(err > bound), f"{what}: O max err {err.max():.3e} (tol {tol:.2e})"
    assert np.max(np.abs(lse - ref_l)) <= TOL_LSE, what
    return float(err.max())


def inputs(dtype, B, H, Hkv, Sq, Sk, D, seed):
    cfg = fi.Config("drop", B, H, Sq, Sk, D, dtype, False, seed=seed)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :Hkv].contiguous()
    inp.v = inp.v[:, :Hkv].contiguous()
    return cfg, inp


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16, fi.FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
def test_dropout_parity(dtype, D, mask):
    native = fi.BF16 if dtype == fi.BF16 else fi.F16
    worst = 0.0
    for i, (H, Hkv, Sq, Sk, keep) in enumerate([(2, 2, 1, 1, 0.9), (4, 2, 65, 130, 0.5),
                                               (3, 1, 200, 97, 0.8), (2, 2, 257, 257, 0.3)]):
        cfg, inp = inputs(dtype, 2, H, Hkv, Sq, Sk, D, seed=1600 + 7 * i + D)
        causal, off = MASKS[mask]
        off = (Sk - Sq) if mask == "bottom_right" else off
        seed, ro = 1000 + i, 7 * i
        q, k, v = fi.values(inp)
        ref_o, ref_l = attention_dropout_fp64(q, k, v, cfg.scale, causal, off, keep, seed, ro)
        for od in (fi.F32, native):
            o, lse = run(cfg, inp, mask, keep, seed, ro, od)
            empty = np.isneginf(ref_l)
            assert np.all(np.isneginf(lse[empty])) and np.all(o[empty] == 0.0)
            e = check(cfg, od, keep, o[~empty], lse[~empty], ref_o[~empty], ref_l[~empty],
                      f"{dtype} D{D} {mask} {Sq}x{Sk} H{H}/{Hkv} keep {keep} {od}")
            worst = max(worst, e) if od == fi.F32 else worst
    print(f"dropout {dtype} D{D} {mask}: worst |dO| (f32 out) {worst:.3e}")


def test_dropout_bshd_layout():
    cfg, inp = inputs(fi.F16, 2, 4, 2, 150, 300, 128, seed=1650)
    q, k, v = fi.values(inp)
    ref_o, ref_l = attention_dropout_fp64(q, k, v, cfg.scale, True, 0, 0.7, 42, 3)
    o, lse = run(cfg, inp, "top_left", 0.7, 42, 3, fi.F32, layout="BSHD")
    check(cfg, fi.F32, 0.7, o, lse, ref_o, ref_l, "bshd")


def test_dropout_full_size_sampled_rows():
    """B4 H32 S4096 D128 fp16, keep 0.9: sampled rows of sampled heads."""
    cfg = fi.HEADLINE
    inp = fi.make_inputs(cfg)
    o, lse = run(cfg, inp, "none", 0.9, 2024, 11, fi.F32)
    assert np.all(np.isfinite(o))
    rng = np.random.default_rng(5)
    worst = 0.0
    for b, h in ((0, 0), (3, 31), (int(rng.integers(4)), int(rng.integers(32)))):
        rows = np.unique(np.concatenate([[0, 1, 127, 128, 4095], rng.integers(0, 4096, 12)]))
        sl = (slice(b, b + 1), slice(h, h + 1))
        q = fi.as_float64(inp.q[sl])
        k = fi.as_float64(inp.k[sl])
        v = fi.as_float64(inp.v[sl])
        ro, rl = _rows_for_head(q, k, v, cfg, b, h, rows)
        e = check(cfg, fi.F32, 0.9, o[b, h, rows], lse[b, h, rows], ro, rl, f"full {b},{h}")
        worst = max(worst, e)
    print(f"dropout full size: worst |dO| {worst:.3e}")


def _rows_for_head(q, k, v, cfg, b, h, rows):
    """Oracle rows of head (b, h) of the full problem (its mask uses the
    query head index b*H + h)."""
    from oracle import dropout_keep_mask, head_forward
    _, l, p = head_forward(q[0, 0], k[0, 0], v[0, 0], cfg.scale, False, rows=rows,
                           return_p=True)
    z = dropout_keep_mask(b * cfg.H + h, rows, k.shape[2], 0.9, 2024, 11)
    return (p * z / 0.9) @ v[0, 0], l


def test_dropout_determinism_and_keep_one():
    cfg, inp = inputs(fi.F16, 1, 4, 4, 300, 300, 64, seed=1660)
    a = run(cfg, inp, "top_left", 0.6, 5, 0, fi.F16)
    b = run(cfg, inp, "top_left", 0.6, 5, 0, fi.F16)
    c = run(cfg, inp, "top_left", 0.6, 6, 0, fi.F16)
    d = run(cfg, inp, "top_left", 0.6, 5, 1, fi.F16)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    assert not np.array_equal(a[0], c[0]) and not np.array_equal(a[0], d[0])
    assert np.array_equal(a[1], c[1])          # lse does not depend on the mask
    # keep_prob = 1 through the dropout entry point is the plain forward
    q, k, v, _ = to_device(inp)
    o1, l1 = torch.empty_like(q), torch.empty(q.shape[:3], device="cuda")
    st = fa.fa_fwd_dropout_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(),
                               l1.data_ptr(), 1, 4, 4, 300, 300, 64, fa.FA_LAYOUT_BNSD, cfg.scale,
                               fa.FA_MASK_CAUSAL_TOP_LEFT, 1.0, 5, 0, fa.FA_F16, fa.FA_F16, None,
                               None, None, torch.cuda.current_stream().cuda_stream)
    assert st == fa.FA_OK
    o2, l2 = fa.fa_fwd(q, k, v, scale=cfg.scale, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))


def _bit_planes(S: int, D: int, lo: int) -> np.ndarray:
    """[S, D]: column d holds 2^(t - lo) at the indices t*D + d with
    lo <= t < lo + 16, and 0 elsewhere (16 distinct powers of two per
    column, each below 2^16, so their sums are exact in fp16 inputs and an
    fp32 accumulator)."""
    x = np.zeros((S, D))
    j = np.arange(S)
    t = j // D - lo
    sel = (t >= 0) & (t < 16)
    x[j[sel], j[sel] % D] = 2.0 ** t[sel]
    return x


def _decode(x: np.ndarray) -> np.ndarray:
    """Integer codes x [R, D] (< 2^16) -> bits [R, 16, D]."""
    c = np.rint(x).astype(np.int64)
    return (c[:, None, :] >> np.arange(16)[None, :, None]) & 1


@pytest.mark.parametrize("D", [64, 128])
def test_forward_every_keep_bit(D):
    """Every keep bit of every row of six heads at Sq = Sk = 4096 against the
    oracle's mask. With Q = 0 every score is 0, so P = 2^-12 exactly for
    every key; V (_bit_planes) gives key t*D + d the value 2^(t - lo) in
    column d, so O[i, d] * Sk * keep_prob is the integer whose bit t - lo is
    the keep bit of key t*D + d. One wrong bit changes an output by at least
    2^-12 / keep_prob, while the arithmetic here is exact up to one fp32
    rounding."""
    B, H, S, keep, seed, off = 2, 3, 4096, 0.8, 1234, 77
    q = torch.zeros(B, H, S, D, dtype=torch.float16, device="cuda")
    k = torch.zeros(B, H, S, D, dtype=torch.float16, device="cuda")
    ref = {(b, h): oracle_mask(b * H + h, S, keep, seed, off) for b in range(B) for h in range(H)}
    for lo in range(0, S // D, 16):
        vp = torch.from_numpy(_bit_planes(S, D, lo)).to(torch.float16)
        v = vp.expand(B, H, S, D).contiguous().cuda()
        o, _ = fa.fa_fwd(q, k, v, scale=D ** -0.5, keep_prob=keep, seed=seed, rng_offset=off,
                         o_dtype=torch.float32)
        torch.cuda.synchronize()
        o = o.double().cpu().numpy() * S * keep
        for b in range(B):
            for h in range(H):
                bits = _decode(o[b, h])                                   # [Sq, 16, D]
                want = ref[(b, h)][:, lo * D:(lo + 16) * D].reshape(S, 16, D)
                bad = np.argwhere(bits != want)
                assert bad.size == 0, (
                    f"D{D} head ({b},{h}): keep bits differ at (row, key) "
                    f"{[(int(r), int((lo + t) * D + d)) for r, t, d in bad[:5]]}")


@pytest.mark.parametrize("D", [64, 128])
def test_backward_every_keep_bit(D):
    """The same through dV = (P Z / keep)^T dO of fa_bwd_dropout: with Q = 0
    and lse = ln Sk every P is 2^-12, keep_prob 0.5 makes P / keep_prob a
    power of two too, and dO (_bit_planes over the query rows) gives row
    t*D + d the value 2^(t - lo) in column d, so dV[j, d] * Sq * keep_prob is
    the integer whose bit t - lo is the keep bit of (row t*D + d, key j)."""
    B, H, S, keep, seed, off = 1, 2, 4096, 0.5, 4321, 9
    q = torch.zeros(B, H, S, D, dtype=torch.float16, device="cuda")
    k = torch.zeros(B, H, S, D, dtype=torch.float16, device="cuda")
    v = torch.zeros(B, H, S, D, dtype=torch.float16, device="cuda")
    o = torch.zeros(B, H, S, D, dtype=torch.float16, device="cuda")
    lse = torch.full((B, H, S), float(np.log(S)), dtype=torch.float32, device="cuda")
    ref = {h: oracle_mask(h, S, keep, seed, off) for h in range(H)}
    for lo in range(0, S // D, 16):
        gp = torch.from_numpy(_bit_planes(S, D, lo)).to(torch.float16)
        do = gp.expand(B, H, S, D).contiguous().cuda()
        _, _, dv = fa.fa_bwd(q, k, v, o, do, lse, scale=D ** -0.5, keep_prob=keep, seed=seed,
                             rng_offset=off, grad_dtype=torch.float32)
        torch.cuda.synchronize()
        dv = dv.double().cpu().numpy() * S * keep
        for h in range(H):
            bits = _decode(dv[0, h])                                     # [Sk, 16, D]
            want = ref[h][lo * D:(lo + 16) * D, :].reshape(16, D, S).transpose(2, 0, 1)
            bad = np.argwhere(bits != want)
            assert bad.size == 0, (
                f"D{D} head {h}: keep bits differ at (row, key) "
                f"{[(int((lo + t) * D + d), int(j)) for j, t, d in bad[:5]]}")


def oracle_mask(bh: int, S: int, keep: float, seed: int, off: int) -> np.ndarray:
    from oracle import dropout_keep_mask
    return dropout_keep_mask(bh, range(S), S, keep, seed, off)
