"""GPU parity of packed variable-length batches (fa_fwd_varlen, through the
C ABI) against the fp64 oracle: sequences without queries or without keys,
lengths around the tile edges, grouped heads, every mask, each input type;
and, at full size, bitwise equality with the fixed-length path when every
sequence has the same length."""
import numpy as np
import pytest
import torch

import attention_fa_fwd_07_amd as fa
import fa_inputs as fi
from oracle import attention_varlen_fp64, head_forward
from parity_util import TOL_LSE, TOL_O, ulp

pytestmark = pytest.mark.gpu

MASKS = {"none": False, "top_left": True, "bottom_right": "bottom_right"}

# (query length, key length) per sequence: tile edges, a sequence without
# queries, one without keys, Sq > Sk and Sq < Sk, single tokens
MIX = [(1, 1), (63, 63), (64, 64), (65, 130), (0, 5), (200, 0), (300, 150), (129, 513),
       (2, 1)]


def descales(vi, dev="cuda"):
    if vi.inp.q.dtype != torch.float8_e4m3fn:
        return {}
    return {n: torch.tensor([d], dtype=torch.float32, device=dev) for n, d in
            (("descale_q", vi.inp.descale_q), ("descale_k", vi.inp.descale_k),
             ("descale_v", vi.inp.descale_v))}


def run_varlen(vi, scale, causal, o_dtype):
    q, k, v = (t.cuda() for t in (vi.inp.q, vi.inp.k, vi.inp.v))
    cq, ck = vi.cu_q.cuda(), vi.cu_k.cuda()
    o = torch.full(tuple(q.shape), float("nan"), dtype=fi.TORCH_DTYPE[o_dtype], device="cuda")
    lse = torch.full((q.shape[1], q.shape[0]), float("nan"), device="cuda")
    fa.fa_fwd_varlen(q, k, v, cq, ck, vi.max_q, scale=scale, causal=causal, out=o, lse=lse,
                     **descales(vi))
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def check(dtype, o_dtype, o, lse, ref_o, ref_l, what):
    empty = np.isneginf(ref_l)                       # [H, Tq]
    assert np.all(np.isneginf(lse[empty])), what
    assert np.all(o.transpose(1, 0, 2)[empty] == 0.0), what
    fin = ~empty
    assert np.all(np.isfinite(lse[fin])) and np.all(np.isfinite(o)), what
    assert np.abs(lse[fin] - ref_l[fin]).max(initial=0.0) <= TOL_LSE, what
    err = np.abs(o - ref_o)
    bound = TOL_O[dtype] + (0.0 if o_dtype == fi.F32 else ulp(ref_o, o_dtype))
    bad = err > bound
    assert not bad.any(), f"{what}: O mismatch at {np.argwhere(bad)[:5].tolist()}, max {err.max():.3e}"


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16, fi.FP8])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("mask", list(MASKS))
def test_varlen_mix(dtype, D, mask):
    native = fi.BF16 if dtype == fi.BF16 else fi.F16
    for i, (H, Hkv) in enumerate([(4, 2), (3, 3)]):
        lens = MIX if i == 0 else MIX[::-1]
        vi = fi.make_varlen_inputs([a for a, _ in lens], [b for _, b in lens], H, Hkv, D,
                                   dtype, seed=1200 + 7 * i + D)
        q64, k64, v64 = fi.values(vi.inp)
        scale = 1.0 / np.sqrt(D)
        causal = mask != "none"
        ref_o, ref_l = attention_varlen_fp64(q64, k64, v64, vi.cu_q.numpy(), vi.cu_k.numpy(),
                                             scale, causal, mask == "bottom_right")
        for od in (fi.F32, native):
            o, lse = run_varlen(vi, scale, MASKS[mask], od)
            check(dtype, od, o, lse, ref_o, ref_l, f"{dtype} D{D} {mask} H{H}/{Hkv} {od}")


def test_varlen_single_sequence_and_max_length_above_need():
    """One sequence; and max_seqlen_q above the longest length (extra
    workgroups find no rows and return)."""
    for (lq, lk, mq) in (([300], [300], 300), ([5, 70], [70, 5], 75)):
        vi = fi.make_varlen_inputs(lq, lk, 4, 1, 128, fi.F16, seed=1250 + len(lq))
        vi.max_q = mq
        q64, k64, v64 = fi.values(vi.inp)
        ref_o, ref_l = attention_varlen_fp64(q64, k64, v64, vi.cu_q.numpy(), vi.cu_k.numpy(),
                                             0.125 / 1.4142135623730951, True, True)
        o, lse = run_varlen(vi, 0.125 / 1.4142135623730951, "bottom_right", fi.F32)
        check(fi.F16, fi.F32, o, lse, ref_o, ref_l, f"single {lq} max {mq}")


@pytest.mark.parametrize("D", [128, 64])
def test_varlen_long_mix_sampled_rows(D):
    """A length mix up to 4096 at H32 fp16, causal: sampled rows of every
    sequence against the oracle (at D = 64 the grid of 8192 workgroups runs
    four per CU)."""
    rng = np.random.default_rng(1260)
    lens = [4096, 1, 1000, 2049, 128, 3000, 64, 777]
    H = 32
    vi = fi.make_varlen_inputs(lens, lens, H, H, D, fi.F16, seed=1261)
    scale = D ** -0.5
    o, lse = run_varlen(vi, scale, True, fi.F16)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    q64, k64, v64 = fi.values(vi.inp)
    cu = vi.cu_q.numpy()
    worst = 0.0
    for b, n in enumerate(lens):
        s = int(cu[b])
        rows = np.unique(np.concatenate([[0, n - 1, n // 2], rng.integers(0, n, 6)]))
        for h in (0, int(rng.integers(H)), H - 1):
            ro, rl = head_forward(q64[s:s + n, h], k64[s:s + n, h], v64[s:s + n, h], scale,
                                  True, rows=rows)
            err = np.abs(o[s + rows, h] - ro)
            assert np.all(err <= TOL_O[fi.F16] + ulp(ro, fi.F16)), (b, h, err.max())
            assert np.abs(lse[h, s + rows] - rl).max() <= TOL_LSE, (b, h)
            worst = max(worst, float(err.max()))
    print(f"long varlen mix: max |dO| over checked rows {worst:.3e}")


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("causal", [False, True])
def test_varlen_equal_lengths_match_fixed_path_bitwise(causal, D):
    """B sequences of one length packed token-major are the BSHD batch; the
    variable-length launch must give the fixed-length path's bits
    (B4 H32 S4096 fp16: the benchmark's shape at D = 128)."""
    B, H, S = 4, 32, 4096
    vi = fi.make_varlen_inputs([S] * B, [S] * B, H, H, D, fi.F16, seed=1270)
    q, k, v = (t.cuda() for t in (vi.inp.q, vi.inp.k, vi.inp.v))
    o1, l1 = fa.fa_fwd_varlen(q, k, v, vi.cu_q.cuda(), vi.cu_k.cuda(), S, causal=causal)
    o2, l2 = fa.fa_fwd(q.view(B, S, H, D), k.view(B, S, H, D), v.view(B, S, H, D),
                       causal=causal, layout="BSHD")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(B * S, H, D).view(torch.int16))
    # lse: [H, B*S] against [B, H, S]
    assert torch.equal(l1.view(H, B, S).permute(1, 0, 2).contiguous().view(torch.int32),
                       l2.view(torch.int32))


@pytest.mark.parametrize("H,Hkv,nseq", [(8, 2, 4), (8, 2, 9), (3, 1, 5)])
def test_varlen_launch_orders(H, Hkv, nseq):
    """The three launch orders: key/value-head groups dealt to the XCDs
    (B*H_kv a multiple of 8), heads dealt (only B*H a multiple of 8), and
    the contiguous order (neither)."""
    rng = np.random.default_rng(1280 + nseq)
    lq = [int(x) for x in rng.integers(1, 400, nseq)]
    lk = [int(x) for x in rng.integers(0, 400, nseq)]
    vi = fi.make_varlen_inputs(lq, lk, H, Hkv, 64, fi.BF16, seed=1281 + nseq)
    q64, k64, v64 = fi.values(vi.inp)
    for mask in MASKS:
        ref_o, ref_l = attention_varlen_fp64(q64, k64, v64, vi.cu_q.numpy(), vi.cu_k.numpy(),
                                             0.125, mask != "none", mask == "bottom_right")
        o, lse = run_varlen(vi, 0.125, MASKS[mask], fi.F32)
        check(fi.BF16, fi.F32, o, lse, ref_o, ref_l, f"H{H}/{Hkv} B{nseq} {mask}")
