"""CPU checks of the per-element gradient bounds the backward parity tests
use (parity_util.grad_bounds / check_grads).

The bound must hold for the arithmetic the kernels do, and it must catch a
wrong value in a single element, also where that element's gradient is
small. Both are checked against an fp64 emulation of the kernels' roundings
(P and dS rounded to the input type before the products, O rounded as
stored, lse in fp32) built on the oracle's own forward.
"""
import numpy as np
import pytest
import torch

import fa_inputs as fi
from oracle import attention_bwd_fp64, attention_fp64, head_forward
from parity_util import as_used, check_grads, grad_bounds


def _round(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32).to(
        fi.TORCH_DTYPE[dtype]).double().numpy()


def _emulate(q, k, v, g, scale, causal, off, o_used, lse_used, dtype):
    """Gradients with the kernels' roundings: P from the given lse, Delta from
    the given O, P and dS rounded to the input type, sums exact."""
    B, H, Sq, D = q.shape
    Hkv = k.shape[1]
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            kv = h // (H // Hkv)
            s = (q[b, h] @ k[b, kv].T) * scale
            if causal:
                key = np.arange(k.shape[2])
                s = np.where(key[None, :] > np.arange(Sq)[:, None] + off, -np.inf, s)
            lse = lse_used[b, h][:, None]
            p = np.where(np.isneginf(lse), 0.0, np.exp(s - np.where(np.isneginf(lse), 0.0, lse)))
            delta = np.sum(g[b, h] * o_used[b, h], axis=1, keepdims=True)
            dp = g[b, h] @ v[b, kv].T
            ds = _round(p * (dp - delta), dtype)
            dq[b, h] = scale * ds @ k[b, kv]
            dk[b, kv] += scale * ds.T @ q[b, h]
            dv[b, kv] += _round(p, dtype).T @ g[b, h]
    return dq, dk, dv


@pytest.mark.parametrize("dtype", [fi.F16, fi.BF16])
@pytest.mark.parametrize("causal,off", [(False, 0), (True, 0), (True, 5)])
def test_emulated_kernel_rounding_within_bounds(dtype, causal, off):
    cfg = fi.Config("bounds", 1, 4, 70, 75, 64, dtype, False, seed=31)
    inp = fi.make_inputs(cfg)
    inp.k = inp.k[:, :2].contiguous()
    inp.v = inp.v[:, :2].contiguous()
    q, k, v = fi.values(inp)
    g = fi.make_cotangent((1, 4, 70, 64), dtype, 32).double().numpy()
    o, lse = attention_fp64(q, k, v, cfg.scale, causal, off)
    ou, lu = as_used(o, dtype), as_used(lse, fi.F32)
    ref = attention_bwd_fp64(q, k, v, g, cfg.scale, causal, off)
    got = _emulate(q, k, v, g, cfg.scale, causal, off, ou, lu, dtype)
    bnd = grad_bounds(q, k, v, g, cfg.scale, causal, off, o_used=ou, lse_used=lu)
    errs = check_grads(dtype, got, ref, bnd, f"emulated {dtype}")
    # the emulation uses a sizeable part of the allowance somewhere
    assert max(errs) > 0.05


def test_single_wrong_element_is_caught():
    """An error of four times one element's own allowance fails, although it
    is below a hundredth of the largest gradient of its tensor (which a bound
    over the whole tensor would have let through)."""
    cfg = fi.Config("bounds", 1, 2, 64, 64, 64, fi.F16, False, seed=33)
    inp = fi.make_inputs(cfg)
    q, k, v = fi.values(inp)
    g = fi.make_cotangent((1, 2, 64, 64), fi.F16, 34).double().numpy()
    o, lse = attention_fp64(q, k, v, cfg.scale, True, 0)
    ou, lu = as_used(o, fi.F16), as_used(lse, fi.F32)
    ref = attention_bwd_fp64(q, k, v, g, cfg.scale, True, 0)
    bnd = grad_bounds(q, k, v, g, cfg.scale, True, 0, o_used=ou, lse_used=lu)
    check_grads(fi.F16, ref, ref, bnd, "exact")
    for t in range(3):
        got = [x.copy() for x in ref]
        tsum, e = bnd[t]
        lim = 2 * 2.0 ** -11 * tsum + 1.01 * e + 2.0 ** -24 * tsum.max()
        idx = np.unravel_index(np.argmin(np.where(tsum > 0, lim, np.inf)), lim.shape)
        delta = 4 * lim[idx]
        assert delta < 0.01 * np.abs(ref[t]).max()
        got[t][idx] += delta
        with pytest.raises(AssertionError):
            check_grads(fi.F16, got, ref, bnd, "planted")


def test_bounds_match_brute_force_term_sums():
    """T of dV is sum_i P_ij |dO_id|, of dQ scale * sum_j P_ij (|dP_ij| +
    |Delta_i|) |K_jd|: recomputed here with explicit loops on a tiny case."""
    rng = np.random.default_rng(35)
    q, k, v, g = (rng.standard_normal((1, 1, 5, 3)) for _ in range(4))
    scale = 0.7
    bnd = grad_bounds(q, k, v, g, scale, True, 0)
    _, _, p = head_forward(q[0, 0], k[0, 0], v[0, 0], scale, True, return_p=True)
    dp = g[0, 0] @ v[0, 0].T
    delta = (p * dp).sum(1)
    for i in range(5):
        for d in range(3):
            tq = sum(scale * p[i, j] * (abs(dp[i, j]) + abs(delta[i])) * abs(k[0, 0, j, d])
                     for j in range(5))
            assert abs(bnd[0][0][0, 0, i, d] - tq) < 1e-12
    for j in range(5):
        for d in range(3):
            tv = sum(p[i, j] * abs(g[0, 0, i, d]) for i in range(5))
            assert abs(bnd[2][0][0, 0, j, d] - tv) < 1e-12
