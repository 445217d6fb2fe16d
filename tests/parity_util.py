"""Shared helpers for the GPU parity tests: run the library, run the oracle,
compare. The oracle and the library see the same seeded inputs."""
from __future__ import annotations

import numpy as np
import torch

import fa_inputs as fi
from oracle import attention_fp64, attention_rows_fp64, dropout_keep_mask, head_forward

# Tolerances on max |delta| against the fp64 oracle: 2e-3 on O and 1e-3 on
# lse for fp16/bf16 inputs, 6e-2 on O for fp8 inputs (lse for fp8: 1e-3).
# They bound the kernel's arithmetic, i.e. O before the cast to its storage
# type (o_dtype = f32). A 16-bit O may in addition be off by one unit in the
# last place of its storage type.
TOL_O = {fi.F16: 2e-3, fi.BF16: 2e-3, fi.FP8: 6e-2}
TOL_LSE = 1e-3


def ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Spacing of the storage type at |x|."""
    mant = {fi.F16: 10, fi.BF16: 7, fi.F32: 23}[dtype]
    e = np.floor(np.log2(np.maximum(np.abs(x), 2.0 ** -14)))
    return 2.0 ** (e - mant)


def to_device(inp: fi.Inputs, dev="cuda"):
    q, k, v = (t.to(dev) for t in (inp.q, inp.k, inp.v))
    ds = None
    if inp.q.dtype == torch.float8_e4m3fn:
        ds = [torch.tensor([d], dtype=torch.float32, device=dev)
              for d in (inp.descale_q, inp.descale_k, inp.descale_v)]
    return q, k, v, ds


def run_gpu(cfg: fi.Config, inp: fi.Inputs, o_dtype: str, fwd=None):
    import attention_fa_fwd_07_amd as fa
    fwd = fwd or fa.fa_fwd
    q, k, v, ds = to_device(inp)
    kw = {}
    if ds is not None:
        kw = dict(descale_q=ds[0], descale_k=ds[1], descale_v=ds[2])
    o, lse = fwd(q, k, v, scale=cfg.scale, causal=cfg.causal,
                 o_dtype=fi.TORCH_DTYPE[o_dtype], **kw)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def oracle_full(cfg: fi.Config, inp: fi.Inputs):
    q, k, v = fi.values(inp)
    return attention_fp64(q, k, v, cfg.scale, cfg.causal)


def compare(cfg: fi.Config, o_dtype: str, o, lse, ref_o, ref_lse, what=""):
    """Assert parity; returns (max |dO|, max |dlse|)."""
    assert np.all(np.isfinite(o)), f"{what}: non-finite O"
    assert np.all(np.isfinite(lse)), f"{what}: non-finite lse"
    tol = TOL_O[cfg.dtype]
    err = np.abs(o - ref_o)
    if o_dtype == fi.F32:
        bound = tol
    else:
        bound = tol + ulp(ref_o, o_dtype)
    bad = err > bound
    assert not np.any(bad), (
        f"{what}: O mismatch at {np.argwhere(bad)[:5].tolist()}, max err {err.max():.3e} "
        f"(tol {tol}, o_dtype {o_dtype})")
    dl = np.abs(lse - ref_lse)
    assert dl.max() <= TOL_LSE, f"{what}: lse max err {dl.max():.3e}"
    return float(err.max()), float(dl.max())


def sample_rows(S: int, rng: np.random.Generator, n: int = 24):
    """Rows to check in a long sequence: the ends, tile edges and random ones."""
    fixed = {0, 1, 31, 32, 63, 64, 127, 128, 129, S // 2, S - 129, S - 128, S - 65, S - 64,
             S - 33, S - 2, S - 1}
    fixed = {r for r in fixed if 0 <= r < S}
    extra = rng.choice(S, size=min(n, S), replace=False)
    return np.array(sorted(fixed | set(int(x) for x in extra)))


def oracle_rows(cfg: fi.Config, inp: fi.Inputs, b: int, h: int, rows):
    q = fi.as_float64(inp.q[b:b + 1, h:h + 1], inp.descale_q)
    k = fi.as_float64(inp.k[b:b + 1, h:h + 1], inp.descale_k)
    v = fi.as_float64(inp.v[b:b + 1, h:h + 1], inp.descale_v)
    return attention_rows_fp64(q, k, v, cfg.scale, cfg.causal, 0, 0, rows)


def grad_bounds(q, k, v, g, scale, causal, off, drop=None, o_used=None, lse_used=None):
    """Per-element error bounds of dQ, dK and dV, as (T, E) per tensor.

    T: the sum of the absolute values of the terms of each gradient element
    that the kernels round to the input type before a product: P in
    dV = P^T dO, dS = P (dP - Delta) in dQ = scale dS K and dK = scale dS^T Q
    (|dS| <= P (|dP| + |Delta|)); the comparison allows TOL * T.
    E: the exact propagation of what the kernels are given that differs from
    the oracle's own values: Delta = rowsum(dO * O) formed from the O they
    receive (o_used, e.g. the oracle's O rounded to the input type, or the
    library's forward output), and P recomputed from the lse they receive
    (lse_used). drop: (keep, seed, offset) of a dropout mask, whose Z / keep
    scales P in dV and dP. Inputs are float64 numpy arrays."""
    B, H, Sq, D = q.shape
    Hkv = k.shape[1]
    T = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    E = [np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)]
    sc = abs(scale)
    for b in range(B):
        for h in range(H):
            kv = h // (H // Hkv)
            _, lse_ex, p = head_forward(q[b, h], k[b, kv], v[b, kv], scale, causal, return_p=True,
                                        offset=off)
            z = 1.0
            if drop is not None:
                z = dropout_keep_mask(b * H + h, range(Sq), k.shape[2], *drop) / drop[0]
            pz = p * z
            o_ex = pz @ v[b, kv]
            dp = (g[b, h] @ v[b, kv].T) * z
            delta = np.sum(p * dp, axis=1, keepdims=True)
            aq, ak = np.abs(q[b, h]), np.abs(k[b, kv])
            w = p * (np.abs(dp) + np.abs(delta))
            T[0][b, h] = sc * w @ ak
            T[1][b, kv] += sc * w.T @ aq
            T[2][b, kv] += pz.T @ np.abs(g[b, h])
            if o_used is not None:
                dd = np.abs(np.sum(g[b, h] * (o_used[b, h] - o_ex), axis=1, keepdims=True))
                E[0][b, h] += sc * dd * (p @ ak)
                E[1][b, kv] += sc * p.T @ (dd * aq)
            if lse_used is not None:
                both_empty = np.isneginf(lse_ex) & np.isneginf(lse_used[b, h])
                with np.errstate(invalid="ignore"):
                    d = np.where(both_empty, 0.0, lse_ex - lse_used[b, h])
                eps = np.abs(np.expm1(d))[:, None]
                ds = np.abs(p * (dp - delta)) * eps
                E[0][b, h] += sc * ds @ ak
                E[1][b, kv] += sc * ds.T @ aq
                E[2][b, kv] += (pz * eps).T @ np.abs(g[b, h])
    return tuple(zip(T, E))


def check_grads(dtype, got, ref, bounds, what, grad_dtype=None):
    """Assert |g - g_ref| <= TOL * T + E (+ one unit in the last place of a
    16-bit gradient type) element by element; returns, per tensor, the
    largest fraction of its element's allowance an error uses."""
    tol = TOL_GRAD[dtype]
    out = []
    for name, gv, r, (t, e) in zip(("dq", "dk", "dv"), got, ref, bounds):
        assert np.all(np.isfinite(gv)), f"{what}: non-finite {name}"
        err = np.abs(gv - r)
        floor = 2.0 ** -24 * float(np.max(t, initial=0.0))
        lim = tol * t + 1.01 * e + floor
        if grad_dtype is not None and grad_dtype != fi.F32:
            lim = lim + ulp(r, grad_dtype)
        bad = err > lim
        assert not np.any(bad), (
            f"{what}: {name} exceeds its element bound at {np.argwhere(bad)[:4].tolist()}: "
            f"err {err[bad][:4].tolist()} bound {lim[bad][:4].tolist()}")
        out.append(float(np.max(err / lim, initial=0.0)))
    return out


# rounding-term tolerance of the backward: 2u (fp16 u = 2^-11, bf16 2^-8)
TOL_GRAD = {fi.F16: 2 * 2.0 ** -11, fi.BF16: 2 * 2.0 ** -8}


def as_used(x: np.ndarray, dtype: str) -> np.ndarray:
    """x as the kernels receive it: float64 -> float32 -> dtype, back to float64."""
    t = torch.from_numpy(np.ascontiguousarray(x)).to(torch.float32)
    if dtype != fi.F32:
        t = t.to(fi.TORCH_DTYPE[dtype])
    return t.double().numpy()
