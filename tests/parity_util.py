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


def term_bounds(q, k, v, g, scale, causal, off, drop=None):
    """Largest sum of absolute term values per gradient tensor (drop: keep,
    seed, offset of a dropout mask, whose Z / keep scales P in dV and dP)."""
    B, H, Sq, D = q.shape
    Hkv = k.shape[1]
    bq = 0.0
    bk = np.zeros(k.shape)
    bv = np.zeros(v.shape)
    for b in range(B):
        for h in range(H):
            kv = h // (H // Hkv)
            _, _, p = head_forward(q[b, h], k[b, kv], v[b, kv], scale, causal, return_p=True,
                                   offset=off)
            z = 1.0
            if drop is not None:
                z = dropout_keep_mask(b * H + h, range(Sq), k.shape[2], *drop) / drop[0]
            dp = (g[b, h] @ v[b, kv].T) * z
            w = p * (np.abs(dp) + np.abs(np.sum(p * dp, axis=1, keepdims=True)))
            bq = max(bq, float(np.max(abs(scale) * w @ np.abs(k[b, kv]))))
            bk[b, kv] += abs(scale) * w.T @ np.abs(q[b, h])
            bv[b, kv] += (p * z).T @ np.abs(g[b, h])
    return bq, float(bk.max()), float(bv.max())
