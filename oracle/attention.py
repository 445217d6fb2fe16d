"""CPU oracle for the attention forward pass (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this module. The GPU library never calls it, and it shares no code
with the GPU library.

What it computes is the plain definition of scaled dot-product attention
that FlashAttention reaches exactly, up to rounding order:

  * scores  S = scale * Q K^T            ("ops-transformer FlashAttention on
    Ascend: build, run and tune", ai6s.net/6a31724f..., section 4.3, the
    PyTorch reference in the correctness check; the default scale there is
    head_dim ** -0.5 and it is applied before the mask);
  * causal mask: scores strictly above the diagonal (key j > query i,
    top-left aligned) are set to -inf (same section: the upper triangle with
    diagonal offset 1 is filled with -inf);
  * P = softmax(S) along the key axis, computed the safe way: subtract the
    row maximum before exponentiating (same page, section 6.2, the
    numerically stable softmax and its second, normalising pass);
  * O = P V;
  * lse = m + ln(sum_j exp(S_ij - m)), the natural-log logsumexp of each
    scaled, masked score row. The pages never define lse; this is the
    reading adopted for the per-row logsumexp output.

Everything is float64 from the exact input values. S and P are
materialised per (batch, head).

Parity status: every function here is pinned by tests that do not re-use
its formulas (brute-force loops, closed forms, invariants and a library
routine); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


def _check(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> None:
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("shape mismatch between q, k, v")


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 causal: bool, rows: np.ndarray | None = None,
                 return_p: bool = False):
    """One (batch, head): q [Sq, D], k/v [Sk, D] float64.

    ``rows`` restricts the computation to those query indices (their causal
    mask still uses the true row index). Returns (O [R, D], lse [R]) and, if
    asked, the probability matrix P [R, Sk].
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows, np.int64)
    s = (q[idx] @ k.T) * np.float64(scale)                       # S = scale*QK^T
    if causal:
        key = np.arange(k.shape[0])
        s = np.where(key[None, :] > idx[:, None], -np.inf, s)      # j > i -> -inf
    m = np.max(s, axis=1, keepdims=True)                           # row max
    p = np.exp(s - m)                                              # safe exp
    l = np.sum(p, axis=1, keepdims=True)                           # row sum
    p = p / l                                                      # softmax
    o = p @ v                                                      # O = P V
    lse = m[:, 0] + np.log(l[:, 0])                                # logsumexp
    if return_p:
        return o, lse, p
    return o, lse


def attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool):
    """Full forward over BNSD tensors: returns O [B,H,Sq,D], lse [B,H,Sq]."""
    _check(q, k, v)
    B, H, Sq, D = q.shape
    o = np.empty((B, H, Sq, D), np.float64)
    lse = np.empty((B, H, Sq), np.float64)
    for b in range(B):
        for h in range(H):
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h], v[b, h], scale, causal)
    return o, lse


def attention_rows_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                        causal: bool, b: int, h: int, rows):
    """Selected query rows of one (b, h) of a BNSD problem."""
    _check(q, k, v)
    return head_forward(q[b, h], k[b, h], v[b, h], scale, causal, rows=rows)


def attention_bruteforce(q, k, v, scale: float, causal: bool):
    """Pure-Python loops, for tiny shapes only: same definition, no numpy math.

    Uses math.exp / math.fsum element by element.
    """
    B, H, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Sk = len(k[0][0])
    o = [[[[0.0] * D for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                scores = []
                for j in range(Sk):
                    if causal and j > i:
                        scores.append(-math.inf)
                    else:
                        dot = math.fsum(float(q[b][h][i][d]) * float(k[b][h][j][d])
                                        for d in range(D))
                        scores.append(scale * dot)
                mx = max(scores)
                e = [math.exp(s - mx) if s != -math.inf else 0.0 for s in scores]
                tot = math.fsum(e)
                for d in range(D):
                    o[b][h][i][d] = math.fsum(e[j] / tot * float(v[b][h][j][d])
                                              for j in range(Sk))
                lse[b][h][i] = mx + math.log(tot)
    return np.array(o, np.float64), np.array(lse, np.float64)
