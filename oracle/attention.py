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
    diagonal offset 1 is filled with -inf). The variant with the diagonal
    moved by ``offset`` (key j visible iff j <= i + offset; offset = Sk - Sq
    aligns it to the bottom-right corner) follows the same rule; a row with
    no visible key (only possible with a negative offset) is defined to give
    O = 0 and lse = -inf, since the softmax of an empty set is undefined;
  * grouped key/value heads: k and v may have H_kv heads with H_kv dividing
    the query head count H; query head h then attends to key/value head
    h // (H / H_kv) (H_kv = 1 shares one key/value head among all);
  * variable-length batches ("Hygon FlashAttention: fixed-defect review",
    chatdocs.ruinique.com/hygon/flash-attention-fixed-bugs, item 17, the
    varlen forward whose packed token offsets outgrow 32 bits): the pages
    name the packed form but do not define it. The reading adopted: the B
    sequences are stored one after another along the token axis, sequence
    b owning query rows cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] ..
    cu_k[b+1]-1, and each is an attention problem of its own (no query sees
    another sequence's keys), its causal diagonal placed inside the
    sequence. A sequence with no key has only rows without a visible key;
  * P = softmax(S) along the key axis, computed the safe way: subtract the
    row maximum before exponentiating (same page, section 6.2, the
    numerically stable softmax and its second, normalising pass);
  * O = P V;
  * lse = m + ln(sum_j exp(S_ij - m)), the natural-log logsumexp of each
    scaled, masked score row. The pages never define lse; this is the
    reading adopted for the per-row logsumexp output.

The backward (``attention_bwd_fp64``) is the gradient of that same
function: for a cotangent dO of O, with P the row-softmax above,
  dV = P^T dO,  dP = dO V^T,  dS = P * (dP - rowsum(P * dP)),
  dQ = scale * dS K,  dK = scale * dS^T Q
(the chain rule through O = P V, the softmax Jacobian diag(p) - p p^T and
S = scale * Q K^T; masked entries have P = 0 and pass no gradient). With
grouped heads, dK and dV of a key/value head sum over its query heads. The
pages mention the backward's dQ pass only for a stride defect ("Hygon
FlashAttention: fixed-defect review", item 13) and state none of its
formulas; these are the derivative of the forward definition.

Dropout (``attention_dropout_fp64``): the pages pass a keep probability
through the call ("Tracing npu_flash_attention through the CANN runtime",
layer 1: keep_prob) and never define it. The reading adopted is inverted
dropout on the normalised probabilities: O = (P * Z / keep_prob) V with Z a
0/1 mask, P the softmax over all visible keys (so lse is unchanged). Z comes
from the counter-based generator Philox4x64-10 (Salmon, Moraes, Dror and
Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC 2011), taken here
from numpy's implementation (numpy.random.Philox), keyed by (seed, offset):
for query head index bh = b*H + h, query row i, 32-key tile t and half
u in {0, 1}, the counter (2t + u, i, bh, 0) gives four 64-bit words w0..w3,
read as sixteen 16-bit values v_n = (w_{n/4} >> 16*(n%4)) & 0xffff; key
32t + 8m + 4u + e (m, e in 0..3) takes v_{4m+e} and is kept iff it is below
thr = round(keep_prob * 65536) (clamped to 1..65535).

Everything is float64 from the exact input values. S and P are
materialised per (batch, head).

Parity status: every function here is pinned by tests that do not re-use
its formulas (brute-force loops, closed forms, invariants and a library
routine); none is "parity unpinned".
"""
from __future__ import annotations

import math

import numpy as np


def _check(q: np.ndarray, k: np.ndarray, v: np.ndarray) -> int:
    """Validates BNSD shapes; returns the query heads per key/value head."""
    if q.ndim != 4 or k.ndim != 4 or v.ndim != 4:
        raise ValueError("q, k, v must be [B, H, S, D]")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[3] != k.shape[3]:
        raise ValueError("shape mismatch between q, k, v")
    if k.shape[1] < 1 or q.shape[1] % k.shape[1] != 0:
        raise ValueError("the key/value head count must divide the query head count")
    return q.shape[1] // k.shape[1]


def head_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                 causal: bool, rows: np.ndarray | None = None,
                 return_p: bool = False, offset: int = 0):
    """One (batch, head): q [Sq, D], k/v [Sk, D] float64.

    ``rows`` restricts the computation to those query indices (their causal
    mask still uses the true row index). With ``causal``, key j is visible to
    query i iff j <= i + offset. Returns (O [R, D], lse [R]) and, if asked,
    the probability matrix P [R, Sk]; a row without a visible key gives
    O = 0, lse = -inf and P = 0.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    idx = np.arange(q.shape[0]) if rows is None else np.asarray(rows, np.int64)
    if k.shape[0] == 0:                                            # no key at all: every
        o = np.zeros((len(idx), v.shape[1]))                       # row is without a
        lse = np.full(len(idx), -np.inf)                           # visible key
        return (o, lse, np.zeros((len(idx), 0))) if return_p else (o, lse)
    s = (q[idx] @ k.T) * np.float64(scale)                       # S = scale*QK^T
    if causal:
        key = np.arange(k.shape[0])
        s = np.where(key[None, :] > idx[:, None] + offset, -np.inf, s)   # j > i + offset -> -inf
    empty = np.all(np.isneginf(s), axis=1)                         # rows without a visible key
    s = np.where(empty[:, None], 0.0, s)                           # (their result is set below)
    m = np.max(s, axis=1, keepdims=True)                           # row max
    p = np.exp(s - m)                                              # safe exp
    l = np.sum(p, axis=1, keepdims=True)                           # row sum
    p = p / l                                                      # softmax
    p[empty] = 0.0
    o = p @ v                                                      # O = P V
    lse = m[:, 0] + np.log(l[:, 0])                                # logsumexp
    lse[empty] = -np.inf
    if return_p:
        return o, lse, p
    return o, lse


def attention_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   causal: bool, offset: int = 0):
    """Full forward over BNSD tensors: returns O [B,H,Sq,D], lse [B,H,Sq].
    k and v may have fewer heads than q (grouped heads, see above)."""
    group = _check(q, k, v)
    B, H, Sq, D = q.shape
    o = np.empty((B, H, Sq, D), np.float64)
    lse = np.empty((B, H, Sq), np.float64)
    for b in range(B):
        for h in range(H):
            kv = h // group
            o[b, h], lse[b, h] = head_forward(q[b, h], k[b, kv], v[b, kv], scale, causal,
                                              offset=offset)
    return o, lse


def attention_varlen_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, cu_q, cu_k,
                          scale: float, causal: bool, bottom_right: bool = False):
    """Packed variable-length batch (see above): q [Tq,H,D], k/v [Tk,H_kv,D],
    cu_q/cu_k the B+1 sequence offsets along the token axis. Sequence b is
    attended on its own; with ``causal`` its diagonal has offset 0 (top-left)
    or Sk_b - Sq_b (``bottom_right``). Returns O [Tq,H,D], lse [H,Tq]."""
    cu_q = [int(x) for x in cu_q]
    cu_k = [int(x) for x in cu_k]
    if len(cu_q) != len(cu_k) or len(cu_q) < 2:
        raise ValueError("cu_q and cu_k must hold the same number (B+1 >= 2) of offsets")
    if cu_q[0] != 0 or cu_k[0] != 0 or cu_q[-1] != q.shape[0] or cu_k[-1] != k.shape[0]:
        raise ValueError("offsets must run from 0 to the packed lengths")
    if any(b < a for a, b in zip(cu_q, cu_q[1:])) or any(b < a for a, b in zip(cu_k, cu_k[1:])):
        raise ValueError("offsets must be nondecreasing")
    Tq, H, D = q.shape
    o = np.zeros((Tq, H, D), np.float64)
    lse = np.full((H, Tq), -np.inf)
    for b in range(len(cu_q) - 1):
        qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if qe == qs:
            continue
        # one BNSD problem with batch 1: [1, heads, tokens, D]
        qb = q[qs:qe].transpose(1, 0, 2)[None]
        kb = k[ks:ke].transpose(1, 0, 2)[None]
        vb = v[ks:ke].transpose(1, 0, 2)[None]
        off = (ke - ks) - (qe - qs) if bottom_right else 0
        ob, lb = attention_fp64(qb, kb, vb, scale, causal, off)
        o[qs:qe] = ob[0].transpose(1, 0, 2)
        lse[:, qs:qe] = lb[0]
    return o, lse


def attention_bwd_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, do: np.ndarray,
                       scale: float, causal: bool, offset: int = 0, keep_prob: float = 1.0,
                       seed: int = 0, rng_offset: int = 0):
    """Gradients of the BNSD forward for the cotangent ``do`` [B,H,Sq,D]:
    returns dq [B,H,Sq,D], dk, dv [B,H_kv,Sk,D]. With keep_prob < 1, of the
    forward with dropout (attention_dropout_fp64, same mask): the mask Z is
    fixed, O = (P * Z / keep_prob) V, so dV = (P * Z / keep_prob)^T dO and
    the gradient reaching P is dP * Z / keep_prob, which then passes the
    softmax Jacobian as above."""
    group = _check(q, k, v)
    if do.shape != q.shape:
        raise ValueError("do must have q's shape")
    B, H, Sq, D = q.shape
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    Sk = k.shape[2]
    for b in range(B):
        for h in range(H):
            kv = h // group
            _, _, p = head_forward(q[b, h], k[b, kv], v[b, kv], scale, causal,
                                   return_p=True, offset=offset)
            zk = 1.0
            if keep_prob != 1.0:
                zk = dropout_keep_mask(b * H + h, range(Sq), Sk, keep_prob, seed,
                                       rng_offset) / keep_prob
            g = np.asarray(do[b, h], np.float64)
            dv[b, kv] += (p * zk).T @ g                                # dV = (P Z/keep)^T dO
            dp = (g @ np.asarray(v[b, kv], np.float64).T) * zk         # dP = dO V^T (Z/keep)
            ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))      # softmax Jacobian
            dq[b, h] = scale * (ds @ np.asarray(k[b, kv], np.float64))  # dQ = scale dS K
            dk[b, kv] += scale * (ds.T @ np.asarray(q[b, h], np.float64))   # dK = scale dS^T Q
    return dq, dk, dv


def dropout_threshold(keep_prob: float) -> int:
    """16-bit threshold of the keep test (a value below it is kept)."""
    if not (0.0 < keep_prob < 1.0):
        raise ValueError("keep_prob must lie in (0, 1)")
    return min(max(int(round(keep_prob * 65536.0)), 1), 65535)


def dropout_keep_mask(bh: int, rows, Sk: int, keep_prob: float, seed: int, rng_offset: int):
    """Z [len(rows), Sk] (0/1) for query head index bh, by the rule above."""
    thr = dropout_threshold(keep_prob)
    nblk = 2 * ((Sk + 31) // 32)                  # counters 2t + u of one row
    key = np.array([seed, rng_offset], dtype=np.uint64)
    z = np.zeros((len(rows), nblk * 16), np.float64)
    for r, i in enumerate(rows):
        # numpy's Philox adds one to the 256-bit counter before each block:
        # start one below (0, i, bh, 0) to get the blocks 0, 1, 2, ...
        c = (int(i) << 64) + (int(bh) << 128) - 1
        ctr = np.array([(c >> (64 * w)) & ((1 << 64) - 1) for w in range(4)], dtype=np.uint64)
        words = np.random.Philox(key=key, counter=ctr).random_raw(4 * nblk).astype(np.uint64)
        v = np.stack([(words >> np.uint64(16 * s)) & np.uint64(0xffff) for s in range(4)],
                     axis=1).reshape(nblk, 16)      # v[block, n]
        # block 2t + u, value n = 4m + e  ->  key 32t + 8m + 4u + e
        t, u = np.divmod(np.arange(nblk), 2)
        m, e = np.divmod(np.arange(16), 4)
        keys = 32 * t[:, None] + 8 * m[None, :] + 4 * u[:, None] + e[None, :]
        z[r, keys.ravel()] = (v.ravel() < thr).astype(np.float64)
    return z[:, :Sk]


def attention_dropout_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                           causal: bool, offset: int, keep_prob: float, seed: int,
                           rng_offset: int = 0, rows=None):
    """Forward with dropout over BNSD tensors (see above): O [B,H,R,D] and
    the (undropped) lse [B,H,R] for the query rows ``rows`` (all by default)."""
    group = _check(q, k, v)
    B, H, Sq, D = q.shape
    Sk = k.shape[2]
    rows = np.arange(Sq) if rows is None else np.asarray(rows, np.int64)
    o = np.empty((B, H, len(rows), D))
    lse = np.empty((B, H, len(rows)))
    for b in range(B):
        for h in range(H):
            kv = h // group
            _, l, p = head_forward(q[b, h], k[b, kv], v[b, kv], scale, causal, rows=rows,
                                   return_p=True, offset=offset)
            z = dropout_keep_mask(b * H + h, rows, Sk, keep_prob, seed, rng_offset)
            o[b, h] = (p * z / keep_prob) @ np.asarray(v[b, kv], np.float64)
            lse[b, h] = l
    return o, lse


def attention_rows_fp64(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                        causal: bool, b: int, h: int, rows, offset: int = 0):
    """Selected query rows of one (b, h) of a BNSD problem."""
    group = _check(q, k, v)
    return head_forward(q[b, h], k[b, h // group], v[b, h // group], scale, causal, rows=rows,
                        offset=offset)


def attention_bruteforce(q, k, v, scale: float, causal: bool, offset: int = 0):
    """Pure-Python loops, for tiny shapes only: same definition, no numpy math.

    Uses math.exp / math.fsum element by element.
    """
    B, H, Sq, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Sk = len(k[0][0])
    Hkv = len(k[0])
    o = [[[[0.0] * D for _ in range(Sq)] for _ in range(H)] for _ in range(B)]
    lse = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h * Hkv // H            # key/value head of query head h
            for i in range(Sq):
                scores = []
                for j in range(Sk):
                    if causal and j - i > offset:
                        scores.append(-math.inf)
                    else:
                        dot = math.fsum(float(q[b][h][i][d]) * float(k[b][g][j][d])
                                        for d in range(D))
                        scores.append(scale * dot)
                if all(s == -math.inf for s in scores):
                    lse[b][h][i] = -math.inf            # no visible key: O stays 0
                    continue
                mx = max(scores)
                e = [math.exp(s - mx) if s != -math.inf else 0.0 for s in scores]
                tot = math.fsum(e)
                for d in range(D):
                    o[b][h][i][d] = math.fsum(e[j] / tot * float(v[b][g][j][d])
                                              for j in range(Sk))
                lse[b][h][i] = mx + math.log(tot)
    return np.array(o, np.float64), np.array(lse, np.float64)
