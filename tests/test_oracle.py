"""Pins for the CPU oracle: brute force, closed forms, invariants, a library
routine and the pages' overflow example. None of them re-types the oracle's
own vectorised formula.

Each pin is a function of an attention implementation ``fn(q, k, v, scale,
causal) -> (O, lse)`` so that the same pins can be run against planted
mistakes (``test_pins_catch_planted_mistakes``): every mutant below must fail
at least one pin.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention_bruteforce, attention_bwd_fp64, attention_dropout_fp64,
                    attention_fp64, attention_rows_fp64, attention_varlen_fp64,
                    dropout_keep_mask, dropout_threshold, head_forward)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_facts.json")


def rand(shape, seed, amp=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * amp


# ---------------------------------------------------------------- pins ----

def pin_bruteforce(fn):
    """Tiny shapes against pure-Python loops (math.exp / math.fsum)."""
    for (B, H, Sq, Sk, D, causal, seed) in [
        (1, 1, 1, 1, 1, False, 1), (2, 1, 3, 5, 2, False, 2), (1, 2, 5, 3, 4, True, 3),
        (2, 2, 7, 7, 3, True, 4), (1, 1, 2, 7, 4, True, 5), (1, 2, 7, 2, 2, False, 6),
    ]:
        q = rand((B, H, Sq, D), seed)
        k = rand((B, H, Sk, D), seed + 100)
        v = rand((B, H, Sk, D), seed + 200)
        scale = 0.7
        o, lse = fn(q, k, v, scale, causal)
        ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), scale, causal)
        assert np.max(np.abs(o - ob)) <= 1e-12
        assert np.max(np.abs(lse - lb)) <= 1e-12


def pin_constant_v(fn):
    """v_j = c for all j  =>  O_i = c for every mask."""
    q = rand((1, 2, 9, 8), 11)
    k = rand((1, 2, 9, 8), 12)
    c = rand((8,), 13)
    v = np.broadcast_to(c, (1, 2, 9, 8)).copy()
    for causal in (False, True):
        o, _ = fn(q, k, v, 0.35, causal)
        assert np.max(np.abs(o - c)) <= 1e-13


def pin_zero_q(fn):
    """Q = 0: non-causal O_i = mean_j v_j, lse = ln Sk; causal prefix means, lse = ln(i+1)."""
    Sq, Sk, D = 6, 6, 4
    q = np.zeros((1, 1, Sq, D))
    k = rand((1, 1, Sk, D), 21)
    v = rand((1, 1, Sk, D), 22)
    o, lse = fn(q, k, v, 1.3, False)
    assert np.allclose(o[0, 0], v[0, 0].mean(axis=0)[None, :], atol=1e-14, rtol=0)
    assert np.allclose(lse[0, 0], math.log(Sk), atol=1e-14, rtol=0)
    o, lse = fn(q, k, v, 1.3, True)
    for i in range(Sq):
        assert np.allclose(o[0, 0, i], v[0, 0, : i + 1].mean(axis=0), atol=1e-14, rtol=0)
        assert abs(lse[0, 0, i] - math.log(i + 1)) <= 1e-14


def pin_causal_row0(fn):
    """Causal row 0 sees only key 0: O_0 = v_0, lse_0 = scale * q_0 . k_0."""
    q = rand((2, 1, 5, 6), 31)
    k = rand((2, 1, 5, 6), 32)
    v = rand((2, 1, 5, 6), 33)
    o, lse = fn(q, k, v, 0.9, True)
    for b in range(2):
        assert np.max(np.abs(o[b, 0, 0] - v[b, 0, 0])) <= 1e-14
        dot = math.fsum(q[b, 0, 0, d] * k[b, 0, 0, d] for d in range(6))
        assert abs(lse[b, 0, 0] - 0.9 * dot) <= 1e-13


def pin_single_key(fn):
    """Sk = 1: O = v_0 for every row; lse = scale * q . k_0."""
    q = rand((1, 1, 4, 5), 41)
    k = rand((1, 1, 1, 5), 42)
    v = rand((1, 1, 1, 5), 43)
    o, lse = fn(q, k, v, 0.5, False)
    assert np.max(np.abs(o[0, 0] - v[0, 0, 0])) <= 1e-14
    for i in range(4):
        dot = math.fsum(q[0, 0, i, d] * k[0, 0, 0, d] for d in range(5))
        assert abs(lse[0, 0, i] - 0.5 * dot) <= 1e-13


def pin_two_keys(fn):
    """Two keys: O = sigma(s0-s1) v0 + sigma(s1-s0) v1, lse = ln(e^s0 + e^s1)."""
    q = rand((1, 1, 3, 4), 51)
    k = rand((1, 1, 2, 4), 52)
    v = rand((1, 1, 2, 4), 53)
    scale = 0.8
    o, lse = fn(q, k, v, scale, False)
    for i in range(3):
        s = [scale * math.fsum(q[0, 0, i, d] * k[0, 0, j, d] for d in range(4)) for j in range(2)]
        w0 = 1.0 / (1.0 + math.exp(s[1] - s[0]))
        w1 = 1.0 / (1.0 + math.exp(s[0] - s[1]))
        want = w0 * v[0, 0, 0] + w1 * v[0, 0, 1]
        assert np.max(np.abs(o[0, 0, i] - want)) <= 1e-14
        hi = max(s)
        assert abs(lse[0, 0, i] - (hi + math.log1p(math.exp(min(s) - hi)))) <= 1e-14


def pin_linear_in_v(fn):
    """O is linear in V (P does not depend on V)."""
    q = rand((1, 2, 7, 4), 61)
    k = rand((1, 2, 9, 4), 62)
    v1 = rand((1, 2, 9, 4), 63)
    v2 = rand((1, 2, 9, 4), 64)
    for causal in (False, True):
        a, _ = fn(q, k, v1, 0.6, causal)
        b, _ = fn(q, k, v2, 0.6, causal)
        c, _ = fn(q, k, v1 - 2.5 * v2, 0.6, causal)
        assert np.max(np.abs(c - (a - 2.5 * b))) <= 1e-12


def pin_key_permutation(fn):
    """Non-causal: permuting the rows of K and V together changes nothing."""
    q = rand((1, 1, 5, 4), 71)
    k = rand((1, 1, 8, 4), 72)
    v = rand((1, 1, 8, 4), 73)
    perm = np.random.default_rng(74).permutation(8)
    a, la = fn(q, k, v, 0.9, False)
    b, lb = fn(q, k[:, :, perm], v[:, :, perm], 0.9, False)
    assert np.max(np.abs(a - b)) <= 1e-13 and np.max(np.abs(la - lb)) <= 1e-13


def pin_library_sdpa(fn):
    """torch's scaled_dot_product_attention (math path, fp64, CPU), top-left causal;
    lse from torch.logsumexp over the masked, scaled scores."""
    for (Sq, Sk, causal, seed) in [(33, 33, False, 81), (40, 40, True, 82), (17, 29, True, 83),
                                   (29, 17, True, 84), (20, 50, False, 85)]:
        q = rand((2, 3, Sq, 16), seed)
        k = rand((2, 3, Sk, 16), seed + 1)
        v = rand((2, 3, Sk, 16), seed + 2)
        scale = 0.25
        o, lse = fn(q, k, v, scale, causal)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        ref = torch.nn.functional.scaled_dot_product_attention(
            tq, tk, tv, is_causal=causal, scale=scale).numpy()
        assert np.max(np.abs(o - ref)) <= 1e-10
        s = torch.matmul(tq, tk.transpose(-1, -2).contiguous()) * scale
        if causal:
            s = s.masked_fill(torch.ones(Sq, Sk, dtype=torch.bool).triu(1), float("-inf"))
        assert np.max(np.abs(lse - torch.logsumexp(s, dim=-1).numpy())) <= 1e-10


def pin_large_logits(fn):
    """Logits far past the fp16 exp-overflow point stay finite (safe softmax).

    The pages put that point at a scaled logit of ln(65504) ~ 11.09, a raw
    logit of ~88.7 at head_dim 64. Here one key leads by ~1000: O = v_lead,
    lse = the leading score.
    """
    facts = json.load(open(GOLDEN))["fp16_exp_overflow"]
    assert abs(math.log(facts["fp16_max"]) - facts["ln_fp16_max"]) < 5e-3
    assert abs(facts["ln_fp16_max"] * math.sqrt(facts["head_dim"]) - facts["raw_logit_threshold"]) < 0.05
    D = facts["head_dim"]
    scale = 1.0 / math.sqrt(D)
    q = np.zeros((1, 1, 2, D))
    k = np.zeros((1, 1, 3, D))
    q[0, 0, :, 0] = 100.0
    k[0, 0, 0, 0] = 80.0    # score 1000
    k[0, 0, 1, 0] = -20.0   # score -250
    k[0, 0, 2, 0] = 10.0    # score 125 (>> 11.09: would overflow a naive fp16 exp)
    v = rand((1, 1, 3, D), 91)
    o, lse = fn(q, k, v, scale, False)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert np.max(np.abs(o[0, 0] - v[0, 0, 0])) <= 1e-14
    assert np.max(np.abs(lse[0, 0] - 1000.0)) <= 1e-12


PINS = [pin_bruteforce, pin_constant_v, pin_zero_q, pin_causal_row0, pin_single_key,
        pin_two_keys, pin_linear_in_v, pin_key_permutation, pin_library_sdpa,
        pin_large_logits]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(attention_fp64)


def test_softmax_rows():
    """P >= 0, rows sum to 1, masked entries are exactly 0."""
    q = rand((7, 6), 101)
    k = rand((11, 6), 102)
    v = rand((11, 6), 103)
    for causal in (False, True):
        _, _, p = head_forward(q, k, v, 0.4, causal, return_p=True)
        assert np.all(p >= 0)
        assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-12
        if causal:
            assert np.all(p[np.triu_indices(7, 1, 11)] == 0.0)


def test_rows_match_full():
    q = rand((2, 2, 40, 8), 111)
    k = rand((2, 2, 40, 8), 112)
    v = rand((2, 2, 40, 8), 113)
    for causal in (False, True):
        o, lse = attention_fp64(q, k, v, 0.3, causal)
        rows = [0, 5, 17, 39]
        orow, lrow = attention_rows_fp64(q, k, v, 0.3, causal, 1, 0, rows)
        assert np.array_equal(orow, o[1, 0, rows]) and np.array_equal(lrow, lse[1, 0, rows])


# ------------------------------------------------- planted mistakes ------

def _mutant(kind):
    def fn(q, k, v, scale, causal):
        B, H, Sq, D = q.shape
        Sk = k.shape[2]
        o = np.empty((B, H, Sq, D))
        lse = np.empty((B, H, Sq))
        for b in range(B):
            for h in range(H):
                qq, kk, vv = q[b, h], k[b, h], v[b, h]
                s = qq @ kk.T * (1.0 if kind == "no_scale" else scale)
                if causal:
                    i = np.arange(Sq)[:, None]
                    j = np.arange(Sk)[None, :]
                    bad = {"mask_diag": j >= i, "mask_flip": j < i}.get(kind, j > i)
                    s = np.where(bad, -np.inf, s)
                m = s.max(axis=1, keepdims=True)
                if kind == "no_max":
                    m = np.zeros_like(m)
                with np.errstate(all="ignore"):
                    p = np.exp(s - m)
                    l = p.sum(axis=1, keepdims=True)
                    pn = p if kind == "no_norm" else p / l
                    if kind == "col_softmax":
                        pn = p / p.sum(axis=0, keepdims=True)
                    o[b, h] = pn @ (kk if kind == "uses_k" else vv)
                    if kind == "lse_no_m":
                        lse[b, h] = np.log(l[:, 0])
                    elif kind == "lse_log2":
                        lse[b, h] = m[:, 0] + np.log2(l[:, 0])
                    else:
                        lse[b, h] = m[:, 0] + np.log(l[:, 0])
        return o, lse
    return fn


MUTANTS = ["no_scale", "mask_diag", "mask_flip", "no_max", "no_norm", "col_softmax",
           "uses_k", "lse_no_m", "lse_log2"]


@pytest.mark.parametrize("kind", MUTANTS)
def test_pins_catch_planted_mistakes(kind):
    fn = _mutant(kind)
    failed = []
    for pin in PINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"


def test_pins_accept_correct_copy():
    """The mutant scaffold without a mistake passes every pin (so the pins
    fail mutants for the planted mistake, not for the scaffold)."""
    fn = _mutant("none")
    for pin in PINS:
        pin(fn)


def test_lse_merge_of_key_subsets():
    """Attention over a key set equals the logsumexp-weighted merge of
    attention over a partition of it: lse = ln sum_r exp(lse_r), O = sum_r
    exp(lse_r - lse) O_r. This is the softmax identity the split-KV path
    relies on; both sides here come from the oracle on different key sets
    (no merge code is shared with the GPU path)."""
    rng = np.random.default_rng(7)
    q = rng.standard_normal((1, 2, 5, 8))
    k = rng.standard_normal((1, 2, 11, 8))
    v = rng.standard_normal((1, 2, 11, 8))
    o_full, l_full = attention_fp64(q, k, v, 0.4, False)
    cuts = [0, 3, 4, 11]
    parts = [attention_fp64(q, k[:, :, a:b], v[:, :, a:b], 0.4, False)
             for a, b in zip(cuts[:-1], cuts[1:])]
    lse = np.log(sum(np.exp(l) for _, l in parts))
    o = sum(np.exp(l - lse)[..., None] * o_r for o_r, l in parts)
    assert np.max(np.abs(lse - l_full)) < 1e-12
    assert np.max(np.abs(o - o_full)) < 1e-12


# ------------- grouped key/value heads and a shifted causal diagonal -----
# fn(q, k, v, scale, causal, offset): k and v may have fewer heads than q
# (query head h uses key/value head h // (H / H_kv)); with causal, key j is
# visible to query i iff j <= i + offset; a row with no visible key gives
# O = 0 and lse = -inf.

def xpin_bruteforce(fn):
    """Tiny shapes with grouped heads and shifted diagonals against the
    pure-Python loops."""
    for (B, H, Hkv, Sq, Sk, D, causal, off, seed) in [
        (1, 4, 2, 3, 5, 2, True, 2, 1), (2, 4, 1, 5, 3, 3, True, -2, 2),
        (1, 6, 3, 4, 4, 2, False, 0, 3), (1, 2, 2, 6, 2, 2, True, -4, 4),
        (1, 3, 1, 2, 6, 3, True, 4, 5),
    ]:
        q = rand((B, H, Sq, D), seed)
        k = rand((B, Hkv, Sk, D), seed + 100)
        v = rand((B, Hkv, Sk, D), seed + 200)
        o, lse = fn(q, k, v, 0.6, causal, off)
        ob, lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.6, causal, off)
        assert np.max(np.abs(o - ob)) <= 1e-12
        fin = np.isfinite(lb)
        assert np.array_equal(np.isfinite(lse), fin)
        assert np.max(np.abs(lse[fin] - lb[fin])) <= 1e-12 and np.all(lse[~fin] == -np.inf)


def xpin_zero_q_bottom_right(fn):
    """Q = 0, bottom-right diagonal (offset = Sk - Sq): row i averages keys
    0 .. i + Sk - Sq, lse = ln(i + Sk - Sq + 1)."""
    Sq, Sk, D = 4, 7, 3
    q = np.zeros((1, 1, Sq, D))
    k = rand((1, 1, Sk, D), 121)
    v = rand((1, 1, Sk, D), 122)
    o, lse = fn(q, k, v, 0.9, True, Sk - Sq)
    for i in range(Sq):
        n = i + Sk - Sq + 1
        assert np.max(np.abs(o[0, 0, i] - v[0, 0, :n].mean(axis=0))) <= 1e-14
        assert abs(lse[0, 0, i] - math.log(n)) <= 1e-14


def xpin_rows_without_keys(fn):
    """Bottom-right with Sq > Sk: the first Sq - Sk rows see no key (O = 0,
    lse = -inf); row Sq - Sk sees key 0 only."""
    Sq, Sk, D = 6, 3, 4
    q = rand((1, 1, Sq, D), 131)
    k = rand((1, 1, Sk, D), 132)
    v = rand((1, 1, Sk, D), 133)
    o, lse = fn(q, k, v, 0.7, True, Sk - Sq)
    assert np.all(o[0, 0, : Sq - Sk] == 0.0) and np.all(lse[0, 0, : Sq - Sk] == -np.inf)
    r = Sq - Sk
    assert np.max(np.abs(o[0, 0, r] - v[0, 0, 0])) <= 1e-14
    dot = math.fsum(q[0, 0, r, d] * k[0, 0, 0, d] for d in range(D))
    assert abs(lse[0, 0, r] - 0.7 * dot) <= 1e-13


def xpin_grouped_equals_repeated(fn):
    """Grouped heads equal the same heads with each key/value head repeated
    for its query heads."""
    q = rand((2, 6, 5, 4), 141)
    k = rand((2, 2, 7, 4), 142)
    v = rand((2, 2, 7, 4), 143)
    for causal, off in ((False, 0), (True, 0), (True, 2)):
        a, la = fn(q, k, v, 0.5, causal, off)
        b, lb = fn(q, np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1), 0.5, causal, off)
        assert np.max(np.abs(a - b)) <= 1e-14 and np.max(np.abs(la - lb)) <= 1e-14


def xpin_library_sdpa(fn):
    """torch's scaled_dot_product_attention (fp64, CPU) with an explicit
    boolean mask for the shifted diagonal and grouped heads; rows without a
    visible key are left out (the library returns NaN there)."""
    for (H, Hkv, Sq, Sk, off, seed) in [(4, 2, 9, 13, 4, 151), (4, 1, 13, 9, -4, 152),
                                        (3, 3, 10, 10, 0, 153)]:
        q = rand((1, H, Sq, 8), seed)
        k = rand((1, Hkv, Sk, 8), seed + 1)
        v = rand((1, Hkv, Sk, 8), seed + 2)
        o, lse = fn(q, k, v, 0.3, True, off)
        keep = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + off
        tq = torch.from_numpy(q)
        tk = torch.from_numpy(np.repeat(k, H // Hkv, axis=1))
        tv = torch.from_numpy(np.repeat(v, H // Hkv, axis=1))
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=keep,
                                                               scale=0.3).numpy()
        rows = keep.any(dim=1).numpy()
        assert np.max(np.abs(o[:, :, rows] - ref[:, :, rows])) <= 1e-10


XPINS = [xpin_bruteforce, xpin_zero_q_bottom_right, xpin_rows_without_keys,
         xpin_grouped_equals_repeated, xpin_library_sdpa]


def _oracle_x(q, k, v, scale, causal, offset):
    return attention_fp64(q, k, v, scale, causal, offset)


@pytest.mark.parametrize("pin", XPINS, ids=lambda p: p.__name__)
def test_oracle_grouped_shifted_pin(pin):
    pin(_oracle_x)


def _xmutant(kind):
    """Independent scaffold for the grouped/shifted pins, with one planted
    mistake per kind ("none": correct)."""
    def fn(q, k, v, scale, causal, offset):
        B, H, Sq, D = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        o = np.zeros((B, H, Sq, D))
        lse = np.full((B, H, Sq), -np.inf)
        for b in range(B):
            for h in range(H):
                g = h % Hkv if kind == "kv_head_mod" else h // (H // Hkv)
                s = q[b, h] @ k[b, g].T * scale
                if causal:
                    i = np.arange(Sq)[:, None]
                    j = np.arange(Sk)[None, :]
                    shift = {"offset_flip": -offset, "offset_ignored": 0}.get(kind, offset)
                    s = np.where(j > i + shift, -np.inf, s)
                for r in range(Sq):
                    if np.all(np.isneginf(s[r])) and kind != "empty_rows_nan":
                        continue
                    with np.errstate(all="ignore"):
                        m = s[r].max()
                        p = np.exp(s[r] - m)
                        o[b, h, r] = p @ v[b, g] / p.sum()
                        lse[b, h, r] = m + np.log(p.sum())
        return o, lse
    return fn


XMUTANTS = ["kv_head_mod", "offset_flip", "offset_ignored", "empty_rows_nan"]


@pytest.mark.parametrize("kind", XMUTANTS)
def test_grouped_shifted_pins_catch_planted_mistakes(kind):
    fn = _xmutant(kind)
    failed = []
    for pin in XPINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"


def test_grouped_shifted_pins_accept_correct_copy():
    fn = _xmutant("none")
    for pin in XPINS:
        pin(fn)


# ------------------------------------------------ variable-length pins ----
# Packed sequences: q [Tq,H,D], k/v [Tk,H_kv,D], offsets cu_q, cu_k; each
# sequence is attended on its own, its diagonal placed inside it; lse [H,Tq].

# (query lengths, key lengths): a sequence without queries, one without
# keys, Sq > Sk and Sq < Sk, a single token
VCASES = [([3, 0, 5, 2, 1], [4, 2, 3, 0, 1]), ([1, 4], [6, 1]), ([5], [5]),
          ([2, 6, 3], [2, 2, 7])]


def _packed(lq, lk, H, Hkv, D, seed):
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int64)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int64)
    q = rand((int(cu_q[-1]), H, D), seed)
    k = rand((int(cu_k[-1]), Hkv, D), seed + 1)
    v = rand((int(cu_k[-1]), Hkv, D), seed + 2)
    return q, k, v, cu_q, cu_k


def vpin_bruteforce(fn):
    """Token by token against the pure-Python loops: query token t finds its
    sequence by scanning the offsets, and that sequence's keys are handed to
    the loops as a batch of one."""
    for c, (lq, lk) in enumerate(VCASES):
        for (H, Hkv, causal, br) in ((4, 2, True, True), (2, 1, True, False), (3, 3, False, False)):
            q, k, v, cu_q, cu_k = _packed(lq, lk, H, Hkv, 2, 170 + c)
            o, lse = fn(q, k, v, cu_q, cu_k, 0.8, causal, br)
            assert o.shape == q.shape and lse.shape == (H, q.shape[0])
            for t in range(q.shape[0]):
                b = 0
                while not (cu_q[b] <= t < cu_q[b + 1]):
                    b += 1
                i = t - cu_q[b]
                ks, ke = int(cu_k[b]), int(cu_k[b + 1])
                off = (ke - ks) - int(cu_q[b + 1] - cu_q[b]) if br else 0
                qq = [[[q[t, h].tolist()] for h in range(H)]]
                kk = [[k[ks:ke, g].tolist() for g in range(Hkv)]]
                vv = [[v[ks:ke, g].tolist() for g in range(Hkv)]]
                # row i of the sequence, seen as row 0 with the diagonal moved by i
                ob, lb = attention_bruteforce(qq, kk, vv, 0.8, causal, off + i)
                for h in range(H):
                    assert np.max(np.abs(o[t, h] - np.array(ob[0][h][0]))) <= 1e-12
                    if lb[0][h][0] == -math.inf:
                        assert lse[h, t] == -np.inf and np.all(o[t, h] == 0.0)
                    else:
                        assert abs(lse[h, t] - lb[0][h][0]) <= 1e-12


def vpin_block_diagonal_sdpa(fn):
    """The whole packed batch as one attention call of torch's
    scaled_dot_product_attention (fp64, CPU) with a block-diagonal boolean
    mask (and the per-sequence diagonal); rows without a visible key, where
    the library gives NaN, must be O = 0 and lse = -inf."""
    for c, (lq, lk) in enumerate(VCASES):
        for causal, br in ((False, False), (True, False), (True, True)):
            H, Hkv = 4, 2
            q, k, v, cu_q, cu_k = _packed(lq, lk, H, Hkv, 8, 180 + c)
            o, lse = fn(q, k, v, cu_q, cu_k, 0.4, causal, br)
            Tq, Tk = q.shape[0], k.shape[0]
            keep = torch.zeros(Tq, Tk, dtype=torch.bool)
            for b in range(len(lq)):
                qs, qe, ks, ke = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
                i = torch.arange(qe - qs)[:, None]
                j = torch.arange(ke - ks)[None, :]
                off = (ke - ks) - (qe - qs) if br else 0
                blk = (j <= i + off) if causal else torch.ones(qe - qs, ke - ks, dtype=torch.bool)
                keep[qs:qe, ks:ke] = blk
            tq = torch.from_numpy(q).permute(1, 0, 2)[None]
            tk = torch.from_numpy(np.repeat(k, H // Hkv, axis=1)).permute(1, 0, 2)[None]
            tv = torch.from_numpy(np.repeat(v, H // Hkv, axis=1)).permute(1, 0, 2)[None]
            ref = torch.nn.functional.scaled_dot_product_attention(
                tq, tk, tv, attn_mask=keep, scale=0.4)[0].permute(1, 0, 2).numpy()
            rows = keep.any(dim=1).numpy()
            assert o.shape == ref.shape
            assert np.max(np.abs(o[rows] - ref[rows]), initial=0.0) <= 1e-10
            assert np.all(o[~rows] == 0.0) and np.all(lse[:, ~rows] == -np.inf)
            assert np.all(np.isfinite(lse[:, rows]))


def vpin_sequence_order(fn):
    """Reordering the sequences of a batch reorders the results and changes
    nothing else."""
    lq, lk = [3, 1, 4, 2], [2, 5, 4, 3]
    q, k, v, cu_q, cu_k = _packed(lq, lk, 2, 1, 4, 190)
    o, lse = fn(q, k, v, cu_q, cu_k, 0.5, True, True)
    order = [2, 0, 3, 1]
    qi = np.concatenate([np.arange(cu_q[b], cu_q[b + 1]) for b in order])
    ki = np.concatenate([np.arange(cu_k[b], cu_k[b + 1]) for b in order])
    cq = np.concatenate([[0], np.cumsum([lq[b] for b in order])])
    ck = np.concatenate([[0], np.cumsum([lk[b] for b in order])])
    o2, l2 = fn(q[qi], k[ki], v[ki], cq, ck, 0.5, True, True)
    l1 = lse[:, qi]
    fin = np.isfinite(l1)
    assert np.array_equal(np.isfinite(l2), fin) and np.all(l2[~fin] == l1[~fin])
    assert np.max(np.abs(o2 - o[qi])) <= 1e-14 and np.max(np.abs(l2[fin] - l1[fin])) <= 1e-14


VPINS = [vpin_bruteforce, vpin_block_diagonal_sdpa, vpin_sequence_order]


@pytest.mark.parametrize("pin", VPINS, ids=lambda p: p.__name__)
def test_oracle_varlen_pin(pin):
    pin(attention_varlen_fp64)


def test_oracle_varlen_rejects_bad_offsets():
    q, k, v, cu_q, cu_k = _packed([2, 3], [3, 2], 2, 1, 4, 195)
    for bq, bk in ((cu_q[:-1], cu_k), (cu_q + 1, cu_k), (cu_q, cu_k[::-1].copy()),
                   (np.array([0, 4, 3, 5]), np.array([0, 1, 2, 5]))):
        with pytest.raises(ValueError):
            attention_varlen_fp64(q, k, v, bq, bk, 0.5, False)


def _vmutant(kind):
    """Independent scaffold for the variable-length pins, with one planted
    mistake per kind ("none": correct)."""
    def fn(q, k, v, cu_q, cu_k, scale, causal, br):
        Tq, H, D = q.shape
        Hkv = k.shape[1]
        o = np.zeros((Tq, H, D))
        lse = np.full((H, Tq), -np.inf)
        kcu = cu_q if kind == "keys_by_query_offsets" else cu_k
        for b in range(len(cu_q) - 1):
            qs, qe = int(cu_q[b]), int(cu_q[b + 1])
            ks, ke = int(kcu[b]), int(kcu[b + 1])
            ks = 0 if kind == "keys_from_start" else ks
            ke = min(ke, k.shape[0])
            if kind == "global_offset":
                off = (k.shape[0] - Tq) if br else 0
            else:
                off = (ke - ks) - (qe - qs) if br else 0
            for h in range(H):
                g = h // (H // Hkv)
                for i in range(qe - qs):
                    s = k[ks:ke, g] @ q[qs + i, h] * scale
                    if causal:
                        s = np.where(np.arange(ke - ks) > i + off, -np.inf, s)
                    if (s.size == 0 or np.all(np.isneginf(s))) and kind != "empty_rows_nan":
                        continue
                    with np.errstate(all="ignore"):
                        m = s.max() if s.size else -np.inf
                        p = np.exp(s - m)
                        o[qs + i, h] = p @ v[ks:ke, g] / p.sum()
                        lse[h, qs + i] = m + np.log(p.sum())
        if kind == "lse_token_major":
            return o, lse.T.copy()
        return o, lse
    return fn


VMUTANTS = ["keys_by_query_offsets", "keys_from_start", "global_offset", "empty_rows_nan",
            "lse_token_major"]


@pytest.mark.parametrize("kind", VMUTANTS)
def test_varlen_pins_catch_planted_mistakes(kind):
    fn = _vmutant(kind)
    failed = []
    for pin in VPINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"


def test_varlen_pins_accept_correct_copy():
    fn = _vmutant("none")
    for pin in VPINS:
        pin(fn)


def test_oracle_empty_key_set():
    """No key at all: every row is without a visible key."""
    q = rand((1, 2, 3, 4), 197)
    z = np.zeros((1, 1, 0, 4))
    for causal, off in ((False, 0), (True, 0), (True, 5)):
        o, lse = attention_fp64(q, z, z, 0.5, causal, off)
        assert np.all(o == 0.0) and np.all(lse == -np.inf)


# ------------------------------------------------------- backward pins ----
# fn(q, k, v, do, scale, causal, offset) -> (dq, dk, dv): the gradient of
# L = sum(O * dO) with respect to q, k, v.

def _loss_bruteforce(q, k, v, do, scale, causal, offset):
    o, _ = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), scale, causal, offset)
    return math.fsum(a * b for a, b in zip(np.asarray(o).ravel().tolist(), do.ravel().tolist()))


def bpin_finite_differences(fn):
    """Central differences of the pure-Python forward (loss sum(O * dO)),
    every element of q, k and v, grouped heads and shifted diagonals (one
    case with rows that see no key)."""
    h = 1e-5
    for (B, H, Hkv, Sq, Sk, D, causal, off, seed) in [
        (1, 2, 1, 3, 4, 2, True, 1, 61), (1, 2, 2, 4, 3, 3, False, 0, 62),
        (1, 4, 2, 4, 2, 2, True, -2, 63), (2, 1, 1, 2, 5, 2, True, 3, 64),
    ]:
        q = rand((B, H, Sq, D), seed)
        k = rand((B, Hkv, Sk, D), seed + 1)
        v = rand((B, Hkv, Sk, D), seed + 2)
        do = rand((B, H, Sq, D), seed + 3)
        dq, dk, dv = fn(q, k, v, do, 0.7, causal, off)
        for x, g in ((q, dq), (k, dk), (v, dv)):
            assert g.shape == x.shape
            for idx in np.ndindex(x.shape):
                keep = x[idx]
                x[idx] = keep + h
                lp = _loss_bruteforce(q, k, v, do, 0.7, causal, off)
                x[idx] = keep - h
                lm = _loss_bruteforce(q, k, v, do, 0.7, causal, off)
                x[idx] = keep
                assert abs((lp - lm) / (2 * h) - g[idx]) <= 1e-7, (idx, g[idx], (lp - lm) / (2 * h))


def bpin_torch_autograd(fn):
    """torch autograd (fp64, CPU) through scaled_dot_product_attention with an
    explicit boolean mask; grouped heads by repeating K and V (autograd sums
    the repeats)."""
    for (H, Hkv, Sq, Sk, causal, off, seed) in [(4, 2, 9, 13, True, 4, 71), (4, 1, 13, 9, True, 0, 72),
                                                (3, 3, 10, 10, False, 0, 73), (2, 1, 7, 20, True, 13, 74)]:
        q = rand((1, H, Sq, 8), seed)
        k = rand((1, Hkv, Sk, 8), seed + 1)
        v = rand((1, Hkv, Sk, 8), seed + 2)
        do = rand((1, H, Sq, 8), seed + 3)
        dq, dk, dv = fn(q, k, v, do, 0.3, causal, off)
        tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
        keep = (torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + off) if causal else None
        rk = tk.repeat_interleave(H // Hkv, dim=1)
        rv = tv.repeat_interleave(H // Hkv, dim=1)
        out = torch.nn.functional.scaled_dot_product_attention(tq, rk, rv, attn_mask=keep, scale=0.3)
        out.backward(torch.from_numpy(do))
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.max(np.abs(mine - ref.numpy())) <= 1e-10


def bpin_invariants(fn):
    """Softmax rows sum to 1: sum_j dV_j = sum_i dO_i and sum_j dK_j = 0;
    constant V rows: O does not depend on q or k (dQ = dK = 0); dO = 0: all
    gradients 0; rows without a visible key: dQ row = 0."""
    q = rand((1, 2, 6, 4), 81)
    k = rand((1, 2, 9, 4), 82)
    v = rand((1, 2, 9, 4), 83)
    do = rand((1, 2, 6, 4), 84)
    for causal, off in ((False, 0), (True, 0), (True, 3)):
        dq, dk, dv = fn(q, k, v, do, 0.5, causal, off)
        assert np.max(np.abs(dv.sum(axis=2) - do.sum(axis=2))) <= 1e-12
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12
    vc = np.broadcast_to(rand((1, 2, 1, 4), 85), v.shape).copy()
    dq, dk, dv = fn(q, k, vc, do, 0.5, True, 1)
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12
    dq, dk, dv = fn(q, k, v, np.zeros_like(do), 0.5, True, 0)
    assert not dq.any() and not dk.any() and not dv.any()
    dq, dk, dv = fn(q, k, v, do, 0.5, True, -2)     # rows 0, 1 see no key
    assert np.all(dq[:, :, :2] == 0.0) and np.all(np.isfinite(dq))


BPINS = [bpin_finite_differences, bpin_torch_autograd, bpin_invariants]


@pytest.mark.parametrize("pin", BPINS, ids=lambda p: p.__name__)
def test_oracle_backward_pin(pin):
    pin(attention_bwd_fp64)


def _bmutant(kind):
    """Independent scaffold for the backward pins, with one planted mistake
    per kind ("none": correct)."""
    def fn(q, k, v, do, scale, causal, offset):
        B, H, Sq, D = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        dq = np.zeros(q.shape)
        dk = np.zeros(k.shape)
        dv = np.zeros(v.shape)
        for b in range(B):
            for h in range(H):
                g = h // (H // Hkv)
                s = q[b, h] @ k[b, g].T * scale
                if causal and kind != "mask_dropped":
                    s = np.where(np.arange(Sk)[None, :] > np.arange(Sq)[:, None] + offset, -np.inf, s)
                p = np.zeros_like(s)
                for r in range(Sq):
                    if np.all(np.isneginf(s[r])):
                        continue
                    e = np.exp(s[r] - s[r].max())
                    p[r] = e if kind == "unnormalised_p" else e / e.sum()
                dp = do[b, h] @ v[b, g].T
                delta = 0.0 if kind == "no_delta" else np.sum(p * dp, axis=1, keepdims=True)
                ds = p * (dp - delta)
                dq[b, h] = (1.0 if kind == "dq_unscaled" else scale) * ds @ k[b, g]
                sign = -1.0 if kind == "dk_sign" else 1.0
                if kind == "group_overwrites":
                    dk[b, g] = sign * scale * ds.T @ q[b, h]
                    dv[b, g] = p.T @ do[b, h]
                else:
                    dk[b, g] += sign * scale * ds.T @ q[b, h]
                    dv[b, g] += p.T @ do[b, h]
        return dq, dk, dv
    return fn


BMUTANTS = ["mask_dropped", "unnormalised_p", "no_delta", "dq_unscaled", "dk_sign",
            "group_overwrites"]


@pytest.mark.parametrize("kind", BMUTANTS)
def test_backward_pins_catch_planted_mistakes(kind):
    fn = _bmutant(kind)
    failed = []
    for pin in BPINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"


def test_backward_pins_accept_correct_copy():
    fn = _bmutant("none")
    for pin in BPINS:
        pin(fn)


# -------------------------------------------------------- dropout pins ----
# fn(q, k, v, scale, causal, offset, keep, seed, rng_offset) -> (O, lse) and
# mfn(bh, rows, Sk, keep, seed, rng_offset) -> Z: the forward with dropout
# and its keep mask.

_M64 = (1 << 64) - 1


def philox4x64_10(ctr, key):
    """Philox4x64-10 written out from its published definition (Salmon et
    al., SC 2011): ten rounds of two 64x64->128-bit products with the round
    multipliers, the key bumped by the Weyl constants between rounds."""
    c = list(ctr)
    k0, k1 = key
    for r in range(10):
        if r:
            k0 = (k0 + 0x9E3779B97F4A7C15) & _M64
            k1 = (k1 + 0xBB67AE8584CAA73B) & _M64
        p0 = 0xD2E7470EE14C6C93 * c[0]
        p1 = 0xCA5A826395121157 * c[2]
        c = [(p1 >> 64) ^ c[1] ^ k0, p1 & _M64, (p0 >> 64) ^ c[3] ^ k1, p0 & _M64]
    return c


def dpin_bits_bruteforce(fn, mfn):
    """Every keep bit against the pure-Python Philox, element by element
    (query heads and rows 0 and large, keys across several tiles and a
    ragged tail)."""
    for (bh, rows, Sk, keep, seed, off) in [(0, [0, 1, 2], 70, 0.8, 0, 0),
                                            (5, [31, 4096], 40, 0.5, 123456789, 3),
                                            (77, [7], 97, 0.1, (1 << 64) - 1, (1 << 63) + 5)]:
        z = mfn(bh, rows, Sk, keep, seed, off)
        thr = min(max(int(round(keep * 65536)), 1), 65535)
        for r, i in enumerate(rows):
            for j in range(Sk):
                t, o32 = divmod(j, 32)
                u, m, e = (o32 >> 2) & 1, o32 >> 3, o32 & 3
                w = philox4x64_10((2 * t + u, i, bh, 0), (seed, off))
                n = 4 * m + e
                val = (w[n // 4] >> (16 * (n % 4))) & 0xffff
                assert z[r, j] == (1.0 if val < thr else 0.0), (bh, i, j)


def dpin_keep_fraction(fn, mfn):
    """The kept fraction over 2^18 draws is thr / 65536 within 5 sigma."""
    for keep in (0.9, 0.5, 0.13):
        z = mfn(3, range(64), 4096, keep, 99, 1)
        p = dropout_threshold(keep) / 65536.0
        sig = math.sqrt(p * (1 - p) / z.size)
        assert abs(z.mean() - p) <= 5 * sig, (keep, z.mean())


def dpin_unbiased(fn, mfn):
    """The mean of O over many seeds is the undropped O (pure-Python loops)
    within 5 standard errors."""
    q = rand((1, 1, 3, 2), 91)
    k = rand((1, 1, 5, 2), 92)
    v = rand((1, 1, 5, 2), 93)
    ref, _ = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(), 0.9, True, 1)
    ref = np.asarray(ref)
    outs = np.stack([fn(q, k, v, 0.9, True, 1, 0.6, s, 0)[0] for s in range(600)])
    se = outs.std(axis=0) / math.sqrt(len(outs))
    assert np.all(np.abs(outs.mean(axis=0) - ref) <= 5 * se + 1e-12)


def dpin_lse_undropped(fn, mfn):
    """lse is the logsumexp of all visible scaled scores (torch.logsumexp)."""
    q = rand((1, 2, 6, 4), 95)
    k = rand((1, 2, 9, 4), 96)
    v = rand((1, 2, 9, 4), 97)
    _, lse = fn(q, k, v, 0.7, True, 2, 0.3, 5, 0)
    s = torch.from_numpy(q) @ torch.from_numpy(k).transpose(-1, -2) * 0.7
    keep = torch.arange(9)[None, :] <= torch.arange(6)[:, None] + 2
    ref = torch.logsumexp(s.masked_fill(~keep, -math.inf), dim=-1).numpy()
    assert np.max(np.abs(lse - ref)) <= 1e-12


def dpin_streams_differ(fn, mfn):
    """Masks of other heads, rows, seeds and offsets are different draws."""
    base = mfn(4, [10], 256, 0.5, 1, 2)
    for other in (mfn(5, [10], 256, 0.5, 1, 2), mfn(4, [11], 256, 0.5, 1, 2),
                  mfn(4, [10], 256, 0.5, 2, 2), mfn(4, [10], 256, 0.5, 1, 3)):
        assert np.mean(other != base) > 0.3


def dpin_threshold_edge(fn, mfn):
    """A value equal to the threshold is dropped, one below it kept: the
    keep probability is chosen so that the threshold equals the value drawn
    for key 0 of row 0 (pure-Python Philox)."""
    for seed in (11, 12, 13):
        w = philox4x64_10((0, 0, 0, 0), (seed, 0))
        v0 = w[0] & 0xffff
        if not 2 <= v0 <= 65534:
            continue
        assert mfn(0, [0], 4, v0 / 65536.0, seed, 0)[0, 0] == 0.0
        assert mfn(0, [0], 4, (v0 + 1) / 65536.0, seed, 0)[0, 0] == 1.0


DPINS = [dpin_bits_bruteforce, dpin_keep_fraction, dpin_unbiased, dpin_lse_undropped,
         dpin_streams_differ, dpin_threshold_edge]


@pytest.mark.parametrize("pin", DPINS, ids=lambda p: p.__name__)
def test_oracle_dropout_pin(pin):
    pin(lambda q, k, v, sc, c, off, kp, seed, ro: attention_dropout_fp64(q, k, v, sc, c, off, kp,
                                                                         seed, ro),
        dropout_keep_mask)


def _dmutant(kind):
    """Independent scaffold (pure-Python Philox) with one planted mistake
    per kind ("none": correct)."""
    def mfn(bh, rows, Sk, keep, seed, off):
        thr = min(max(int(round(keep * 65536)), 1), 65535)
        z = np.zeros((len(rows), Sk))
        for r, i in enumerate(rows):
            cache = {}
            for j in range(Sk):
                t, o32 = divmod(j, 32)
                u, m, e = (o32 >> 2) & 1, o32 >> 3, o32 & 3
                ctr = (2 * t + u, i, 0 if kind == "head_ignored" else bh, 0)
                if ctr not in cache:
                    cache[ctr] = philox4x64_10(ctr, (seed, off))
                w = cache[ctr]
                n = 4 * m + e
                wi = 3 - n // 4 if kind == "word_order" else n // 4
                val = (w[wi] >> (16 * (n % 4))) & 0xffff
                kept = val <= thr if kind == "keep_le" else val < thr
                z[r, j] = 1.0 if kept else 0.0
        return z

    def fn(q, k, v, scale, causal, offset, keep, seed, ro):
        B, H, Sq, D = q.shape
        Sk = k.shape[2]
        o = np.zeros((B, H, Sq, D))
        lse = np.zeros((B, H, Sq))
        for b in range(B):
            for h in range(H):
                s = q[b, h] @ k[b, h].T * scale
                if causal:
                    s = np.where(np.arange(Sk)[None, :] > np.arange(Sq)[:, None] + offset, -np.inf, s)
                mx = s.max(axis=1, keepdims=True)
                p = np.exp(s - mx)
                p /= p.sum(axis=1, keepdims=True)
                z = mfn(b * H + h, range(Sq), Sk, keep, seed, ro)
                pd = p * z
                o[b, h] = (pd if kind == "no_rescale" else pd / keep) @ v[b, h]
                ex = np.exp(s - mx) * (z if kind == "lse_dropped" else 1.0)
                with np.errstate(divide="ignore"):
                    lse[b, h] = mx[:, 0] + np.log(ex.sum(axis=1))
        return o, lse
    return fn, mfn


DMUTANTS = ["head_ignored", "word_order", "keep_le", "no_rescale", "lse_dropped"]


@pytest.mark.parametrize("kind", DMUTANTS)
def test_dropout_pins_catch_planted_mistakes(kind):
    fn, mfn = _dmutant(kind)
    failed = []
    for pin in DPINS:
        try:
            with np.errstate(all="ignore"):
                pin(fn, mfn)
        except (AssertionError, ValueError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"no pin catches the planted mistake {kind!r}"


def test_dropout_pins_accept_correct_copy():
    fn, mfn = _dmutant("none")
    for pin in DPINS:
        pin(fn, mfn)


# ------------------------------------------------ backward with dropout ----

def test_oracle_backward_dropout_finite_differences():
    """With the mask fixed the dropped forward is differentiable: central
    differences of the oracle's own dropout forward (whose mask is pinned
    above), every element of q, k and v."""
    h = 1e-6
    for (H, Hkv, Sq, Sk, causal, off, keep, seed) in [(2, 1, 3, 40, True, 37, 0.6, 3),
                                                      (2, 2, 4, 5, False, 0, 0.5, 4)]:
        q = rand((1, H, Sq, 3), 500 + seed)
        k = rand((1, Hkv, Sk, 3), 501 + seed)
        v = rand((1, Hkv, Sk, 3), 502 + seed)
        do = rand((1, H, Sq, 3), 503 + seed)
        dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.8, causal, off, keep, seed, 9)

        def loss():
            o, _ = attention_dropout_fp64(q, k, v, 0.8, causal, off, keep, seed, 9)
            return float(np.sum(o * do))
        for x, g in ((q, dq), (k, dk), (v, dv)):
            for idx in np.ndindex(x.shape):
                keep_x = x[idx]
                x[idx] = keep_x + h
                lp = loss()
                x[idx] = keep_x - h
                lm = loss()
                x[idx] = keep_x
                assert abs((lp - lm) / (2 * h) - g[idx]) <= 1e-6, (idx, g[idx])


def test_oracle_backward_dropout_torch_autograd():
    """torch autograd (fp64) through softmax, the fixed mask and P V."""
    H, Hkv, Sq, Sk, off, keep = 4, 2, 9, 37, 28, 0.7
    q = rand((1, H, Sq, 8), 511)
    k = rand((1, Hkv, Sk, 8), 512)
    v = rand((1, Hkv, Sk, 8), 513)
    do = rand((1, H, Sq, 8), 514)
    dq, dk, dv = attention_bwd_fp64(q, k, v, do, 0.4, True, off, keep, 21, 2)
    z = np.stack([dropout_keep_mask(h, range(Sq), Sk, keep, 21, 2) for h in range(H)])[None]
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    s = tq @ tk.repeat_interleave(H // Hkv, dim=1).transpose(-1, -2) * 0.4
    vis = torch.arange(Sk)[None, :] <= torch.arange(Sq)[:, None] + off
    p = torch.softmax(s.masked_fill(~vis, -math.inf), dim=-1)
    o = (p * torch.from_numpy(z) / keep) @ tv.repeat_interleave(H // Hkv, dim=1)
    o.backward(torch.from_numpy(do))
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.max(np.abs(mine - ref.numpy())) <= 1e-10


def test_oracle_backward_keep_one_is_plain():
    q, k, v, do = (rand((1, 2, 5, 4), 520 + i) for i in range(4))
    a = attention_bwd_fp64(q, k, v, do, 0.5, True, 0)
    b = attention_bwd_fp64(q, k, v, do, 0.5, True, 0, 1.0, 7, 7)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_backward_dropout_pins_catch_planted_mistakes():
    """Mask dropped from dP, or from dV: the autograd comparison fails."""
    H, Sq, Sk, keep = 2, 6, 40, 0.6
    q, k, v, do = (rand((1, H, Sq if i in (0, 3) else Sk, 4), 530 + i) for i in range(4))
    z = np.stack([dropout_keep_mask(h, range(Sq), Sk, keep, 5, 0) for h in range(H)])[None] / keep
    tq, tk, tv = (torch.from_numpy(x.copy()).requires_grad_() for x in (q, k, v))
    p = torch.softmax(tq @ tk.transpose(-1, -2) * 0.5, dim=-1)
    ((p * torch.from_numpy(z)) @ tv).backward(torch.from_numpy(do))
    pn = p.detach().numpy()
    for kind in ("no_mask_on_dp", "no_mask_on_dv"):
        dp = do @ v.transpose(0, 1, 3, 2) * (1.0 if kind == "no_mask_on_dp" else z)
        ds = pn * (dp - np.sum(pn * dp, axis=-1, keepdims=True))
        dv = (pn * (1.0 if kind == "no_mask_on_dv" else z)).transpose(0, 1, 3, 2) @ do
        dq = 0.5 * ds @ k
        bad = [np.max(np.abs(a - b.numpy())) > 1e-8 for a, b in ((dq, tq.grad), (dv, tv.grad))]
        assert any(bad), kind
