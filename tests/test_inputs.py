"""Seeded input generators: determinism, dtypes, fp8 quantisation."""
import numpy as np
import torch

import fa_inputs as fi


def test_deterministic_and_seed_sensitive():
    cfg = fi.CONFIGS[0].replace(H=2, Sq=64, Sk=64)
    a = fi.make_inputs(cfg)
    b = fi.make_inputs(cfg)
    c = fi.make_inputs(cfg, seed=7)
    assert torch.equal(a.q, b.q) and torch.equal(a.k, b.k) and torch.equal(a.v, b.v)
    assert not torch.equal(a.q, c.q)


def test_shapes_and_dtypes():
    for cfg in fi.CONFIGS:
        small = cfg.replace(B=1, H=1, Sq=min(cfg.Sq, 130), Sk=min(cfg.Sk, 130))
        x = fi.make_inputs(small)
        assert tuple(x.q.shape) == (1, 1, small.Sq, cfg.D)
        assert tuple(x.k.shape) == (1, 1, small.Sk, cfg.D) == tuple(x.v.shape)
        assert x.q.dtype == fi.TORCH_DTYPE[cfg.dtype]


def test_cast_is_round_to_nearest_even():
    q, _, _ = fi.draw(fi.CONFIGS[0].replace(H=1, Sq=256, Sk=256))
    x = fi.make_inputs(fi.CONFIGS[0].replace(H=1, Sq=256, Sk=256))
    # the recipe: float64 -> float32 -> float16, each step round-to-nearest-even
    assert np.array_equal(x.q.numpy(), q.astype(np.float32).astype(np.float16))


def test_amplitude():
    cfg = fi.CONFIGS[3].replace(H=1, Sq=512, Sk=512)
    q, _, _ = fi.draw(cfg)
    assert 2.7 < q.std() < 3.3


def test_e4m3_quantiser_clamps_and_roundtrips():
    x = np.array([0.0, 1.0, -2.5, 1000.0, -1e6, 3.0e-3])
    codes, s = fi.quantize_e4m3(x)
    assert codes.dtype == torch.float8_e4m3fn
    vals = codes.double().numpy()
    assert np.all(np.isfinite(vals))
    assert np.max(np.abs(vals)) <= 448.0
    # amax maps to +-448
    assert vals[4] == -448.0
    back = fi.as_float64(codes, s)
    assert abs(back[4] - (-1e6)) <= 1e6 * 2 ** -3
    # small values: relative error of e4m3 (3 mantissa bits) is <= 2^-4
    y = np.random.default_rng(3).standard_normal(4096)
    c, s = fi.quantize_e4m3(y)
    r = fi.as_float64(c, s)
    big = np.abs(y) > 64 * s   # normal range of e4m3 is >= 2^-6 in code units
    assert np.all(np.abs(r[big] - y[big]) <= np.abs(y[big]) * 2 ** -4 + 1e-12)


def test_flop_convention():
    assert fi.HEADLINE.flops() == 4.0 * 4 * 32 * 4096 * 4096 * 128
    assert fi.CONFIGS[1].flops() == 4.0 * 2 * 16 * 2048 * 2048 * 128 / 2
