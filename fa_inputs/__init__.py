"""Seeded synthetic inputs for the attention forward pass.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and stores them in the input dtypes;
it holds none of the attention arithmetic.

Workloads follow the shapes the pages use:
  * B1 H8 S512 D64 fp16 BNSD, scale 1/8: the minimal ``npu_flash_attention``
    call ("Tracing npu_flash_attention through the CANN runtime",
    ai6s.net/6a114bb2..., section "a minimal reproducible call").
  * B4 H32 S4096 D128 fp16: the runtime-decomposition example
    ("How the CANN runtime splits one FlashAttention call",
    ai6s.net/6a0eff03..., tile_level example).
  * B1 H32 S8192 D128: the long-sequence configuration
    ("ops-transformer FlashAttention on Ascend: build, run and tune",
    ai6s.net/6a31724f..., section 7, long-sequence config block).
  * S=4097 exercises a length one past a tile multiple (same runtime page,
    tiling remark on 4097 vs 4096).

Generator recipe: ``numpy.random.default_rng(seed)`` (PCG64), standard
normal draws in float64, shape (B, H, S, D) in C order, drawn in the order
q, k, v; an optional amplitude multiplies the draws in float64; the cast to
fp16 / bf16 goes through torch, which rounds float64 to float32 and then to
the target type, each step to nearest even. fp8 inputs are
quantised per tensor to OCP e4m3fn with ``s = amax|x| / 448`` and a clamp to
+-448 before the cast (torch's cast is not saturating).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

E4M3_MAX = 448.0

# dtype names used across the package, the tests and the benchmark
F16, BF16, FP8, F32 = "f16", "bf16", "fp8_e4m3", "f32"

TORCH_DTYPE = {
    F16: torch.float16,
    BF16: torch.bfloat16,
    FP8: torch.float8_e4m3fn,
    F32: torch.float32,
}


@dataclass(frozen=True)
class Config:
    """One attention workload: BNSD tensors [B, H, S, D]."""

    name: str
    B: int
    H: int
    Sq: int
    Sk: int
    D: int
    dtype: str
    causal: bool
    amp: float = 1.0
    o_dtype: str = F16
    seed: int = 0
    scale: float = field(default=0.0)

    def __post_init__(self):
        if self.scale == 0.0:
            object.__setattr__(self, "scale", 1.0 / math.sqrt(self.D))

    def flops(self) -> float:
        """4*B*H*Sq*Sk*D, halved for causal: the convention of the metric."""
        f = 4.0 * self.B * self.H * self.Sq * self.Sk * self.D
        return f / 2 if self.causal else f

    def replace(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        if "D" in kw and "scale" not in kw:
            d["scale"] = 0.0
        return Config(**d)


# The five workloads. Seeds are 1000 + index (1-based).
CONFIGS = [
    Config("b1h8s512d64_f16", 1, 8, 512, 512, 64, F16, False, seed=1001),
    Config("b2h16s2048d128_bf16_causal", 2, 16, 2048, 2048, 128, BF16, True,
           o_dtype=BF16, seed=1002),
    Config("b4h32s4096d128_f16", 4, 32, 4096, 4096, 128, F16, False, seed=1003),
    Config("b3h12s4097d64_f16x3_causal", 3, 12, 4097, 4097, 64, F16, True,
           amp=3.0, seed=1004),
    Config("b1h32s8192d128_fp8_causal", 1, 32, 8192, 8192, 128, FP8, True,
           seed=1005),
]
HEADLINE = CONFIGS[2]


@dataclass
class Inputs:
    """Device-independent input tensors (CPU torch tensors in the input dtype).

    For fp8, ``q``/``k``/``v`` hold e4m3fn codes and ``descale_*`` the
    per-tensor fp32 factors: the value of an element is code * descale.
    """

    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    descale_q: float = 1.0
    descale_k: float = 1.0
    descale_v: float = 1.0


def quantize_e4m3(x: np.ndarray) -> tuple[torch.Tensor, float]:
    """Per-tensor e4m3fn quantisation: codes and the fp32 descale s."""
    amax = float(np.max(np.abs(x)))
    s = np.float32(amax / E4M3_MAX) if amax > 0 else np.float32(1.0)
    y = np.clip(x / np.float64(s), -E4M3_MAX, E4M3_MAX)
    codes = torch.from_numpy(y).to(torch.float32).to(torch.float8_e4m3fn)
    return codes, float(s)


def draw(cfg: Config, seed: int | None = None) -> tuple[np.ndarray, ...]:
    """float64 draws for q, k, v in that order."""
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    q = rng.standard_normal((cfg.B, cfg.H, cfg.Sq, cfg.D))
    k = rng.standard_normal((cfg.B, cfg.H, cfg.Sk, cfg.D))
    v = rng.standard_normal((cfg.B, cfg.H, cfg.Sk, cfg.D))
    if cfg.amp != 1.0:
        q *= cfg.amp
        k *= cfg.amp
        v *= cfg.amp
    return q, k, v


def make_inputs(cfg: Config, seed: int | None = None) -> Inputs:
    """Seeded inputs in the configuration's dtype (CPU tensors)."""
    q, k, v = draw(cfg, seed)
    if cfg.dtype == FP8:
        cq, sq = quantize_e4m3(q)
        ck, sk = quantize_e4m3(k)
        cv, sv = quantize_e4m3(v)
        return Inputs(cq, ck, cv, sq, sk, sv)
    td = TORCH_DTYPE[cfg.dtype]
    return Inputs(*(torch.from_numpy(x).to(torch.float32).to(td) for x in (q, k, v)))


def as_float64(x: torch.Tensor, descale: float = 1.0) -> np.ndarray:
    """Exact float64 value of an input tensor (fp8: code * descale)."""
    y = x.to(torch.float64).numpy()
    if x.dtype == torch.float8_e4m3fn:
        y = y * np.float64(np.float32(descale))
    return y


def values(inp: Inputs) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """float64 q, k, v values as the kernel sees them."""
    return (as_float64(inp.q, inp.descale_q), as_float64(inp.k, inp.descale_k),
            as_float64(inp.v, inp.descale_v))


@dataclass
class VarlenInputs:
    """A packed batch of sequences of different lengths (CPU tensors):
    q [Tq,H,D], k/v [Tk,H_kv,D]; ``cu_q``/``cu_k`` int32 [B+1] offsets."""

    inp: Inputs
    cu_q: torch.Tensor
    cu_k: torch.Tensor
    max_q: int


def make_varlen_inputs(lens_q, lens_k, H: int, Hkv: int, D: int, dtype: str, seed: int,
                       amp: float = 1.0) -> VarlenInputs:
    """Seeded packed inputs: standard normal float64 draws of shapes
    (Tq,H,D), (Tk,Hkv,D), (Tk,Hkv,D) in the order q, k, v (times ``amp``),
    cast or quantised per tensor as ``make_inputs`` does."""
    if len(lens_q) != len(lens_k) or not lens_q:
        raise ValueError("one query and one key length per sequence")
    tq, tk = int(sum(lens_q)), int(sum(lens_k))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((tq, H, D)) * amp
    k = rng.standard_normal((tk, Hkv, D)) * amp
    v = rng.standard_normal((tk, Hkv, D)) * amp
    if dtype == FP8:
        (cq, sq), (ck, sk), (cv, sv) = quantize_e4m3(q), quantize_e4m3(k), quantize_e4m3(v)
        inp = Inputs(cq, ck, cv, sq, sk, sv)
    else:
        td = TORCH_DTYPE[dtype]
        inp = Inputs(*(torch.from_numpy(x).to(torch.float32).to(td) for x in (q, k, v)))
    cu_q = torch.tensor([0] + list(np.cumsum(lens_q)), dtype=torch.int32)
    cu_k = torch.tensor([0] + list(np.cumsum(lens_k)), dtype=torch.int32)
    return VarlenInputs(inp, cu_q, cu_k, int(max(lens_q)))


def make_cotangent(shape, dtype: str, seed: int) -> torch.Tensor:
    """Seeded gradient of the output for the backward pass: standard normal
    float64 draws of ``shape`` cast to ``dtype`` as ``make_inputs`` does
    (16-bit types only)."""
    x = np.random.default_rng(seed).standard_normal(shape)
    return torch.from_numpy(x).to(torch.float32).to(TORCH_DTYPE[dtype])
