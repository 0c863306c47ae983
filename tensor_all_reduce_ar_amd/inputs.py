"""Seeded synthetic inputs for the all-reduce core.

This module only draws random numbers and rounds them to the element type; it
holds none of the all-reduce arithmetic. Both the GPU tests/benchmark and the
CPU oracle consume what it returns.

Workloads follow the shapes of the "All Reduce Plugin" page (the partials are
[tokens, hidden] activations of a row-parallel linear, one per tensor-parallel
rank) and the fields of "type.d2" AllReduceFusionParams (bias [hidden], residual
[tokens, hidden], RMSNorm weight [hidden], eps).

Distributions: ``normal(mean, var)`` takes the VARIANCE as its second number, so
partials of variance 1/R sum to a unit-variance activation, the scale of the
residual stream. Values are drawn in fp32 with numpy's PCG64 generator (the same
bits on every machine for a given numpy version) and rounded to the element
type with round-to-nearest-even (numpy for fp16, torch for bf16).

Arrays are numpy: fp32 as float32, fp16 as float16, bf16 as uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Tuple

import numpy as np

DTYPES = ("fp32", "fp16", "bf16")


def to_dtype(x32: np.ndarray, dtype: str) -> np.ndarray:
    """Round an fp32 array to the element type (nearest even)."""
    x32 = np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        with np.errstate(over="ignore"):
            return x32.astype(np.float16)
    if dtype == "bf16":
        import torch
        return torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    raise ValueError(dtype)


def normal(shape, seed: int, mean: float, var: float, dtype: str) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.standard_normal(size=shape, dtype=np.float32)
    x *= np.float32(math.sqrt(var))
    x += np.float32(mean)
    return to_dtype(x, dtype)


def uniform(shape, seed: int, lo: float, hi: float, dtype: str) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    x = rng.random(size=shape, dtype=np.float32)
    x *= np.float32(hi - lo)
    x += np.float32(lo)
    return to_dtype(x, dtype)


@dataclasses.dataclass
class Workload:
    """One call's inputs. ``op`` is "sum" (fusion op NONE) or "fused"
    (fusion op RESIDUAL_RMS_NORM)."""
    name: str
    op: str
    dtype: str
    ranks: int
    n: int
    hidden: int
    partials: List[np.ndarray]
    bias: Optional[np.ndarray] = None
    residual: Optional[np.ndarray] = None
    weight: Optional[np.ndarray] = None
    eps: float = 0.0
    seeds: Dict[str, int] = dataclasses.field(default_factory=dict)
    distribution: str = ""  # how the values were drawn, for reports

    @property
    def rows(self) -> int:
        return self.n // self.hidden

    @property
    def itemsize(self) -> int:
        return 4 if self.dtype == "fp32" else 2

    def algorithmic_bytes(self) -> int:
        """Bytes the op must move: each input read once, each output written
        once. Sum: R partials + 1 output. Fused: R partials, residual, S and
        the normed output over n elements, plus weight (and bias) over hidden."""
        s = self.itemsize
        if self.op == "sum":
            return (self.ranks + 1) * self.n * s
        per_elem = self.ranks + 2 + (1 if self.residual is not None else 0)
        per_col = 1 + (1 if self.bias is not None else 0)
        return per_elem * self.n * s + per_col * self.hidden * s


def _sum_workload(name, dtype, ranks, n, hidden, seed0, dist) -> Workload:
    parts = []
    for r in range(ranks):
        if dist == "uniform":
            parts.append(uniform((n,), seed0 + r, -1.0, 1.0, dtype))
        else:
            parts.append(normal((n,), seed0 + r, 0.0, 1.0 / ranks, dtype))
    drawn = "uniform[lo, hi]: partials U[-1, 1]" if dist == "uniform" else \
        f"normal(mean, variance): partials N(0, 1/{ranks})"
    return Workload(name, "sum", dtype, ranks, n, hidden, parts, seeds={"partials": seed0},
                    distribution=f"{drawn}, rounded to {dtype}")


def _fused_workload(name, dtype, ranks, rows, hidden, seed0, seed_b, seed_q, seed_w, eps) -> Workload:
    n = rows * hidden
    parts = [normal((n,), seed0 + r, 0.0, 1.0 / ranks, dtype) for r in range(ranks)]
    bias = normal((hidden,), seed_b, 0.0, 0.02, dtype) if seed_b is not None else None
    residual = normal((n,), seed_q, 0.0, 1.0, dtype)
    weight = normal((hidden,), seed_w, 1.0, 0.1, dtype)
    seeds = {"partials": seed0, "residual": seed_q, "weight": seed_w}
    if seed_b is not None:
        seeds["bias"] = seed_b
    drawn = f"partials N(0, 1/{ranks}), " + ("bias N(0, 0.02), " if seed_b is not None else "") + \
        "residual N(0, 1), weight N(1, 0.1)"
    return Workload(name, "fused", dtype, ranks, n, hidden, parts, bias, residual, weight, eps, seeds,
                    f"normal(mean, variance): {drawn}, rounded to {dtype}")


# The named workloads. Names say what each is: op, type, ranks, shape.
SUM_FP32_R2_4x256 = "sum-fp32-r2-4x256"
FUSED_FP16_R8_16x4096 = "fused-fp16-r8-16x4096-bias"
SUM_BF16_R4_8192x8192 = "sum-bf16-r4-8192x8192"
FUSED_BF16_R8_2048x8192 = "fused-bf16-r8-2048x8192"
SUM_FP16_R2_1000003 = "sum-fp16-r2-n1000003"
FUSED_FP16_R2_5120_TOKENS = (1, 7, 64, 4096)


def fused_fp16_r2_5120_name(tokens: int) -> str:
    return f"fused-fp16-r2-{tokens}x5120-bias"


def workload_names() -> List[str]:
    return [SUM_FP32_R2_4x256, FUSED_FP16_R8_16x4096, SUM_BF16_R4_8192x8192, FUSED_BF16_R8_2048x8192,
            SUM_FP16_R2_1000003] + [fused_fp16_r2_5120_name(t) for t in FUSED_FP16_R2_5120_TOKENS]


def make(name: str) -> Workload:
    """Build a named workload on the host."""
    if name == SUM_FP32_R2_4x256:
        return _sum_workload(name, "fp32", 2, 4 * 256, 256, 1001, "uniform")
    if name == FUSED_FP16_R8_16x4096:
        return _fused_workload(name, "fp16", 8, 16, 4096, 2001, 2100, 2101, 2102, 1e-6)
    if name == SUM_BF16_R4_8192x8192:
        return _sum_workload(name, "bf16", 4, 8192 * 8192, 8192, 3001, "normal")
    if name == FUSED_BF16_R8_2048x8192:
        return _fused_workload(name, "bf16", 8, 2048, 8192, 4001, None, 4101, 4102, 1e-5)
    if name == SUM_FP16_R2_1000003:
        return _sum_workload(name, "fp16", 2, 1_000_003, 1_000_003, 5001, "normal")
    for t in FUSED_FP16_R2_5120_TOKENS:
        if name == fused_fp16_r2_5120_name(t):
            return _fused_workload(name, "fp16", 2, t, 5120, 5101, 5200, 5201, 5202, 1e-6)
    raise KeyError(name)


def random_sum(dtype: str, ranks: int, n: int, seed: int) -> Workload:
    """Sum inputs of any size (variance 1/R partials)."""
    return _sum_workload(f"sum-{dtype}-r{ranks}-n{n}", dtype, ranks, n, max(1, n), seed, "normal")


def random_fused(dtype: str, ranks: int, rows: int, hidden: int, seed: int, eps: float = 1e-6,
                 bias: bool = True, residual: bool = True) -> Workload:
    """Fused inputs of any shape; seeds seed+r for the partials, then
    seed+100 (bias), seed+101 (residual), seed+102 (weight)."""
    w = _fused_workload(f"fused-{dtype}-r{ranks}-{rows}x{hidden}", dtype, ranks, rows, hidden, seed,
                        seed + 100 if bias else None, seed + 101, seed + 102, eps)
    if not residual:
        w.residual = None
        w.distribution = w.distribution.replace("residual N(0, 1), ", "")
    return w


# ------------------------------------------------- counter-based values
# For arrays too large to draw on the host (indices past 2^31), element i of
# stream `seed` is a function of (seed, i) alone, so the device can fill the
# whole array and the host can recompute any sampled element. The hash is
# SplitMix64's finalizer (Steele, Lea & Flood, "Fast splittable pseudorandom
# number generators", OOPSLA 2014); its top 24 bits give a multiple of 2^-23
# in [-1, 1), exactly representable in fp32 and rounded once to the element
# type.
_M64 = (1 << 64) - 1


def _splitmix64(x):
    """SplitMix64 finalizer on uint64 numpy arrays (wrapping arithmetic)."""
    x = (x + np.uint64(0x9E3779B97F4A7C15))
    x = (x ^ (x >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    x = (x ^ (x >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return x ^ (x >> np.uint64(31))


def counter_values(seed: int, idx: np.ndarray, dtype: str) -> np.ndarray:
    """Values of stream `seed` at element indices `idx` (host, numpy)."""
    with np.errstate(over="ignore"):
        x = _splitmix64(np.asarray(idx, dtype=np.uint64) ^ np.uint64((seed * 0x632BE59BD9B4E019) & _M64))
    top = (x >> np.uint64(40)).astype(np.int64)  # 24 bits
    v = (top - (1 << 23)).astype(np.float32) * np.float32(2.0 ** -23)
    return to_dtype(v, dtype)


def counter_fill_device(seed: int, n: int, dtype: str, chunk: int = 1 << 26):
    """The same stream for indices 0..n-1, built on the current torch device
    chunk by chunk (torch int64 arithmetic wraps like uint64)."""
    import torch
    tdt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    out = torch.empty(n, dtype=tdt, device="cuda")
    key = (seed * 0x632BE59BD9B4E019) & _M64

    def s64(v):  # uint64 constant as a wrapped int64
        return v - (1 << 64) if v >= (1 << 63) else v

    def srl(t, k):  # logical right shift of int64 holding uint64 bits
        return (t >> k) & ((1 << (64 - k)) - 1)

    for start in range(0, n, chunk):
        m = min(chunk, n - start)
        x = torch.arange(start, start + m, dtype=torch.int64, device="cuda") ^ s64(key)
        x = x + s64(0x9E3779B97F4A7C15)
        x = (x ^ srl(x, 30)) * s64(0xBF58476D1CE4E5B9)
        x = (x ^ srl(x, 27)) * s64(0x94D049BB133111EB)
        x = x ^ srl(x, 31)
        top = srl(x, 40)
        v = (top - (1 << 23)).to(torch.float32) * (2.0 ** -23)
        out[start:start + m] = v.to(tdt)
    return out
