"""Helpers for the GPU parity tests: host<->device copies of the seeded
inputs, guarded output buffers, and the comparison rules.

Comparison rules (fp32 sums bit-exact; fp32 fused output within 1e-5
relative; fp16/bf16 within 2 units in the last place, the distance between
order-preserving integer encodings, with +0 == -0 and NaN == NaN).
"""
from __future__ import annotations

import sys

import numpy as np
import torch

TORCH_DT = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}
NP_DT = {"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}
GUARD_BYTES = 64 << 10  # canary bytes before and after each output


def note(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def dev(a: np.ndarray, dtype: str) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def slab(host_parts, dtype: str):
    """Device copies of the partials placed in one allocation from
    ar.allocate_workspace (the slots of ar_partials_layout); returns
    (allocation, views)."""
    from tensor_all_reduce_ar_amd import ar
    ws = ar.allocate_workspace(host_parts[0].size, TORCH_DT[dtype], len(host_parts))
    for v, h in zip(ws.partials, host_parts):
        v.copy_(dev(h, dtype))
    return ws.buffer, ws.partials


def host_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def bits(a: np.ndarray) -> np.ndarray:
    a = np.ascontiguousarray(a)
    return a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint16)


def empty_host(n: int, dtype: str) -> np.ndarray:
    return np.zeros(n, NP_DT[dtype])


class Guarded:
    """A device buffer of n elements with GUARD_BYTES of canary on each side,
    filled with a fixed pattern, to catch writes out of bounds."""
    PATTERN16, PATTERN32 = 0x5A3C, 0x5A3C7E11

    def __init__(self, n: int, dtype: str, offset_elems: int = 0):
        self.n, self.dtype, self.offset = n, dtype, offset_elems
        self.guard = GUARD_BYTES // (4 if dtype == "fp32" else 2)
        size = 2 * self.guard + n + offset_elems
        idt = torch.int32 if dtype == "fp32" else torch.int16
        pat = self.PATTERN32 if dtype == "fp32" else self.PATTERN16
        self.raw = torch.full((size,), pat, dtype=idt, device="cuda").view(TORCH_DT[dtype])
        self.t = self.raw[self.guard + offset_elems:self.guard + offset_elems + n]

    def check_guards(self):
        b = host_bits(self.raw)
        pat = self.PATTERN32 if self.dtype == "fp32" else self.PATTERN16
        lo = b[:self.guard + self.offset]
        hi = b[self.guard + self.offset + self.n:]
        assert np.all(lo == pat) and np.all(hi == pat), "write outside the output buffer"


def ordered(b: np.ndarray) -> np.ndarray:
    """Order-preserving integer image of 16-bit float encodings (+0 == -0)."""
    b = b.astype(np.int64)
    return np.where(b & 0x8000, 0x8000 - b, b)


def assert_bitexact(got_bits: np.ndarray, ref_bits: np.ndarray, dtype: str, what: str):
    if np.array_equal(got_bits, ref_bits):
        return
    nanmask = _nan(got_bits, dtype) & _nan(ref_bits, dtype)
    bad = (got_bits != ref_bits) & ~nanmask
    idx = np.flatnonzero(bad)
    assert idx.size == 0, f"{what}: {idx.size} elements differ, first at {idx[:5]}: got {got_bits[idx[:5]]} " \
                          f"want {ref_bits[idx[:5]]}"


def _nan(b: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return (b & 0x7F800000 == 0x7F800000) & (b & 0x007FFFFF != 0)
    if dtype == "fp16":
        return (b & 0x7C00 == 0x7C00) & (b & 0x03FF != 0)
    return (b & 0x7F80 == 0x7F80) & (b & 0x007F != 0)


def max_ulp(got_bits: np.ndarray, ref_bits: np.ndarray, dtype: str) -> int:
    nan_g, nan_r = _nan(got_bits, dtype), _nan(ref_bits, dtype)
    assert np.array_equal(nan_g, nan_r), "NaN positions differ"
    keep = ~nan_r
    if not keep.any():
        return 0
    return int(np.abs(ordered(got_bits[keep]) - ordered(ref_bits[keep])).max())


def assert_output_close(got_bits: np.ndarray, ref_bits: np.ndarray, dtype: str, what: str):
    if dtype == "fp32":
        g, r = got_bits.view(np.float32).astype(np.float64), ref_bits.view(np.float32).astype(np.float64)
        nan_r = np.isnan(r)
        assert np.array_equal(np.isnan(g), nan_r), f"{what}: NaN positions differ"
        g, r = g[~nan_r], r[~nan_r]
        inf = np.isinf(r)
        assert np.array_equal(g[inf], r[inf]), f"{what}: infinities differ"
        err = np.abs(g[~inf] - r[~inf])
        tol = 1e-5 * np.abs(r[~inf])
        bad = np.flatnonzero(err > tol)
        assert bad.size == 0, f"{what}: {bad.size} elements beyond 1e-5 relative, worst rel " \
                              f"{(err / np.maximum(np.abs(r[~inf]), 1e-300)).max():.3g}"
    else:
        u = max_ulp(got_bits, ref_bits, dtype)
        assert u <= 2, f"{what}: {u} ulp apart (limit 2)"
