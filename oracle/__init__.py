"""CPU oracle for the all-reduce core (test infrastructure only).

This package is the plain, slow reference that the GPU library is checked
against: the C file ``ar_oracle.c`` beside this one, built with gcc and called
through ctypes. Only the tests, the smoke check and the benchmark's CPU-baseline
leg may import it. It shares no code with the GPU library and does not import
it; the GPU library never imports this package.

What it computes (sources: "All Reduce Plugin" page, class AllReducePlugin:
sum of tensor-parallel partials, passthrough for one rank; "type.d2" page,
classes AllReduceParams / AllReduceFusionParams and enum AllReduceFusionOp;
"allreduce.d2" page, the standalone and fused kernel branches):

* ``ar_sum``: out = round_T(sum over ranks in order, in fp32).
* ``ar_residual_rmsnorm``: S = round_T((sum + bias) + residual) in fp32, then
  out = round_T(S / sqrt(mean(S^2) + eps) * weight) in fp64.
* ``rmsnorm``: the norm step alone (the unfused branch's rms_norm_kernel).

Every function has pins in ``tests/test_oracle.py``; none is "parity unpinned".

Arrays are numpy arrays on the host. fp16 and bf16 data are passed as their
raw 16-bit patterns (``numpy.uint16``) or as float16 arrays; fp32 as float32.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ar_oracle.c")
_LIB = os.path.join(_HERE, "liboracle_ar.so")

FP32, FP16, BF16 = 0, 1, 2
_DTYPES = {"fp32": FP32, "fp16": FP16, "bf16": BF16}

GCC_FLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/liboracle_ar.so``."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        L = ctypes.CDLL(_LIB)
        vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
        L.oracle_ar_sum.argtypes = [i32, i32, ctypes.POINTER(vp), sz, vp]
        L.oracle_ar_sum.restype = i32
        L.oracle_rmsnorm.argtypes = [i32, sz, i32, vp, vp, ctypes.c_float, vp]
        L.oracle_rmsnorm.restype = i32
        L.oracle_ar_residual_rmsnorm.argtypes = [i32, i32, ctypes.POINTER(vp), sz, i32, vp, vp, vp,
                                                 ctypes.c_float, vp, vp]
        L.oracle_ar_residual_rmsnorm.restype = i32
        for name in ("oracle_f64_from_f16", "oracle_f64_from_bf16"):
            getattr(L, name).argtypes = [ctypes.c_uint16]
            getattr(L, name).restype = ctypes.c_double
        for name in ("oracle_f16_from_f64", "oracle_bf16_from_f64"):
            getattr(L, name).argtypes = [ctypes.c_double]
            getattr(L, name).restype = ctypes.c_uint16
        _lib = L
    return _lib


def dtype_code(dtype: str) -> int:
    return _DTYPES[dtype]


def _itemsize(code: int) -> int:
    return 4 if code == FP32 else 2


def _buf(a: Optional[np.ndarray], code: int, n: int, name: str):
    """Pointer to a C-contiguous host array holding n elements of the type."""
    if a is None:
        return None
    if not a.flags.c_contiguous:
        raise ValueError(f"{name} must be C-contiguous")
    if a.dtype.itemsize != _itemsize(code):
        raise ValueError(f"{name}: element size {a.dtype.itemsize} does not match the type")
    if a.size < n:
        raise ValueError(f"{name}: {a.size} elements, need {n}")
    return a.ctypes.data


def _parts(parts: Sequence[np.ndarray], code: int, n: int):
    arr = (ctypes.c_void_p * max(1, len(parts)))()
    for r, p in enumerate(parts):
        arr[r] = _buf(p, code, n, f"partial {r}")
    return arr


def ar_sum(dtype: str, parts: Sequence[np.ndarray], out: np.ndarray, n: Optional[int] = None) -> None:
    code = dtype_code(dtype)
    n = parts[0].size if n is None else n
    rc = lib().oracle_ar_sum(code, len(parts), _parts(parts, code, n), n, _buf(out, code, n, "out"))
    if rc:
        raise ValueError("oracle_ar_sum rejected its arguments")


def rmsnorm(dtype: str, x: np.ndarray, weight: np.ndarray, eps: float, out: np.ndarray, hidden: int) -> None:
    code = dtype_code(dtype)
    n = x.size
    rc = lib().oracle_rmsnorm(code, n, hidden, _buf(x, code, n, "x"), _buf(weight, code, hidden, "weight"),
                              eps, _buf(out, code, n, "out"))
    if rc:
        raise ValueError("oracle_rmsnorm rejected its arguments")


def ar_residual_rmsnorm(dtype: str, parts: Sequence[np.ndarray], hidden: int, weight: np.ndarray, eps: float,
                        out: np.ndarray, intermediate: np.ndarray, bias: Optional[np.ndarray] = None,
                        residual: Optional[np.ndarray] = None) -> None:
    code = dtype_code(dtype)
    n = parts[0].size
    rc = lib().oracle_ar_residual_rmsnorm(
        code, len(parts), _parts(parts, code, n), n, hidden,
        _buf(bias, code, hidden, "bias"), _buf(residual, code, n, "residual"),
        _buf(weight, code, hidden, "weight"), eps, _buf(out, code, n, "out"),
        _buf(intermediate, code, n, "intermediate"))
    if rc:
        raise ValueError("oracle_ar_residual_rmsnorm rejected its arguments")


def f64_from_f16(h: int) -> float:
    return lib().oracle_f64_from_f16(h)


def f64_from_bf16(h: int) -> float:
    return lib().oracle_f64_from_bf16(h)


def f16_from_f64(x: float) -> int:
    return lib().oracle_f16_from_f64(x)


def bf16_from_f64(x: float) -> int:
    return lib().oracle_bf16_from_f64(x)
