"""ctypes binding of ``libstream_ceiling.so`` (C ABI in include/stream_ceiling.h).

Measurement only: ``sc_stream(inputs, outputs, shape)`` reads every input
tensor and writes every output tensor once (outputs = bitwise XOR of the
inputs) with plain streaming code in one of SHAPES (a workgroup shape and a
store form), so that timing it on an all-reduce call's own buffers, in every
shape, gives that call's practical HBM ceiling.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libstream_ceiling.so")
SC_MAX_IN, SC_MAX_OUT = 12, 2
SC_OK = 0
# SC_SHAPE_* of include/stream_ceiling.h: lanes x packs per lane per step;
# "/sc1": device-scope buffer stores instead of non-temporal global stores;
# "/bl": non-temporal buffer loads instead of non-temporal global loads
_GEOMETRIES = ("512x2", "256x4", "256x8", "128x8")
SHAPES = {g + s + b: _GEOMETRIES[g] + ("/sc1" if s else "") + ("/bl" if b else "")
          for b in (0, 8) for s in (0, 4) for g in range(4)}

_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m tensor_all_reduce_ar_amd.build`")
    L = ctypes.CDLL(path)
    L.sc_stream.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p),
                            ctypes.c_int32, ctypes.c_size_t, ctypes.c_int32, ctypes.c_void_p]
    L.sc_stream.restype = ctypes.c_int32
    _lib = L
    return L


def sc_stream_raw(inputs: Sequence[int], outputs: Sequence[int], nbytes: int, shape: int = 0, stream: int = 0) -> int:
    """sc_stream on raw device addresses; returns the status."""
    ins = (ctypes.c_void_p * max(1, len(inputs)))(*inputs)
    outs = (ctypes.c_void_p * max(1, len(outputs)))(*outputs) if outputs else None
    return load().sc_stream(ins, len(inputs), outs, len(outputs), nbytes, shape, ctypes.c_void_p(stream))


def sc_stream(inputs: Sequence, outputs: Sequence, shape: int = 0, stream=None) -> None:
    """Read every tensor of `inputs` and write every tensor of `outputs` once
    (contiguous device tensors of one byte size, a multiple of 16)."""
    import torch
    nbytes = inputs[0].numel() * inputs[0].element_size()
    for t in list(inputs) + list(outputs):
        if not t.is_cuda or not t.is_contiguous() or t.numel() * t.element_size() != nbytes:
            raise ValueError("sc_stream needs contiguous device tensors of one byte size")
    h = int((stream or torch.cuda.current_stream()).cuda_stream)
    st = sc_stream_raw([t.data_ptr() for t in inputs], [t.data_ptr() for t in outputs], nbytes, shape, h)
    if st != SC_OK:
        raise RuntimeError(f"sc_stream failed with status {st}")
