"""ctypes binding of ``libar.so`` (C ABI in include/ar.h).

Argument marshalling only: every step of both ops runs in the HIP kernels of
csrc/ar.hip. torch supplies device memory and streams; tensors must be
contiguous CUDA (HIP) tensors of one dtype. The library is loaded on first use
and a missing library is an error (there is no fallback path).

Entry points, same names as the C ABI:
  ar_sum(partials, out)                                   fusion op NONE
  ar_residual_rmsnorm(partials, weight, eps, out, intermediate,
                      bias=None, residual=None, hidden_size=None)
                                                          fusion op RESIDUAL_RMS_NORM
  ar_rmsnorm(x, weight, eps, out, intermediate, ...)      the unfused path's norm step
  ar_sum_slice / ar_residual_rmsnorm_slice(..., slice_index, num_slices)
                                                          one share of a two-shot split
  ar_slice_range(params, fusion_op, slice_index, num_slices)
  ar_configuration_supported(params, fusion_op), ar_workspace_size(params),
  ar_partials_layout(elts_total, dtype, ranks), ar_status_string(code), ar_last_hip_error()
plus ``allocate_workspace`` (one device allocation holding the R partials at
the slots ar_partials_layout gives), ``prepare_sum`` /
``prepare_residual_rmsnorm`` / ``prepare_rmsnorm`` and the slice forms
``prepare_sum_slice`` / ``prepare_residual_rmsnorm_slice`` (a call whose
argument block is built and checked once, for loops that run the op on the
same buffers again and again), and ``Params`` / ``make_params``, ``call`` and
``call_slice`` for raw-pointer use.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libar.so")

AR_MAX_RANKS = 8
AR_FP32, AR_FP16, AR_BF16 = 0, 1, 2
AR_FUSION_NONE, AR_FUSION_RESIDUAL_RMS_NORM = 0, 1
AR_OK = 0
AR_ERR_NULL, AR_ERR_RANKS, AR_ERR_DTYPE, AR_ERR_SHAPE = -1, -2, -3, -4
AR_ERR_EPS, AR_ERR_ALIAS, AR_ERR_ALIGN, AR_ERR_SLICE, AR_ERR_HIP = -5, -6, -7, -8, -100
AR_SLOT_STAGGER_BYTES, AR_SLOT_ALIGN_BYTES = 4096, 256

# Every function include/ar.h declares.
EXPORTS = ("ar_sum", "ar_residual_rmsnorm", "ar_rmsnorm", "ar_sum_slice", "ar_residual_rmsnorm_slice",
           "ar_slice_range", "ar_configuration_supported", "ar_workspace_size", "ar_partials_layout",
           "ar_status_string", "ar_last_hip_error")


class FusionParams(ctypes.Structure):
    """ar_fusion_params_t (mirrors "type.d2" AllReduceFusionParams)."""
    _fields_ = [
        ("bias_buffer", ctypes.c_void_p),
        ("residual_buffer", ctypes.c_void_p),
        ("hidden_size", ctypes.c_int32),
        ("weight_buffer", ctypes.c_void_p),
        ("eps", ctypes.c_float),
        ("intermediate_buffer", ctypes.c_void_p),
    ]


class Params(ctypes.Structure):
    """ar_params_t (mirrors "type.d2" AllReduceParams)."""
    _fields_ = [
        ("elts_total", ctypes.c_size_t),
        ("ranks", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("input_buffer_ptrs", ctypes.c_void_p * AR_MAX_RANKS),
        ("local_output_buffer_ptr", ctypes.c_void_p),
        ("fusion_params", FusionParams),
    ]


class ArError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        msg = f"{what}: {ar_status_string(status)}"
        if status == AR_ERR_HIP:
            msg += f" (hipError_t {ar_last_hip_error()})"
        super().__init__(msg)


_lib: Optional[ctypes.CDLL] = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m tensor_all_reduce_ar_amd.build`")
    L = ctypes.CDLL(path)
    P = ctypes.POINTER(Params)
    L.ar_sum.argtypes = [P, ctypes.c_void_p]
    L.ar_sum.restype = ctypes.c_int32
    L.ar_residual_rmsnorm.argtypes = [P, ctypes.c_void_p]
    L.ar_residual_rmsnorm.restype = ctypes.c_int32
    L.ar_rmsnorm.argtypes = [P, ctypes.c_void_p]
    L.ar_rmsnorm.restype = ctypes.c_int32
    for name in ("ar_sum_slice", "ar_residual_rmsnorm_slice"):
        getattr(L, name).argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p]
        getattr(L, name).restype = ctypes.c_int32
    L.ar_slice_range.argtypes = [P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                 ctypes.POINTER(ctypes.c_size_t)]
    L.ar_slice_range.restype = ctypes.c_int32
    L.ar_configuration_supported.argtypes = [P, ctypes.c_int32]
    L.ar_configuration_supported.restype = ctypes.c_int32
    L.ar_workspace_size.argtypes = [P]
    L.ar_workspace_size.restype = ctypes.c_size_t
    L.ar_partials_layout.argtypes = [ctypes.c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_size_t),
                                     ctypes.POINTER(ctypes.c_size_t)]
    L.ar_partials_layout.restype = ctypes.c_int32
    L.ar_status_string.argtypes = [ctypes.c_int32]
    L.ar_status_string.restype = ctypes.c_char_p
    L.ar_last_hip_error.argtypes = []
    L.ar_last_hip_error.restype = ctypes.c_int32
    _lib = L
    return L


def ar_status_string(status: int) -> str:
    return load().ar_status_string(status).decode()


def ar_last_hip_error() -> int:
    return load().ar_last_hip_error()


_PtrArray = ctypes.c_void_p * AR_MAX_RANKS


def make_params(elts_total: int, ranks: int, dtype: int, inputs: Sequence[int], output: int,
                hidden_size: int = 0, weight: int = 0, eps: float = 0.0, intermediate: int = 0,
                bias: int = 0, residual: int = 0) -> Params:
    """Fill an ar_params_t from raw device addresses (0 = NULL); entries of
    `inputs` past AR_MAX_RANKS are ignored, missing ones are NULL."""
    ptrs = _PtrArray(*[q or None for q in list(inputs)[:AR_MAX_RANKS]])
    fusion = FusionParams(bias or None, residual or None, hidden_size, weight or None, eps, intermediate or None)
    return Params(elts_total, ranks, dtype, ptrs, output or None, fusion)


def call(fn: str, params: Params, stream: Optional[int] = None) -> int:
    """Call ar_sum / ar_residual_rmsnorm / ar_rmsnorm with a filled Params; returns the status."""
    return getattr(load(), fn)(ctypes.byref(params), ctypes.c_void_p(stream or 0))


def call_slice(fn: str, params: Params, slice_index: int, num_slices: int, stream: Optional[int] = None) -> int:
    """Call ar_sum_slice / ar_residual_rmsnorm_slice; returns the status."""
    return getattr(load(), fn)(ctypes.byref(params), slice_index, num_slices, ctypes.c_void_p(stream or 0))


def ar_slice_range(params: Params, fusion_op: int, slice_index: int, num_slices: int):
    """(status, begin, end) of a slice; begin/end are element indices."""
    b, e = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = load().ar_slice_range(ctypes.byref(params), fusion_op, slice_index, num_slices, ctypes.byref(b),
                               ctypes.byref(e))
    return st, b.value, e.value


def ar_configuration_supported(params: Params, fusion_op: int) -> int:
    return load().ar_configuration_supported(ctypes.byref(params), fusion_op)


def ar_workspace_size(params: Optional[Params] = None) -> int:
    return load().ar_workspace_size(ctypes.byref(params) if params is not None else None)


def ar_partials_layout(elts_total: int, dtype: int, ranks: int):
    """(status, slot byte offsets, total bytes) of the recommended one-allocation
    layout of `ranks` partials of `elts_total` elements of type `dtype`."""
    offs = (ctypes.c_size_t * max(1, ranks))()
    total = ctypes.c_size_t(0)
    st = load().ar_partials_layout(elts_total, dtype, ranks, offs if ranks > 0 else None, ctypes.byref(total))
    return st, [offs[r] for r in range(max(0, ranks))] if st == AR_OK else [], total.value


class Workspace:
    """One device allocation holding R partials of ``elts_total`` elements at
    the slot offsets of ar_partials_layout.

    ``buffer`` is the allocation (uint8, ``total_bytes`` long), ``partials``
    the R typed 1-D views (one per rank, in rank order), ``offsets`` their
    byte offsets in it. The views are what the producers of the partials
    write and what ar_sum / ar_residual_rmsnorm read; they share ``buffer``'s
    memory, which lives as long as any of them does."""

    def __init__(self, buffer, partials, offsets, total_bytes: int):
        self.buffer, self.partials, self.offsets, self.total_bytes = buffer, partials, offsets, total_bytes


def allocate_workspace(elts_total: int, dtype, ranks: int, device=None) -> Workspace:
    """Allocate the R partials in one device allocation laid out by
    ar_partials_layout (the one-GPU counterpart of the comm-buffer workspace
    that CustomAllReduceHelper sizes and allocates in "allreduce.d2",
    allocate_workspace(mapping, size): there each rank's buffer is a peer's;
    here every slot is local). The slots are 256-byte aligned and staggered by
    4 KiB, which the fused kernel reads faster than separate power-of-two
    allocations. ``dtype`` is a torch dtype (float32, float16, bfloat16);
    ``device`` defaults to the current CUDA (HIP) device. The contents are
    uninitialised. Raises ArError if the layout is rejected."""
    import torch
    code = _dtype_code(torch.empty(0, dtype=dtype))
    st, offs, total = ar_partials_layout(int(elts_total), code, int(ranks))
    if st != AR_OK:
        raise ArError(st, "ar_partials_layout")
    dev = torch.device("cuda") if device is None else torch.device(device)
    buf = torch.empty(total, dtype=torch.uint8, device=dev)
    size = torch.empty(0, dtype=dtype).element_size()
    views = [buf[o:o + int(elts_total) * size].view(dtype) for o in offs]
    return Workspace(buf, views, offs, total)


# ------------------------------------------------------------ torch front end
_CODES = {}


def _dtype_code(t) -> int:
    if not _CODES:
        import torch
        _CODES.update({torch.float32: AR_FP32, torch.float16: AR_FP16, torch.bfloat16: AR_BF16})
    code = _CODES.get(t.dtype)
    if code is None:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return code


def _check(t, name: str, dtype, numel: int, device=None):
    """t.data_ptr() once t is a contiguous device tensor of `numel` elements
    of `dtype` (on `device`, if given); raises otherwise. The usual case is
    one chained test of cheap attributes; the messages are built only when it
    fails."""
    idx = t.get_device()  # -1 for a host tensor
    if t.dtype is dtype and idx >= 0 and (device is None or idx == device.index) and t.numel() == numel \
            and t.is_contiguous():
        return t.data_ptr()
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, the output on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    raise ValueError(f"{name} has {t.numel()} elements, expected {numel}")


def _stream_handle(stream, device) -> int:
    import torch
    if stream is None:
        # torch's current stream on `device` as a raw handle; the raw query
        # skips building a Stream object (about 2 us a call)
        raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        if raw is not None:
            return int(raw(device.index))
        stream = torch.cuda.current_stream(device)
    elif stream.device != device:
        raise ValueError(f"stream is on {stream.device}, the buffers on {device}")
    return int(stream.cuda_stream)


def _run(fn, params, stream, device, slice_args=None) -> None:
    """Launch on the buffers' device (the library uses the current one);
    switches device only when that device is not already current."""
    import torch
    if device.index == torch.cuda.current_device():
        h = _stream_handle(stream, device)
        st = call(fn, params, h) if slice_args is None else call_slice(fn, params, *slice_args, h)
    else:
        with torch.cuda.device(device):
            h = _stream_handle(stream, device)
            st = call(fn, params, h) if slice_args is None else call_slice(fn, params, *slice_args, h)
    if st != AR_OK:
        raise ArError(st, fn)


def ar_sum(partials: Sequence, out, stream=None) -> None:
    """out = sum of the partials (fusion op NONE), on `stream` (default: torch's current)."""
    _run("ar_sum", _sum_params(partials, out), stream, out.device)


def _fused_params(partials, weight, eps, out, intermediate, bias, residual, hidden_size) -> Params:
    if not 1 <= len(partials) <= AR_MAX_RANKS:
        raise ValueError(f"need 1..{AR_MAX_RANKS} partials, got {len(partials)}")
    n, dt = out.numel(), out.dtype
    optr = _check(out, "out", dt, n)
    d = out.device
    H = int(hidden_size if hidden_size is not None else weight.numel())
    ptrs = [_check(p, f"partial {r}", dt, n, d) for r, p in enumerate(partials)]
    return make_params(
        n, len(partials), _dtype_code(out), ptrs, optr, hidden_size=H,
        weight=_check(weight, "weight", dt, H, d), eps=float(eps),
        intermediate=_check(intermediate, "intermediate", dt, n, d),
        bias=_check(bias, "bias", dt, H, d) if bias is not None else 0,
        residual=_check(residual, "residual", dt, n, d) if residual is not None else 0)


def _sum_params(partials, out) -> Params:
    if not 1 <= len(partials) <= AR_MAX_RANKS:
        raise ValueError(f"need 1..{AR_MAX_RANKS} partials, got {len(partials)}")
    n, dt = out.numel(), out.dtype
    optr = _check(out, "out", dt, n)
    ptrs = [_check(p, f"partial {r}", dt, n, out.device) for r, p in enumerate(partials)]
    return make_params(n, len(partials), _dtype_code(out), ptrs, optr)


def ar_residual_rmsnorm(partials: Sequence, weight, eps: float, out, intermediate, bias=None, residual=None,
                        hidden_size: Optional[int] = None, stream=None) -> None:
    """Fusion op RESIDUAL_RMS_NORM: intermediate = ((sum + bias) + residual),
    out = RMSNorm(intermediate) * weight over rows of hidden_size elements
    (default: the weight's length)."""
    params = _fused_params(partials, weight, eps, out, intermediate, bias, residual, hidden_size)
    _run("ar_residual_rmsnorm", params, stream, out.device)


def ar_rmsnorm(x, weight, eps: float, out, intermediate, bias=None, residual=None,
               hidden_size: Optional[int] = None, stream=None) -> None:
    """The unfused path's norm step on one input x: intermediate =
    (x + bias) + residual, out = RMSNorm(intermediate) * weight."""
    params = _fused_params([x], weight, eps, out, intermediate, bias, residual, hidden_size)
    _run("ar_rmsnorm", params, stream, out.device)


def ar_sum_slice(partials: Sequence, out, slice_index: int, num_slices: int, stream=None) -> None:
    """Slice `slice_index` of `num_slices` of ar_sum, written in place into out."""
    _run("ar_sum_slice", _sum_params(partials, out), stream, out.device, (slice_index, num_slices))


def ar_residual_rmsnorm_slice(partials: Sequence, weight, eps: float, out, intermediate, slice_index: int,
                              num_slices: int, bias=None, residual=None, hidden_size: Optional[int] = None,
                              stream=None) -> None:
    """Rows of slice `slice_index` of `num_slices` of ar_residual_rmsnorm, in place."""
    params = _fused_params(partials, weight, eps, out, intermediate, bias, residual, hidden_size)
    _run("ar_residual_rmsnorm_slice", params, stream, out.device, (slice_index, num_slices))


class PreparedCall:
    """One entry point bound to one set of buffers: the ar_params_t block is
    built and the tensors checked once, when the call is prepared; each call
    then only reads the current stream and calls the C entry point, whose own
    validation still runs. The call keeps references to its tensors, so they
    stay allocated while it exists; they must not be resized or re-pointed
    (the block holds their addresses). Raises ArError on a non-zero status."""

    def __init__(self, fn: str, params: Params, device, tensors, slice_args=None):
        self.fn, self.params, self.device, self._keep = fn, params, device, tensors
        self._slice = tuple(slice_args) if slice_args is not None else None
        self._c = getattr(load(), fn)
        self._pp = ctypes.byref(params)
        import torch
        self._raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        self._dev = getattr(torch._C, "_cuda_getDevice", None)

    def __call__(self, stream=None) -> None:
        idx = self.device.index
        if self._dev is not None and self._dev() == idx:
            if stream is None and self._raw is not None:
                h = self._raw(idx)
            else:
                h = _stream_handle(stream, self.device)
            if self._slice is None:
                st = self._c(self._pp, ctypes.c_void_p(h))
            else:
                st = self._c(self._pp, self._slice[0], self._slice[1], ctypes.c_void_p(h))
            if st != AR_OK:
                raise ArError(st, self.fn)
            return
        _run(self.fn, self.params, stream, self.device, self._slice)


def prepare_sum(partials: Sequence, out) -> PreparedCall:
    """ar_sum on these buffers, ready to call: ``prepare_sum(parts, out)()``."""
    return PreparedCall("ar_sum", _sum_params(partials, out), out.device, (list(partials), out))


def prepare_residual_rmsnorm(partials: Sequence, weight, eps: float, out, intermediate, bias=None, residual=None,
                             hidden_size: Optional[int] = None) -> PreparedCall:
    """ar_residual_rmsnorm on these buffers, ready to call."""
    params = _fused_params(partials, weight, eps, out, intermediate, bias, residual, hidden_size)
    return PreparedCall("ar_residual_rmsnorm", params, out.device,
                        (list(partials), weight, out, intermediate, bias, residual))


def prepare_sum_slice(partials: Sequence, out, slice_index: int, num_slices: int) -> PreparedCall:
    """ar_sum_slice on these buffers and this slice, ready to call."""
    return PreparedCall("ar_sum_slice", _sum_params(partials, out), out.device, (list(partials), out),
                        (slice_index, num_slices))


def prepare_residual_rmsnorm_slice(partials: Sequence, weight, eps: float, out, intermediate, slice_index: int,
                                   num_slices: int, bias=None, residual=None,
                                   hidden_size: Optional[int] = None) -> PreparedCall:
    """ar_residual_rmsnorm_slice on these buffers and this slice, ready to call."""
    params = _fused_params(partials, weight, eps, out, intermediate, bias, residual, hidden_size)
    return PreparedCall("ar_residual_rmsnorm_slice", params, out.device,
                        (list(partials), weight, out, intermediate, bias, residual), (slice_index, num_slices))


def prepare_rmsnorm(x, weight, eps: float, out, intermediate, bias=None, residual=None,
                    hidden_size: Optional[int] = None) -> PreparedCall:
    """ar_rmsnorm (the unfused path's norm step) on these buffers, ready to call."""
    params = _fused_params([x], weight, eps, out, intermediate, bias, residual, hidden_size)
    return PreparedCall("ar_rmsnorm", params, out.device, (x, weight, out, intermediate, bias, residual))
