"""The C ABI on the host (no GPU): the library loads and exports every
function include/ar.h declares, the ctypes mirrors match the C layout, and
every validation error is returned before any HIP call.

Validation calls use made-up addresses: they are never dereferenced because
each call is rejected (or is a no-op) before anything is launched.
"""
import ctypes
import math
import os
import re
import subprocess

import pytest

from tensor_all_reduce_ar_amd import ar

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ar.h")
A = 0x7F0000000000  # made-up, 256-byte aligned device-like addresses
MB = 1 << 20


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(ar_[a-z_0-9]+)\s*\(", text, flags=re.M)


def test_library_exports_every_declared_function():
    lib = ar.load()
    declared = header_functions()
    assert set(declared) == set(ar.EXPORTS), declared
    for name in declared:
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", ar.LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r"\bT (ar_\w+)", nm.stdout))
    assert set(declared) <= exported


def _c_layout(tmp_path):
    src = tmp_path / "layout.c"
    src.write_text(r'''
#include <stdio.h>
#include <stddef.h>
#include "ar.h"
#define OFF(T, f) printf(#T "." #f " %zu\n", offsetof(T, f))
int main(void) {
  printf("sizeof.ar_params_t %zu\nsizeof.ar_fusion_params_t %zu\n", sizeof(ar_params_t), sizeof(ar_fusion_params_t));
  OFF(ar_params_t, elts_total); OFF(ar_params_t, ranks); OFF(ar_params_t, dtype);
  OFF(ar_params_t, input_buffer_ptrs); OFF(ar_params_t, local_output_buffer_ptr); OFF(ar_params_t, fusion_params);
  OFF(ar_fusion_params_t, bias_buffer); OFF(ar_fusion_params_t, residual_buffer); OFF(ar_fusion_params_t, hidden_size);
  OFF(ar_fusion_params_t, weight_buffer); OFF(ar_fusion_params_t, eps); OFF(ar_fusion_params_t, intermediate_buffer);
  printf("enum.AR_MAX_RANKS %d\nenum.AR_FP32 %d\nenum.AR_FP16 %d\nenum.AR_BF16 %d\n", AR_MAX_RANKS, AR_FP32, AR_FP16, AR_BF16);
  printf("enum.AR_FUSION_NONE %d\nenum.AR_FUSION_RESIDUAL_RMS_NORM %d\n", AR_FUSION_NONE, AR_FUSION_RESIDUAL_RMS_NORM);
  printf("enum.AR_OK %d\nenum.AR_ERR_NULL %d\nenum.AR_ERR_RANKS %d\nenum.AR_ERR_DTYPE %d\nenum.AR_ERR_SHAPE %d\n",
         AR_OK, AR_ERR_NULL, AR_ERR_RANKS, AR_ERR_DTYPE, AR_ERR_SHAPE);
  printf("enum.AR_ERR_EPS %d\nenum.AR_ERR_ALIAS %d\nenum.AR_ERR_ALIGN %d\nenum.AR_ERR_HIP %d\n",
         AR_ERR_EPS, AR_ERR_ALIAS, AR_ERR_ALIGN, AR_ERR_HIP);
  printf("enum.AR_ERR_SLICE %d\n", AR_ERR_SLICE);
  printf("enum.AR_SLOT_STAGGER_BYTES %d\nenum.AR_SLOT_ALIGN_BYTES %d\n", AR_SLOT_STAGGER_BYTES, AR_SLOT_ALIGN_BYTES);
  return 0;
}
''')
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-Wall", "-I", os.path.join(ROOT, "include"), "-o", str(exe), str(src)],
                   check=True)
    out = subprocess.run([str(exe)], capture_output=True, text=True, check=True).stdout
    return {k: int(v) for k, v in (line.split() for line in out.strip().splitlines())}


def test_ctypes_mirrors_match_the_header(tmp_path):
    c = _c_layout(tmp_path)
    assert c["sizeof.ar_params_t"] == ctypes.sizeof(ar.Params)
    assert c["sizeof.ar_fusion_params_t"] == ctypes.sizeof(ar.FusionParams)
    for f, *_ in ar.Params._fields_:
        assert c[f"ar_params_t.{f}"] == getattr(ar.Params, f).offset, f
    for f, *_ in ar.FusionParams._fields_:
        assert c[f"ar_fusion_params_t.{f}"] == getattr(ar.FusionParams, f).offset, f
    for name in ("AR_MAX_RANKS", "AR_FP32", "AR_FP16", "AR_BF16", "AR_FUSION_NONE", "AR_FUSION_RESIDUAL_RMS_NORM",
                 "AR_OK", "AR_ERR_NULL", "AR_ERR_RANKS", "AR_ERR_DTYPE", "AR_ERR_SHAPE", "AR_ERR_EPS",
                 "AR_ERR_ALIAS", "AR_ERR_ALIGN", "AR_ERR_SLICE", "AR_ERR_HIP", "AR_SLOT_STAGGER_BYTES",
                 "AR_SLOT_ALIGN_BYTES"):
        assert c[f"enum.{name}"] == getattr(ar, name), name


def test_fusion_op_values_follow_the_type_sheet():
    # "type.d2", enum AllReduceFusionOp: NONE 0, RESIDUAL_RMS_NORM 1
    assert (ar.AR_FUSION_NONE, ar.AR_FUSION_RESIDUAL_RMS_NORM) == (0, 1)


def sum_params(n=1024, ranks=2, dtype=ar.AR_FP32, inputs=None, out=None):
    inputs = inputs if inputs is not None else [A + r * 16 * MB for r in range(ranks)]
    return ar.make_params(n, ranks, dtype, inputs, out if out is not None else A + 512 * MB)


def fused_params(n=4096, ranks=2, dtype=ar.AR_BF16, hidden=1024, eps=1e-6, **kw):
    d = dict(inputs=[A + r * 16 * MB for r in range(ranks)], output=A + 256 * MB, weight=A + 300 * MB,
             intermediate=A + 320 * MB, bias=A + 340 * MB, residual=A + 360 * MB)
    d.update(kw)
    return ar.make_params(n, ranks, dtype, d["inputs"], d["output"], hidden_size=hidden, weight=d["weight"],
                          eps=eps, intermediate=d["intermediate"], bias=d["bias"], residual=d["residual"])


def sum_status(p):
    return ar.ar_configuration_supported(p, ar.AR_FUSION_NONE)


def fused_status(p):
    return ar.ar_configuration_supported(p, ar.AR_FUSION_RESIDUAL_RMS_NORM)


def test_null_params():
    lib = ar.load()
    assert lib.ar_sum(None, None) == ar.AR_ERR_NULL
    assert lib.ar_residual_rmsnorm(None, None) == ar.AR_ERR_NULL
    assert lib.ar_configuration_supported(None, 0) == ar.AR_ERR_NULL


@pytest.mark.parametrize("ranks", [0, -1, 9, 100])
def test_bad_rank_count(ranks):
    p = sum_params(ranks=2)
    p.ranks = ranks
    assert ar.call("ar_sum", p) == ar.AR_ERR_RANKS
    assert ar.call("ar_residual_rmsnorm", fused_params_with(ranks=ranks)) == ar.AR_ERR_RANKS


def fused_params_with(**kw):
    p = fused_params()
    for k, v in kw.items():
        setattr(p, k, v)
    return p


@pytest.mark.parametrize("dtype", [-1, 3, 7])
def test_bad_dtype(dtype):
    assert ar.call("ar_sum", sum_params(dtype=dtype)) == ar.AR_ERR_DTYPE
    assert ar.call("ar_residual_rmsnorm", fused_params(dtype=dtype)) == ar.AR_ERR_DTYPE


def test_null_buffers():
    assert ar.call("ar_sum", sum_params(inputs=[A, 0])) == ar.AR_ERR_NULL
    assert ar.call("ar_sum", sum_params(out=0)) == ar.AR_ERR_NULL
    for k in ("output", "weight", "intermediate"):
        assert ar.call("ar_residual_rmsnorm", fused_params(**{k: 0})) == ar.AR_ERR_NULL, k
    assert ar.call("ar_residual_rmsnorm", fused_params(inputs=[A, 0])) == ar.AR_ERR_NULL
    # bias and residual are optional: NULL is valid
    assert fused_status(fused_params(bias=0, residual=0)) == 1


@pytest.mark.parametrize("hidden,n", [(0, 4096), (-8, 4096), (1000, 4096), (3, 10)])
def test_bad_shape(hidden, n):
    assert ar.call("ar_residual_rmsnorm", fused_params(n=n, hidden=hidden)) == ar.AR_ERR_SHAPE


@pytest.mark.parametrize("eps", [math.nan, math.inf, -math.inf, -1e-6])
def test_bad_eps(eps):
    assert ar.call("ar_residual_rmsnorm", fused_params(eps=eps)) == ar.AR_ERR_EPS


def test_empty_is_a_noop_without_any_hip_call():
    assert ar.call("ar_sum", sum_params(n=0)) == ar.AR_OK
    assert ar.call("ar_residual_rmsnorm", fused_params(n=0)) == ar.AR_OK
    # still validated: bad ranks/dtype/shape/eps are reported for empty calls too
    assert ar.call("ar_sum", sum_params(n=0, ranks=9, inputs=[A] * 8)) == ar.AR_ERR_RANKS
    assert ar.call("ar_residual_rmsnorm", fused_params(n=0, hidden=0)) == ar.AR_ERR_SHAPE


def test_in_place_sum_passthrough_is_a_noop():
    # one rank, output == input: nothing to do, no HIP call
    assert ar.call("ar_sum", sum_params(ranks=1, inputs=[A], out=A)) == ar.AR_OK


def test_aliasing_rules():
    n, s = 1024, 4
    # exact aliasing of the output with a partial: allowed (in place)
    assert sum_status(sum_params(n=n, inputs=[A, A + MB], out=A)) == 1
    # partial overlap: rejected
    assert ar.call("ar_sum", sum_params(n=n, inputs=[A, A + MB], out=A + s * 8)) == ar.AR_ERR_ALIAS
    # fused: intermediate may be the residual or a partial; output may be a partial
    assert fused_status(fused_params(intermediate=A + 360 * MB)) == 1
    assert fused_status(fused_params(output=A)) == 1
    # output and intermediate may not overlap each other
    assert ar.call("ar_residual_rmsnorm", fused_params(output=A + 320 * MB)) == ar.AR_ERR_ALIAS
    # outputs may not overlap bias / weight
    assert ar.call("ar_residual_rmsnorm", fused_params(weight=A + 256 * MB + 64)) == ar.AR_ERR_ALIAS
    assert ar.call("ar_residual_rmsnorm", fused_params(bias=A + 320 * MB)) == ar.AR_ERR_ALIAS
    # partial overlap of the intermediate with the residual
    assert ar.call("ar_residual_rmsnorm", fused_params(intermediate=A + 360 * MB + 32)) == ar.AR_ERR_ALIAS


def test_alignment_rules():
    # element alignment is required
    assert ar.call("ar_sum", sum_params(dtype=ar.AR_FP16, inputs=[A + 1, A + MB])) == ar.AR_ERR_ALIGN
    assert ar.call("ar_sum", sum_params(dtype=ar.AR_FP32, out=A + 512 * MB + 2)) == ar.AR_ERR_ALIGN
    assert ar.call("ar_residual_rmsnorm", fused_params(weight=A + 300 * MB + 1)) == ar.AR_ERR_ALIGN
    # element-aligned but not 16-byte aligned: valid, element-wise path
    assert sum_status(sum_params(dtype=ar.AR_FP16, inputs=[A + 2, A + MB])) == 0
    assert sum_status(sum_params(dtype=ar.AR_FP32, out=A + 512 * MB + 4)) == 0
    assert sum_status(sum_params(dtype=ar.AR_FP16)) == 1
    assert fused_status(fused_params(residual=A + 360 * MB + 2)) == 0
    # a row whose byte size is not a multiple of 16 takes the element-wise path
    assert fused_status(fused_params(n=4100 * 2, hidden=4100)) == 0
    assert fused_status(fused_params(n=5120 * 3, hidden=5120, dtype=ar.AR_FP16)) == 1
    # rows wider than the register path still take the vector (two-pass) path
    assert fused_status(fused_params(n=65536 * 2, hidden=65536)) == 1


def test_workspace_and_status_strings():
    assert ar.ar_workspace_size(sum_params()) == 0
    assert ar.ar_workspace_size(None) == 0
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8, -100, 1, -99, 12345):
        s = ar.ar_status_string(code)
        assert isinstance(s, str) and s
    assert ar.ar_status_string(ar.AR_ERR_ALIAS).startswith("AR_ERR_ALIAS")


@pytest.mark.parametrize("dtype,size", [(ar.AR_FP32, 4), (ar.AR_FP16, 2), (ar.AR_BF16, 2)])
@pytest.mark.parametrize("n", [0, 1, 100, 4096, 2048 * 8192, (1 << 31) + 1003])
def test_partials_layout(dtype, size, n):
    """Slots: consecutive, in order, each 256-byte aligned, at least the
    partial's bytes apart, and 4 KiB further apart than the rounded size."""
    for ranks in range(1, 9):
        st, offs, total = ar.ar_partials_layout(n, dtype, ranks)
        assert st == ar.AR_OK and len(offs) == ranks
        stride = -(-n * size // 256) * 256 + 4096
        assert offs == [r * stride for r in range(ranks)]
        assert total == ranks * stride
        for r in range(ranks):
            assert offs[r] % 256 == 0
            assert offs[r] + n * size <= (offs[r + 1] if r + 1 < ranks else total)


def test_partials_layout_errors():
    assert ar.ar_partials_layout(100, 7, 2)[0] == ar.AR_ERR_DTYPE
    assert ar.ar_partials_layout(100, ar.AR_FP16, 0)[0] == ar.AR_ERR_RANKS
    assert ar.ar_partials_layout(100, ar.AR_FP16, 9)[0] == ar.AR_ERR_RANKS
    total = ctypes.c_size_t(0)
    assert ar.load().ar_partials_layout(100, ar.AR_FP16, 2, None, ctypes.byref(total)) == ar.AR_ERR_NULL
    offs = (ctypes.c_size_t * 2)()
    assert ar.load().ar_partials_layout(100, ar.AR_FP16, 2, offs, None) == ar.AR_ERR_NULL


def test_unknown_fusion_op_rejected():
    assert ar.ar_configuration_supported(sum_params(), 2) < 0


def hip_devices_visible() -> bool:
    """Whether the HIP runtime libar.so links sees a device (asked directly,
    not through torch, whose device list can differ). Any doubt counts as yes."""
    try:
        hip = ctypes.CDLL("libamdhip64.so")
    except OSError:
        try:
            hip = ctypes.CDLL("/opt/rocm/lib/libamdhip64.so")
        except OSError:
            return True
    n = ctypes.c_int(0)
    rc = hip.hipGetDeviceCount(ctypes.byref(n))
    return rc == 0 and n.value > 0 or rc not in (0, 100)  # 100: hipErrorNoDevice


no_hip_device = pytest.mark.skipif(hip_devices_visible(),
                                   reason="host-only case: a HIP device is visible, and a validation bug here "
                                          "would launch on made-up addresses")


@no_hip_device
def test_launch_without_a_device_reports_hip_error():
    """Forced from the host: with no GPU present, a valid call reaches the
    launch, which fails; the status is AR_ERR_HIP and nothing is thrown."""
    assert ar.call("ar_sum", sum_params()) == ar.AR_ERR_HIP
    assert ar.ar_last_hip_error() != 0
    assert ar.call("ar_residual_rmsnorm", fused_params()) == ar.AR_ERR_HIP


SIZE_MAX = (1 << 64) - 1


@no_hip_device
@pytest.mark.parametrize("n,dtype", [((1 << 62) + 16, ar.AR_FP32), (SIZE_MAX // 2 + 1, ar.AR_FP16),
                                     (SIZE_MAX // 2 + 1, ar.AR_BF16), (SIZE_MAX // 4 + 1, ar.AR_FP32),
                                     (SIZE_MAX, ar.AR_BF16)])
def test_sizes_whose_bytes_wrap_are_rejected_everywhere(n, dtype):
    """elts_total * sizeof(T) past SIZE_MAX: every entry point returns
    AR_ERR_SHAPE before any HIP call (the wrapped byte count would otherwise
    pass every aliasing check and launch over the whole size)."""
    hidden = 16
    for ranks in (1, 2, 8):
        sp = sum_params(n=n, ranks=ranks, dtype=dtype)
        fp = fused_params(n=n, ranks=ranks, dtype=dtype, hidden=hidden) if n % hidden == 0 else None
        assert ar.call("ar_sum", sp) == ar.AR_ERR_SHAPE
        assert sum_status(sp) == ar.AR_ERR_SHAPE
        assert ar.call_slice("ar_sum_slice", sp, 0, 2) == ar.AR_ERR_SHAPE
        assert ar.ar_slice_range(sp, ar.AR_FUSION_NONE, 0, 2)[0] == ar.AR_ERR_SHAPE
        if fp is not None:
            assert ar.call("ar_residual_rmsnorm", fp) == ar.AR_ERR_SHAPE
            assert fused_status(fp) == ar.AR_ERR_SHAPE
            assert ar.call_slice("ar_residual_rmsnorm_slice", fp, 1, 2) == ar.AR_ERR_SHAPE
            assert ar.ar_slice_range(fp, ar.AR_FUSION_RESIDUAL_RMS_NORM, 0, 2)[0] == ar.AR_ERR_SHAPE
            if ranks == 1:
                assert ar.call("ar_rmsnorm", fp) == ar.AR_ERR_SHAPE


@no_hip_device
def test_buffers_past_the_end_of_the_address_space_are_rejected():
    top = SIZE_MAX & ~255
    n = 1 << 40  # 2 TiB of fp16: fits size_t, not below `top`
    assert ar.call("ar_sum", sum_params(n=n, dtype=ar.AR_FP16, out=top - (1 << 38))) == ar.AR_ERR_SHAPE
    assert ar.call("ar_sum", sum_params(n=n, dtype=ar.AR_FP16, inputs=[A, top - 256])) == ar.AR_ERR_SHAPE
    assert ar.call("ar_residual_rmsnorm", fused_params(n=n, dtype=ar.AR_FP16, residual=top)) == ar.AR_ERR_SHAPE
    assert ar.call("ar_residual_rmsnorm", fused_params(n=1 << 20, hidden=1 << 20, weight=top)) == ar.AR_ERR_SHAPE


def test_partials_layout_rejects_sizes_that_do_not_fit():
    assert ar.ar_partials_layout((1 << 62) + 1, ar.AR_FP32, 8)[0] == ar.AR_ERR_SHAPE
    assert ar.ar_partials_layout(1 << 59, ar.AR_FP32, 8)[0] == ar.AR_ERR_SHAPE   # ranks * stride wraps
    assert ar.ar_partials_layout(SIZE_MAX // 2, ar.AR_FP16, 1)[0] == ar.AR_ERR_SHAPE  # round-up wraps
    st, offs, total = ar.ar_partials_layout(1 << 58, ar.AR_FP32, 8)
    assert st == ar.AR_OK and total == 8 * ((1 << 60) + 4096)


def test_product_path_fails_loudly_without_the_library(tmp_path):
    """No fallback: a missing library is an error, not a silent CPU path."""
    saved = ar._lib
    try:
        ar._lib = None
        with pytest.raises(RuntimeError, match="missing"):
            ar.load(str(tmp_path / "libar.so"))
    finally:
        ar._lib = saved


def test_torch_front_end_checks_arguments():
    import torch
    x = torch.zeros(8)
    with pytest.raises(ValueError):
        ar.ar_sum([x, x], x)  # host tensors are not device buffers
    with pytest.raises(ValueError):
        ar.ar_sum([], x)


# ------------------------------------------------- two-shot slices (host)
@pytest.mark.parametrize("dtype,size", [(ar.AR_FP32, 4), (ar.AR_FP16, 2), (ar.AR_BF16, 2)])
@pytest.mark.parametrize("n", [1, 7, 8, 100, 1000003, 8192 * 8192])
@pytest.mark.parametrize("num", [1, 2, 3, 4, 7, 8])
def test_sum_slices_partition_with_aligned_starts(dtype, size, n, num):
    """Slices cover [0, N) in order without gaps or overlap; each starts on a
    16-byte boundary; all but the last non-empty one have the same length."""
    p = sum_params(n=n, dtype=dtype)
    ranges = []
    for k in range(num):
        st, b, e = ar.ar_slice_range(p, ar.AR_FUSION_NONE, k, num)
        assert st == ar.AR_OK
        ranges.append((b, e))
    assert ranges[0][0] == 0 and ranges[-1][1] == n
    for (b0, e0), (b1, e1) in zip(ranges, ranges[1:]):
        assert e0 == b1 and b1 <= e1
    for b, e in ranges:
        if e > b:  # empty trailing slices sit at N
            assert (b * size) % 16 == 0
    lens = [e - b for b, e in ranges if e > b]
    assert len(set(lens[:-1])) <= 1 and lens[-1] <= lens[0]
    assert lens[0] >= -(-n // num)  # at least the even share (the elts_per_rank of a two-shot split)


@pytest.mark.parametrize("rows,num", [(1, 1), (1, 8), (7, 2), (2048, 8), (4096, 3), (33, 8)])
def test_fused_slices_are_whole_rows(rows, num):
    H = 1024
    p = fused_params(n=rows * H, hidden=H)
    covered = 0
    for k in range(num):
        st, b, e = ar.ar_slice_range(p, ar.AR_FUSION_RESIDUAL_RMS_NORM, k, num)
        assert st == ar.AR_OK and b == covered and b % H == 0 and e % H == 0 and e >= b
        covered = e
    assert covered == rows * H


def test_slice_arguments_validated():
    p = sum_params()
    for k, num in ((0, 0), (-1, 2), (2, 2), (0, 1025)):
        assert ar.ar_slice_range(p, ar.AR_FUSION_NONE, k, num)[0] == ar.AR_ERR_SLICE
        assert ar.call_slice("ar_sum_slice", p, k, num) == ar.AR_ERR_SLICE
        assert ar.call_slice("ar_residual_rmsnorm_slice", fused_params(), k, num) == ar.AR_ERR_SLICE
    # the full params are validated first
    assert ar.call_slice("ar_sum_slice", sum_params(ranks=9, inputs=[A] * 8), 0, 2) == ar.AR_ERR_RANKS
    assert ar.call_slice("ar_residual_rmsnorm_slice", fused_params(hidden=0), 0, 2) == ar.AR_ERR_SHAPE
    assert ar.ar_slice_range(p, 7, 0, 2)[0] == ar.AR_ERR_SHAPE


def test_empty_slice_is_a_noop_without_any_hip_call():
    # 10 bf16 elements in 8 slices: the share rounds up to one 16-byte pack (8
    # elements), so slice 0 is [0, 8), slice 1 is [8, 10) and slices 2..7 are empty
    p = sum_params(n=10, dtype=ar.AR_BF16)
    assert ar.ar_slice_range(p, ar.AR_FUSION_NONE, 5, 8)[1:] == (10, 10)
    assert ar.call_slice("ar_sum_slice", p, 5, 8) == ar.AR_OK
    assert ar.call_slice("ar_residual_rmsnorm_slice", fused_params(n=2 * 1024, hidden=1024), 5, 8) == ar.AR_OK


def test_rmsnorm_entry_needs_one_input():
    assert ar.call("ar_rmsnorm", fused_params(ranks=2)) == ar.AR_ERR_RANKS
    assert ar.call("ar_rmsnorm", fused_params(ranks=1, hidden=0)) == ar.AR_ERR_SHAPE
    assert ar.load().ar_rmsnorm(None, None) == ar.AR_ERR_NULL


def test_allocate_workspace_rejects_what_the_layout_rejects():
    """The allocator asks ar_partials_layout first, so a bad rank count or a
    size that does not fit fails before any device allocation."""
    import torch
    with pytest.raises(ar.ArError, match="AR_ERR_RANKS"):
        ar.allocate_workspace(100, torch.float16, 9)
    with pytest.raises(ar.ArError, match="AR_ERR_SHAPE"):
        ar.allocate_workspace((1 << 62) + 1, torch.float32, 8)
    with pytest.raises(TypeError):
        ar.allocate_workspace(100, torch.int32, 2)
