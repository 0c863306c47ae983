"""GPU parity for the unfused baseline and the two-shot split on one GPU.

Unfused path ("allreduce.d2", the branch that runs the all-reduce first and
rms_norm_kernel after it): ar_sum writes the rounded sum X, then ar_rmsnorm
adds bias and residual to X and normalizes. Its oracle is the same
composition of oracle calls. Without bias and residual it equals the fused op
bit for bit.

Two-shot split ("allreduce.d2" twoShotAllReduceKernel; "type.d2"
elts_per_rank): each slice call computes one rank's share in place in the full
output; all slices together must equal the oracle's full result, and one
slice must write exactly its range.

Partials layout (ar_partials_layout, the one-GPU counterpart of the comm-buffer
workspace of "allreduce.d2" CustomAllReduceHelper): partials placed in one
allocation at the recommended staggered slots give the oracle's results.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_ar_amd as ar
from tensor_all_reduce_ar_amd import inputs

from gpu_util import (Guarded, assert_bitexact, assert_output_close, bits, dev, empty_host, host_bits, note, slab)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DTYPES = ("fp32", "fp16", "bf16")


def oracle_sum(w):
    ref = empty_host(w.n, w.dtype)
    oracle.ar_sum(w.dtype, w.partials, ref)
    return ref


def oracle_fused(w, parts=None):
    out, inter = empty_host(w.n, w.dtype), empty_host(w.n, w.dtype)
    oracle.ar_residual_rmsnorm(w.dtype, parts if parts is not None else w.partials, w.hidden, w.weight, w.eps,
                               out, inter, bias=w.bias, residual=w.residual)
    return bits(out), bits(inter)


# -------------------------------------------------------- unfused baseline
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", [1, 2, 8])
def test_unfused_path_matches_the_oracle_composition(dtype, ranks):
    note(f"[next] unfused {dtype} R={ranks}")
    w = inputs.random_fused(dtype, ranks, 12, 2048, 900 + ranks)
    parts = [dev(p, dtype) for p in w.partials]
    x = torch.empty_like(parts[0])
    ar.ar_sum(parts, x)
    out, inter = Guarded(w.n, dtype), Guarded(w.n, dtype)
    ar.ar_rmsnorm(x, dev(w.weight, dtype), w.eps, out.t, inter.t, bias=dev(w.bias, dtype),
                  residual=dev(w.residual, dtype))
    torch.cuda.synchronize()
    out.check_guards()
    inter.check_guards()
    xs = oracle_sum(w)
    assert_bitexact(host_bits(x), bits(xs), dtype, "unfused sum")
    ref_out, ref_inter = oracle_fused(w, parts=[xs])
    assert_bitexact(host_bits(inter.t), ref_inter, dtype, "unfused intermediate")
    assert_output_close(host_bits(out.t), ref_out, dtype, "unfused output")


@pytest.mark.parametrize("dtype", DTYPES)
def test_unfused_equals_fused_without_bias_and_residual(dtype):
    w = inputs.random_fused(dtype, 4, 9, 4096, 950, bias=False, residual=False)
    parts = [dev(p, dtype) for p in w.partials]
    weight = dev(w.weight, dtype)
    x = torch.empty_like(parts[0])
    ar.ar_sum(parts, x)
    out_u, inter_u = torch.empty_like(x), torch.empty_like(x)
    ar.ar_rmsnorm(x, weight, w.eps, out_u, inter_u)
    out_f, inter_f = torch.empty_like(x), torch.empty_like(x)
    ar.ar_residual_rmsnorm(parts, weight, w.eps, out_f, inter_f)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(inter_u), host_bits(inter_f))
    assert np.array_equal(host_bits(out_u), host_bits(out_f))


# ---------------------------------------------------------- two-shot split
def _slices(p_fn, fusion_op, num):
    return [ar.ar_slice_range(p_fn(), fusion_op, k, num)[1:] for k in range(num)]


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("num", [2, 3, 4, 8])
def test_sum_slices_compose_to_the_full_sum(dtype, num):
    for n in (1, 100, 100003):
        note(f"[next] sum slices {dtype} n={n} S={num}")
        w = inputs.random_sum(dtype, 4, n, 1200 + num)
        parts = [dev(p, dtype) for p in w.partials]
        out = Guarded(n, dtype)
        for k in range(num):
            ar.ar_sum_slice(parts, out.t, k, num)
        torch.cuda.synchronize()
        out.check_guards()
        assert_bitexact(host_bits(out.t), bits(oracle_sum(w)), dtype, f"sum slices n={n} S={num}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_one_sum_slice_writes_exactly_its_range(dtype):
    n, num = 50000, 8
    w = inputs.random_sum(dtype, 3, n, 1300)
    parts = [dev(p, dtype) for p in w.partials]
    ref = bits(oracle_sum(w))
    for k in (0, 3, 7):
        out = Guarded(n, dtype)
        before = host_bits(out.t)
        ar.ar_sum_slice(parts, out.t, k, num)
        torch.cuda.synchronize()
        out.check_guards()
        params = ar.make_params(n, 3, {"fp32": 0, "fp16": 1, "bf16": 2}[dtype], [p.data_ptr() for p in parts],
                                out.t.data_ptr())
        st, b, e = ar.ar_slice_range(params, ar.AR_FUSION_NONE, k, num)
        assert st == 0 and e > b
        got = host_bits(out.t)
        assert_bitexact(got[b:e], ref[b:e], dtype, f"slice {k}")
        assert np.array_equal(got[:b], before[:b]) and np.array_equal(got[e:], before[e:])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("num", [2, 8])
def test_fused_slices_compose_to_the_full_op(dtype, num):
    w = inputs.random_fused(dtype, 4, 33, 1024, 1400 + num)
    parts = [dev(p, dtype) for p in w.partials]
    weight, bias, res = dev(w.weight, dtype), dev(w.bias, dtype), dev(w.residual, dtype)
    out, inter = Guarded(w.n, dtype), Guarded(w.n, dtype)
    for k in range(num):
        ar.ar_residual_rmsnorm_slice(parts, weight, w.eps, out.t, inter.t, k, num, bias=bias, residual=res)
    full_out, full_inter = torch.empty_like(parts[0]), torch.empty_like(parts[0])
    ar.ar_residual_rmsnorm(parts, weight, w.eps, full_out, full_inter, bias=bias, residual=res)
    torch.cuda.synchronize()
    out.check_guards()
    inter.check_guards()
    ref_out, ref_inter = oracle_fused(w)
    assert_bitexact(host_bits(inter.t), ref_inter, dtype, "fused slices intermediate")
    assert_output_close(host_bits(out.t), ref_out, dtype, "fused slices output")
    # each row runs the same code either way: bit-identical to the unsliced call
    assert np.array_equal(host_bits(out.t), host_bits(full_out))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("num", [2, 4])
def test_fused_slices_of_wide_rows(dtype, num):
    """Slices of rows wider than 4096 packs (the chunked path: every row cut
    into the same chunks whatever the slice) compose to the unsliced call
    bit for bit, and match the oracle."""
    hidden = 16388 * (1 if dtype == "fp32" else 2) * 2
    w = inputs.random_fused(dtype, 3, 9, hidden, 1450 + num)
    parts = [dev(p, dtype) for p in w.partials]
    weight, bias, res = dev(w.weight, dtype), dev(w.bias, dtype), dev(w.residual, dtype)
    out, inter = Guarded(w.n, dtype), Guarded(w.n, dtype)
    for k in range(num):
        ar.ar_residual_rmsnorm_slice(parts, weight, w.eps, out.t, inter.t, k, num, bias=bias, residual=res)
    full_out, full_inter = torch.empty_like(parts[0]), torch.empty_like(parts[0])
    ar.ar_residual_rmsnorm(parts, weight, w.eps, full_out, full_inter, bias=bias, residual=res)
    torch.cuda.synchronize()
    out.check_guards()
    inter.check_guards()
    ref_out, ref_inter = oracle_fused(w)
    assert_bitexact(host_bits(inter.t), ref_inter, dtype, "wide-row slices intermediate")
    assert_output_close(host_bits(out.t), ref_out, dtype, "wide-row slices output")
    assert np.array_equal(host_bits(out.t), host_bits(full_out))


@pytest.mark.parametrize("dtype", DTYPES)
def test_prepared_slices_match_the_plain_slices(dtype):
    """Prepared slice calls (one per slice, on the current stream and on a
    side stream) write bitwise what the plain slice calls write, and the
    slices of both ops compose to the oracle's full results."""
    num = 4
    ws = inputs.random_sum(dtype, 3, 70001, 1450)
    wf = inputs.random_fused(dtype, 4, 37, 2048, 1460)
    sp = [dev(p, dtype) for p in ws.partials]
    fp = [dev(p, dtype) for p in wf.partials]
    weight, bias, res = dev(wf.weight, dtype), dev(wf.bias, dtype), dev(wf.residual, dtype)
    s_out = Guarded(ws.n, dtype)
    f_out, f_inter = Guarded(wf.n, dtype), Guarded(wf.n, dtype)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for k in range(num):
        cs = ar.prepare_sum_slice(sp, s_out.t, k, num)
        cf = ar.prepare_residual_rmsnorm_slice(fp, weight, wf.eps, f_out.t, f_inter.t, k, num, bias=bias,
                                               residual=res)
        if k % 2:
            cs(side)
            cf(side)
        else:
            cs()
            cf()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for g in (s_out, f_out, f_inter):
        g.check_guards()
    assert_bitexact(host_bits(s_out.t), bits(oracle_sum(ws)), dtype, "prepared sum slices")
    ref_out, ref_inter = oracle_fused(wf)
    assert_bitexact(host_bits(f_inter.t), ref_inter, dtype, "prepared fused slices intermediate")
    assert_output_close(host_bits(f_out.t), ref_out, dtype, "prepared fused slices output")
    p_out, p_inter = torch.empty_like(fp[0]), torch.empty_like(fp[0])
    for k in range(num):
        ar.ar_residual_rmsnorm_slice(fp, weight, wf.eps, p_out, p_inter, k, num, bias=bias, residual=res)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(f_out.t), host_bits(p_out)) and np.array_equal(host_bits(f_inter.t),
                                                                                     host_bits(p_inter))
    with pytest.raises(ar.ArError, match="AR_ERR_SLICE"):
        ar.prepare_sum_slice(sp, s_out.t, num, num)()


def test_two_shot_split_at_the_large_shapes():
    """Eight slices of the large fused workload and four of the large sum
    compose to the oracle's full results."""
    w = inputs.make(inputs.FUSED_BF16_R8_2048x8192)
    parts = [dev(p, w.dtype) for p in w.partials]
    weight, res = dev(w.weight, w.dtype), dev(w.residual, w.dtype)
    out, inter = torch.empty_like(parts[0]), torch.empty_like(parts[0])
    for k in range(8):
        ar.ar_residual_rmsnorm_slice(parts, weight, w.eps, out, inter, k, 8, residual=res)
    torch.cuda.synchronize()
    ref_out, ref_inter = oracle_fused(w)
    assert_bitexact(host_bits(inter), ref_inter, w.dtype, "large fused, 8 slices, intermediate")
    assert_output_close(host_bits(out), ref_out, w.dtype, "large fused, 8 slices, output")
    del parts, out, inter
    s = inputs.make(inputs.SUM_BF16_R4_8192x8192)
    sp = [dev(p, s.dtype) for p in s.partials]
    so = torch.empty_like(sp[0])
    for k in range(4):
        ar.ar_sum_slice(sp, so, k, 4)
    torch.cuda.synchronize()
    assert_bitexact(host_bits(so), bits(oracle_sum(s)), s.dtype, "large sum, 4 slices")


# ------------------------------------------------------- partials layout
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", [1, 2, 8])
def test_ops_on_partials_in_the_recommended_layout(dtype, ranks):
    note(f"[next] slab layout {dtype} R={ranks}")
    w = inputs.random_fused(dtype, ranks, 37, 4096, 1600 + ranks)
    base, parts = slab(w.partials, dtype)
    out, inter = Guarded(w.n, dtype), Guarded(w.n, dtype)
    ar.ar_residual_rmsnorm(parts, dev(w.weight, dtype), w.eps, out.t, inter.t, bias=dev(w.bias, dtype),
                           residual=dev(w.residual, dtype))
    s_out = Guarded(w.n, dtype)
    ar.ar_sum(parts, s_out.t)
    torch.cuda.synchronize()
    for g in (out, inter, s_out):
        g.check_guards()
    ref_out, ref_inter = oracle_fused(w)
    assert_bitexact(host_bits(inter.t), ref_inter, dtype, "slab layout intermediate")
    assert_output_close(host_bits(out.t), ref_out, dtype, "slab layout output")
    assert_bitexact(host_bits(s_out.t), bits(oracle_sum(w)), dtype, "slab layout sum")
    del base


def test_large_fused_workload_in_the_recommended_layout():
    w = inputs.make(inputs.FUSED_BF16_R8_2048x8192)
    base, parts = slab(w.partials, w.dtype)
    out, inter = torch.empty_like(parts[0]), torch.empty_like(parts[0])
    ar.ar_residual_rmsnorm(parts, dev(w.weight, w.dtype), w.eps, out, inter, residual=dev(w.residual, w.dtype))
    torch.cuda.synchronize()
    ref_out, ref_inter = oracle_fused(w)
    assert_bitexact(host_bits(inter), ref_inter, w.dtype, "large fused, slab layout, intermediate")
    assert_output_close(host_bits(out), ref_out, w.dtype, "large fused, slab layout, output")
    del base


@pytest.mark.parametrize("dtype", DTYPES)
def test_allocate_workspace_places_partials_at_the_layout_slots(dtype):
    """ar.allocate_workspace (the one-GPU counterpart of "allreduce.d2"
    CustomAllReduceHelper.allocate_workspace): one allocation, R typed views at
    exactly the byte offsets ar_partials_layout reports, 256-byte aligned and
    disjoint; writing the partials into the views and running both ops on them
    gives the oracle's results."""
    ranks, rows, hidden = 4, 33, 2560
    note(f"[next] allocate_workspace {dtype} R={ranks}")
    w = inputs.random_fused(dtype, ranks, rows, hidden, 1700)
    code = {"fp32": ar.AR_FP32, "fp16": ar.AR_FP16, "bf16": ar.AR_BF16}[dtype]
    st, offs, total = ar.ar_partials_layout(w.n, code, ranks)
    ws = ar.allocate_workspace(w.n, {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype],
                               ranks)
    assert st == ar.AR_OK and ws.offsets == offs and ws.total_bytes == total == ws.buffer.numel()
    base = ws.buffer.data_ptr()
    for r, v in enumerate(ws.partials):
        assert v.is_contiguous() and v.numel() == w.n and v.data_ptr() - base == offs[r]
        assert v.data_ptr() % 256 == 0
        v.copy_(dev(w.partials[r], dtype))
    out, inter, s_out = Guarded(w.n, dtype), Guarded(w.n, dtype), Guarded(w.n, dtype)
    ar.ar_residual_rmsnorm(ws.partials, dev(w.weight, dtype), w.eps, out.t, inter.t, bias=dev(w.bias, dtype),
                           residual=dev(w.residual, dtype))
    ar.ar_sum(ws.partials, s_out.t)
    torch.cuda.synchronize()
    for g in (out, inter, s_out):
        g.check_guards()
    ref_out, ref_inter = oracle_fused(w)
    assert_bitexact(host_bits(inter.t), ref_inter, dtype, "workspace intermediate")
    assert_output_close(host_bits(out.t), ref_out, dtype, "workspace output")
    assert_bitexact(host_bits(s_out.t), bits(oracle_sum(w)), dtype, "workspace sum")
    # the slots were not disturbed by the calls (inputs are read only)
    for r, v in enumerate(ws.partials):
        assert_bitexact(host_bits(v), bits(w.partials[r]), dtype, f"workspace slot {r} after the calls")
