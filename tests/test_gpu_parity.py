"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on
the same seeded inputs.

Rules: sums and the pre-norm sum S are compared bit for bit (same fp32 adds
in the same rank order, one rounding); the normed output is within 1e-5
relative for fp32 and within 2 ulp for fp16/bf16. Every output buffer has
canary guard bands that must come back untouched.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_ar_amd as ar
from tensor_all_reduce_ar_amd import inputs
from tensor_all_reduce_ar_amd.ar import call, make_params

from gpu_util import (TORCH_DT, Guarded, assert_bitexact, assert_output_close, bits, dev, empty_host, host_bits,
                      max_ulp, note)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

DTYPES = ("fp32", "fp16", "bf16")
CODE = {"fp32": ar.AR_FP32, "fp16": ar.AR_FP16, "bf16": ar.AR_BF16}


def run_sum(w: inputs.Workload, offsets=None, out_offset=0):
    """Run ar_sum on the workload; partial r may start `offsets[r]` elements
    into its device buffer (to make pointers unaligned)."""
    offsets = offsets or [0] * w.ranks
    bufs = []
    for p, off in zip(w.partials, offsets):
        t = torch.empty(w.n + off, dtype=TORCH_DT[w.dtype], device="cuda")
        t[off:].copy_(dev(p, w.dtype))
        bufs.append(t[off:])
    out = Guarded(w.n, w.dtype, out_offset)
    ar.ar_sum(bufs, out.t)
    torch.cuda.synchronize()
    out.check_guards()
    return host_bits(out.t)


def ref_sum(w: inputs.Workload):
    ref = empty_host(w.n, w.dtype)
    oracle.ar_sum(w.dtype, w.partials, ref)
    return bits(ref)


def run_fused(w: inputs.Workload, stream=None):
    parts = [dev(p, w.dtype) for p in w.partials]
    out, inter = Guarded(w.n, w.dtype), Guarded(w.n, w.dtype)
    ar.ar_residual_rmsnorm(parts, dev(w.weight, w.dtype), w.eps, out.t, inter.t,
                           bias=dev(w.bias, w.dtype) if w.bias is not None else None,
                           residual=dev(w.residual, w.dtype) if w.residual is not None else None,
                           hidden_size=w.hidden, stream=stream)
    torch.cuda.synchronize()
    out.check_guards()
    inter.check_guards()
    return host_bits(out.t), host_bits(inter.t)


def ref_fused(w: inputs.Workload):
    out, inter = empty_host(w.n, w.dtype), empty_host(w.n, w.dtype)
    oracle.ar_residual_rmsnorm(w.dtype, w.partials, w.hidden, w.weight, w.eps, out, inter, bias=w.bias,
                               residual=w.residual)
    return bits(out), bits(inter)


def check_fused(w, got_out, got_inter):
    ref_out, ref_inter = ref_fused(w)
    assert_bitexact(got_inter, ref_inter, w.dtype, f"{w.name} intermediate")
    assert_output_close(got_out, ref_out, w.dtype, f"{w.name} output")
    return ref_out


# ---------------------------------------------------- the named workloads
@pytest.mark.parametrize("name", inputs.workload_names())
def test_named_workload_matches_oracle(name):
    note(f"[parity] workload {name}")
    w = inputs.make(name)
    if w.op == "sum":
        assert_bitexact(run_sum(w), ref_sum(w), w.dtype, name)
    else:
        got_out, got_inter = run_fused(w)
        ref_out = check_fused(w, got_out, got_inter)
        if w.dtype != "fp32":
            note(f"[parity] {name}: output max {max_ulp(got_out, ref_out, w.dtype)} ulp from the oracle")


def test_golden_small_workloads():
    """The small workloads also match the oracle's stored digests."""
    import hashlib
    import json
    import os
    with open(os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")) as f:
        gold = json.load(f)
    w = inputs.make(inputs.SUM_FP32_R2_4x256)
    got = run_sum(w)
    assert hashlib.sha256(got.tobytes()).hexdigest() == gold["workloads"][w.name]["out_sha256"]
    for name in (inputs.FUSED_FP16_R8_16x4096, inputs.fused_fp16_r2_5120_name(7)):
        w = inputs.make(name)
        _, inter = run_fused(w)
        assert hashlib.sha256(inter.tobytes()).hexdigest() == gold["workloads"][name]["intermediate_sha256"]


# ------------------------------------------------------------------ sums
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", range(1, 9))
def test_sum_sizes_and_tails(dtype, ranks):
    for n in (1, 7, 8, 9, 15, 16, 17, 1027, 2 * 256 * 8 + 5, 70001, 1_000_003):
        note(f"[parity] sum {dtype} R={ranks} n={n}")
        w = inputs.random_sum(dtype, ranks, n, 1000 + 10 * ranks + n % 97)
        assert_bitexact(run_sum(w), ref_sum(w), dtype, f"sum {dtype} R={ranks} n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", [2, 6])
def test_sum_sizes_at_the_shape_switch(dtype, ranks):
    """Calls below CUs x 1024 packs take 256-lane x 1-pack steps, larger ones
    1024-pack steps (512 x 2 up to 5 ranks, 256 x 4 from 6); either way the
    packs after the last full step and the tail elements form a unit of their
    own. Sizes just below and above the switch, with and without a remainder
    and a tail, against the oracle."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    v = 4 if dtype == "fp32" else 8
    switch = cus * 1024  # packs
    for npacks, tail in ((switch - 1, 0), (switch - 1, v - 1), (switch, 0), (switch, 3), (switch + 77, 5),
                         (switch + 1023, v - 1), (2 * switch + 1024, 0)):
        n = npacks * v + tail
        note(f"[parity] sum {dtype} R={ranks} n={n} (switch at {switch} packs)")
        w = inputs.random_sum(dtype, ranks, n, 2000 + ranks + npacks % 101 + tail)
        assert_bitexact(run_sum(w), ref_sum(w), dtype, f"sum {dtype} R={ranks} n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_unaligned_pointers(dtype):
    """Element-aligned but not 16-byte aligned buffers take the element-wise kernel."""
    for offs, oo in (([1, 0, 0], 0), ([0, 0, 0], 1), ([3, 1, 2], 3)):
        note(f"[parity] sum unaligned {dtype} offsets={offs} out={oo}")
        w = inputs.random_sum(dtype, 3, 4099, 77)
        assert_bitexact(run_sum(w, offs, oo), ref_sum(w), dtype, f"unaligned {offs}/{oo}")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("byte_offset", [2, 4, 8])
def test_sum_pointer_byte_offsets(dtype, byte_offset):
    """Every buffer (partials and output) shifted by the same byte offset, for
    the offsets that keep element alignment, over sizes with and without a
    tail."""
    size = 4 if dtype == "fp32" else 2
    if byte_offset % size:
        pytest.skip("offset breaks element alignment (rejected with AR_ERR_ALIGN)")
    k = byte_offset // size
    for ranks in (2, 5, 8):
        for n in (16, 1027, 100003):
            note(f"[parity] sum {dtype} R={ranks} n={n} byte offset {byte_offset}")
            w = inputs.random_sum(dtype, ranks, n, 1500 + ranks + n % 89)
            assert_bitexact(run_sum(w, [k] * ranks, k), ref_sum(w), dtype, f"offset {byte_offset} B R={ranks} n={n}")


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_in_place(dtype):
    w = inputs.random_sum(dtype, 4, 100003, 5)
    parts = [dev(p, dtype) for p in w.partials]
    ar.ar_sum(parts, parts[2])  # output is partial 2
    torch.cuda.synchronize()
    assert_bitexact(host_bits(parts[2]), ref_sum(w), dtype, "in place")
    one = dev(w.partials[0], dtype)
    ar.ar_sum([one], one)  # one rank, in place: nothing to do
    torch.cuda.synchronize()
    assert_bitexact(host_bits(one), bits(w.partials[0]), dtype, "passthrough in place")


def test_sum_special_values_fp32():
    s = 2.0 ** -149
    p0 = np.array([np.inf, np.inf, np.nan, 1.0, -0.0, -0.0, s, 3 * s, 1.0, 2.0 ** -24] * 7, np.float32)
    p1 = np.array([-np.inf, 1.0, 1.0, np.nan, -0.0, 0.0, s, -s, 2.0 ** -24, 2.0 ** -24] * 7, np.float32)
    p2 = np.array([0.0, 0.0, 0.0, 0.0, -0.0, -0.0, s, 0.0, 2.0 ** -24, 1.0] * 7, np.float32)
    w = inputs.Workload("special", "sum", "fp32", 3, p0.size, p0.size, [p0, p1, p2])
    assert_bitexact(run_sum(w), ref_sum(w), "fp32", "special values")
    assert_bitexact(run_sum(w, [1, 2, 3]), ref_sum(w), "fp32", "special values, element path")


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_sum_rounding_edges(dtype):
    """Overflow to Inf (fp16: 65504 + 16), ties to even, and values the
    one-rounding rule decides, through both kernels."""
    big = 65504.0 if dtype == "fp16" else 3.3895314e38
    vals0 = [big, big, 1.0, 1.0, -1.0, 1.0, 0.5, -0.0] * 5
    vals1 = [16.0, 15.0, 2.0 ** -11, 3 * 2.0 ** -11, -2.0 ** -8, 2.0 ** -9, 2.0 ** -12, -0.0] * 5
    if dtype == "bf16":
        vals1[:2] = [big / 2, 2.0 ** 100] * 1
    p0 = inputs.to_dtype(np.array(vals0, np.float32), dtype)
    p1 = inputs.to_dtype(np.array(vals1, np.float32), dtype)
    p2 = inputs.to_dtype(np.array([0.0, 0.0, 0.0, 0.0, 0.0, 2.0 ** -9, 0.0, -0.0] * 5, np.float32), dtype)
    w = inputs.Workload("edges", "sum", dtype, 3, p0.size, p0.size, [p0, p1, p2])
    assert_bitexact(run_sum(w), ref_sum(w), dtype, "edges vector")
    assert_bitexact(run_sum(w, [1, 0, 0]), ref_sum(w), dtype, "edges element")


def test_sum_deterministic_and_on_a_side_stream():
    """100 calls on a side stream, each into a fresh output: the first matches
    the oracle and every other one is bitwise the first."""
    w = inputs.random_sum("bf16", 4, 1 << 20, 9)
    parts = [dev(p, "bf16") for p in w.partials]
    s = torch.cuda.Stream()
    outs = []
    with torch.cuda.stream(s):
        for _ in range(100):
            o = torch.empty_like(parts[0])
            ar.ar_sum(parts, o, stream=s)
            outs.append(o)
    s.synchronize()
    first = host_bits(outs[0])
    assert_bitexact(first, ref_sum(w), "bf16", "side stream")
    ref = outs[0].view(torch.int16)
    for k, o in enumerate(outs[1:], 1):
        assert torch.equal(o.view(torch.int16), ref), f"call {k} differs from the first"


# ------------------------------------------------------------ fused op
@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [8, 64, 520, 4096, 4100, 5120, 8192, 10240, 12288, 14336, 16384, 20480, 65536])
def test_fused_widths(dtype, hidden):
    """Few rows: the register-row kernel in its latency layout (one pack per
    lane up to 1024 packs a row, two up to 2048), the 512-lane register path
    for rows of 2049..4096 packs (16-bit types, and fp32 at these two ranks),
    the chunked path past 4096 packs, and the element kernel for rows whose
    byte size is not a multiple of 16 (4100 fp16/bf16)."""
    for rows in (1, 7, 33, 64):
        if rows * hidden > 1 << 21:
            continue
        note(f"[parity] fused {dtype} H={hidden} rows={rows}")
        w = inputs.random_fused(dtype, 2, rows, hidden, 300 + rows)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [8, 64, 512, 1000, 1024, 2000, 2048, 2560, 3072, 3584, 4096, 4100, 5120, 6144,
                                    6500, 7168, 8192, 8200, 9216, 10240, 12288, 13312, 14336, 16376, 16384,
                                    16392, 18432, 20480, 24576, 28672, 32760, 32768, 32776])
def test_fused_widths_at_the_layout_switch(dtype, hidden):
    """Up to one row per CU the register-row kernel takes its latency layout
    (up to 1024 lanes a row). With more rows: one wave per row for rows of 128
    and 256 packs (8 or 4 rows per workgroup; the last group may be short),
    the multi-row kernel for rows of 512 packs (2 rows per iteration),
    64 or 128 lanes in the pipelined full-row variant for rows of 320, 384 and
    640 packs, 256 lanes with 4..8 packs in the same variant for rows of 1024,
    1280, 1536, 1792 and 2048 packs, and in its ragged form (last slot partly
    covered, down to one lane: 1025 and 2047 packs) for the other rows of
    1025..2047 packs, 512 lanes with 5..8 packs (full or ragged) for rows of
    2049..4096 packs in 16-bit types, up to 512 lanes with 1..8 packs per
    lane for the rest, and past that the two-pass kernel (fp32 rows of
    2049..4096 packs at the 8 ranks used here) or the chunked path (rows of
    more than 4096 packs). The row count at the switch and one past it."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for rows in (cus, cus + 1):
        note(f"[parity] fused {dtype} H={hidden} rows={rows} (CUs {cus})")
        w = inputs.random_fused(dtype, 8 if hidden >= 8192 else 3, rows, hidden, 350 + rows % 7)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [4096, 8192, 9216, 16384, 20480])
def test_fused_rows_at_the_latency_switch(dtype, hidden):
    """Rows of 1024..2048 packs leave the latency layout once they exceed three
    quarters of the CUs: the row counts on both sides of that switch (and
    for 16-bit rows past 2048 packs, which take the 512-lane register path at
    any row count, the same counts)."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for rows in (cus * 3 // 4, cus * 3 // 4 + 1):
        note(f"[parity] fused {dtype} H={hidden} rows={rows} (CUs {cus})")
        w = inputs.random_fused(dtype, 8, rows, hidden, 380 + rows % 5)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("ranks", [1, 2, 3, 7, 8])
@pytest.mark.parametrize("hidden", [8196, 8200, 9216, 10240, 10244, 12288, 14336, 16376, 16384])
def test_fp32_rows_of_2049_to_4096_packs(ranks, hidden):
    """fp32 rows of 2049..4096 packs: the 512-lane register path wherever its
    instance fits in registers - every row up to 2 ranks (5..8 packs per lane,
    full, or ragged down to one lane in the last slot at 8196), and rows of
    up to 2560 packs at more ranks (at 8 ranks only the full 10240) - and the
    two-pass wide kernel for the rest (10244 and wider from 3 ranks, the
    ragged 8-rank rows); a few rows and more rows than CUs, then the same call
    with the intermediate written over the residual and the output over the
    last partial."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for rows in (3, cus + 1):
        note(f"[parity] fused fp32 R={ranks} H={hidden} rows={rows}")
        w = inputs.random_fused("fp32", ranks, rows, hidden, 730 + rows % 7 + ranks)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)
    ref_out, ref_inter = ref_fused(w)
    parts = [dev(p, "fp32") for p in w.partials]
    res = dev(w.residual, "fp32")
    ar.ar_residual_rmsnorm(parts, dev(w.weight, "fp32"), w.eps, parts[-1], res, bias=dev(w.bias, "fp32"),
                           residual=res)
    torch.cuda.synchronize()
    assert_bitexact(host_bits(res), ref_inter, "fp32", "intermediate in place of the residual")
    assert_output_close(host_bits(parts[-1]), ref_out, "fp32", "output in place of the last partial")


CHUNKED_CASES = [("bf16", 8, 32776), ("fp16", 2, 65536), ("bf16", 3, 131072), ("fp16", 1, 40968),
                 ("fp32", 8, 16388), ("fp32", 2, 32768), ("fp32", 3, 20488), ("fp32", 6, 16392)]


@pytest.mark.parametrize("dtype,ranks,hidden", CHUNKED_CASES)
def test_fused_wide_rows_chunked(dtype, ranks, hidden):
    """Rows of more than 4096 packs: one workgroup per chunk of 1024 packs
    over three launches, the chunks' sums of squares passed through the head
    words of the output. Widths with a short last chunk (4097, 4098, 5121 and
    5122 packs) and 8 and 16 whole chunks, in every type; 1, 7, half the CUs
    and a few more than the CUs rows."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for rows in (1, 7, cus // 2, cus + 3):
        if rows * hidden > 12 << 20:
            continue
        note(f"[parity] fused chunked {dtype} R={ranks} H={hidden} rows={rows} (CUs {cus})")
        w = inputs.random_fused(dtype, ranks, rows, hidden, 760 + rows % 11 + ranks)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


def test_fused_wide_rows_chunked_aliasing_and_repeat():
    """The chunked path with the output written over a partial (whose head
    words then carry the sums of squares between the launches) and the
    intermediate over the residual; then two plain calls, bitwise equal."""
    for dtype, ranks, rows, hidden in (("bf16", 4, 9, 65536), ("fp32", 3, 5, 16392)):
        note(f"[parity] fused chunked aliasing {dtype} R={ranks} H={hidden} rows={rows}")
        w = inputs.random_fused(dtype, ranks, rows, hidden, 790)
        ref_out, ref_inter = ref_fused(w)
        parts = [dev(p, dtype) for p in w.partials]
        res = dev(w.residual, dtype)
        ar.ar_residual_rmsnorm(parts, dev(w.weight, dtype), w.eps, parts[1], res, bias=dev(w.bias, dtype),
                               residual=res)
        torch.cuda.synchronize()
        assert_bitexact(host_bits(res), ref_inter, dtype, "intermediate in place of the residual")
        assert_output_close(host_bits(parts[1]), ref_out, dtype, "output in place of partial 1")
        a, b = run_fused(w), run_fused(w)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), "repeat calls differ"


def test_fused_wide_rows_chunked_from_a_graph():
    """A chunked call (three launches) captured into a HIP graph and replayed
    three times, outputs filled with NaN before each replay and new partials
    copied in before the last: every replay matches the oracle."""
    note("[parity] fused chunked graph replay")
    ws = [inputs.random_fused("bf16", 8, 6, 65536, 800 + k) for k in range(2)]
    parts = [dev(p, "bf16") for p in ws[0].partials]
    wt, b, q = dev(ws[0].weight, "bf16"), dev(ws[0].bias, "bf16"), dev(ws[0].residual, "bf16")
    out, inter = torch.empty_like(parts[0]), torch.empty_like(parts[0])
    call = ar.prepare_residual_rmsnorm(parts, wt, ws[0].eps, out, inter, bias=b, residual=q)
    call()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        k = 1 if rep == 2 else 0
        if rep == 2:
            for t, p in zip(parts, ws[1].partials):
                t.copy_(dev(p, "bf16"))
        out.fill_(float("nan"))
        inter.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        w = inputs.Workload("graph-chunked", "fused", "bf16", 8, ws[k].n, ws[k].hidden, ws[k].partials,
                            ws[0].bias, ws[0].residual, ws[0].weight, ws[0].eps)
        check_fused(w, host_bits(out), host_bits(inter))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", range(1, 9))
def test_fused_ranks(dtype, ranks):
    note(f"[parity] fused {dtype} R={ranks}")
    w = inputs.random_fused(dtype, ranks, 9, 2048, 500 + ranks)
    got_out, got_inter = run_fused(w)
    check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("bias,residual", [(False, False), (True, False), (False, True)])
def test_fused_optional_terms(dtype, bias, residual):
    for hidden in (1024, 4100):
        note(f"[parity] fused {dtype} bias={bias} residual={residual} H={hidden}")
        w = inputs.random_fused(dtype, 3, 5, hidden, 600, bias=bias, residual=residual)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("bias,residual", [(False, False), (True, False), (False, True)])
def test_fused_optional_terms_in_the_throughput_layouts(dtype, bias, residual):
    """More rows than CUs, so every register-row layout runs: the wave-per-row
    kernel (1024), the multi-row kernel (4096), the pipelined variant full on
    128 and 256 lanes (5120, 8192) and ragged on 256 lanes (9216), the
    512-lane register path in 16-bit types, ragged (18440), and the plain
    slots (6144) - each without bias, without residual, or without both."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for hidden in (1024, 4096, 5120, 6144, 8192, 9216, 18440):
        note(f"[parity] fused {dtype} bias={bias} residual={residual} H={hidden} rows={cus + 2}")
        w = inputs.random_fused(dtype, 3, cus + 2, hidden, 610, bias=bias, residual=residual)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("ranks", range(1, 9))
def test_fused_ranks_in_the_pipelined_layouts(ranks):
    """Every rank count through the pipelined slot walks: full on 256 lanes
    (8192), ragged on 256 lanes (9216), and on 512 lanes full and ragged
    (20480, 20488), bf16, more rows than CUs."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    for hidden in (8192, 9216, 20480, 20488):
        note(f"[parity] fused bf16 R={ranks} H={hidden} rows={cus + 1}")
        w = inputs.random_fused("bf16", ranks, cus + 1, hidden, 650 + ranks)
        got_out, got_inter = run_fused(w)
        check_fused(w, got_out, got_inter)


@pytest.mark.parametrize("dtype", DTYPES)
def test_fused_aliasing(dtype):
    """intermediate == residual (S replaces the residual in place), and
    output == a partial."""
    w = inputs.random_fused(dtype, 4, 6, 4096, 700)
    ref_out, ref_inter = ref_fused(w)
    parts = [dev(p, dtype) for p in w.partials]
    res = dev(w.residual, dtype)
    ar.ar_residual_rmsnorm(parts, dev(w.weight, dtype), w.eps, parts[1], res, bias=dev(w.bias, dtype),
                           residual=res)
    torch.cuda.synchronize()
    assert_bitexact(host_bits(res), ref_inter, dtype, "intermediate in place of the residual")
    assert_output_close(host_bits(parts[1]), ref_out, dtype, "output in place of partial 1")


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("hidden", [512, 1024, 2048, 2560, 3072, 4096, 5120, 8192, 9216, 10240, 16384, 18432,
                                    32768])
def test_fused_aliasing_in_the_throughput_layouts(dtype, hidden):
    """More rows than CUs (the wave-per-row and multi-row kernels, the full-row
    variant whose S stores come after all of a row's loads - on 64, 128 and
    256 lanes, and ragged - and the plain slots):
    intermediate == residual and output == a partial still give the oracle's
    results."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    w = inputs.random_fused(dtype, 8, cus + 3, hidden, 720)
    ref_out, ref_inter = ref_fused(w)
    parts = [dev(p, dtype) for p in w.partials]
    res = dev(w.residual, dtype)
    ar.ar_residual_rmsnorm(parts, dev(w.weight, dtype), w.eps, parts[5], res, bias=dev(w.bias, dtype),
                           residual=res)
    torch.cuda.synchronize()
    assert_bitexact(host_bits(res), ref_inter, dtype, "intermediate in place of the residual")
    assert_output_close(host_bits(parts[5]), ref_out, dtype, "output in place of partial 5")


@pytest.mark.parametrize("dtype", DTYPES)
def test_fused_unaligned_pointers(dtype):
    w = inputs.random_fused(dtype, 2, 4, 1024, 800)
    parts = []
    for r, p in enumerate(w.partials):
        t = torch.empty(w.n + 1 + r, dtype=TORCH_DT[dtype], device="cuda")
        t[1 + r:].copy_(dev(p, dtype))
        parts.append(t[1 + r:])
    out, inter = Guarded(w.n, dtype, 1), Guarded(w.n, dtype, 2)
    ar.ar_residual_rmsnorm(parts, dev(w.weight, dtype), w.eps, out.t, inter.t, bias=dev(w.bias, dtype),
                           residual=dev(w.residual, dtype))
    torch.cuda.synchronize()
    out.check_guards()
    inter.check_guards()
    check_fused(w, host_bits(out.t), host_bits(inter.t))


def test_fused_special_rows():
    """Zero rows with eps > 0 give zeros; a constant row gives +-weight;
    eps = 0 with a zero row gives NaN on both sides."""
    H = 1024
    for dtype in DTYPES:
        zero = inputs.to_dtype(np.zeros(3 * H, np.float32), dtype)
        const = inputs.to_dtype(np.full(3 * H, -0.75, np.float32), dtype)
        weight = inputs.normal((H,), 3, 1.0, 0.1, dtype)
        for parts, eps in (([zero, zero], 1e-6), ([const, zero], 0.0), ([zero], 0.0)):
            w = inputs.Workload("special-rows", "fused", dtype, len(parts), 3 * H, H, parts, None, None, weight, eps)
            got_out, got_inter = run_fused(w)
            check_fused(w, got_out, got_inter)


def test_fused_deterministic_at_full_size():
    """The large fused workload, 100 times: bitwise identical each time."""
    w = inputs.make(inputs.FUSED_BF16_R8_2048x8192)
    parts = [dev(p, w.dtype) for p in w.partials]
    weight, res = dev(w.weight, w.dtype), dev(w.residual, w.dtype)
    out, inter = torch.empty_like(parts[0]), torch.empty_like(parts[0])
    first = None
    for i in range(100):
        out.fill_(float("nan"))
        ar.ar_residual_rmsnorm(parts, weight, w.eps, out, inter, residual=res)
        torch.cuda.synchronize()
        b = (host_bits(out), host_bits(inter))
        if first is None:
            first = b
        else:
            assert np.array_equal(b[0], first[0]) and np.array_equal(b[1], first[1]), f"run {i} differs"


def test_raw_params_validation_on_device():
    """Validation through the raw C ABI with real device buffers."""
    t = torch.zeros(1024, device="cuda")
    p = make_params(1024, 2, ar.AR_FP32, [t.data_ptr(), t.data_ptr() + 8], t.data_ptr() + 4)
    assert call("ar_sum", p) == ar.ar.AR_ERR_ALIAS
    p = make_params(1024, 2, ar.AR_FP32, [t.data_ptr(), t.data_ptr()], t.data_ptr() + 2)
    assert call("ar_sum", p) == ar.ar.AR_ERR_ALIGN
    torch.cuda.synchronize()
    assert torch.count_nonzero(t).item() == 0


def test_concurrent_streams_do_not_interfere():
    """The library keeps no per-call state on the device: two streams running
    different entry points at the same time both match their references."""
    a = inputs.random_fused("bf16", 8, 256, 8192, 1600)
    b = inputs.random_sum("fp16", 4, 1 << 22, 1601)
    ap = [dev(p, a.dtype) for p in a.partials]
    aw, aq = dev(a.weight, a.dtype), dev(a.residual, a.dtype)
    bp = [dev(p, b.dtype) for p in b.partials]
    ref_out, ref_inter = torch.empty_like(ap[0]), torch.empty_like(ap[0])
    ar.ar_residual_rmsnorm(ap, aw, a.eps, ref_out, ref_inter, residual=aq)
    ref_sum = torch.empty_like(bp[0])
    ar.ar_sum(bp, ref_sum)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(8):
        o, i, s = torch.empty_like(ap[0]), torch.empty_like(ap[0]), torch.empty_like(bp[0])
        with torch.cuda.stream(s1):
            ar.ar_residual_rmsnorm(ap, aw, a.eps, o, i, residual=aq, stream=s1)
        with torch.cuda.stream(s2):
            ar.ar_sum(bp, s, stream=s2)
        outs.append((o, i, s))
    torch.cuda.synchronize()
    want = (host_bits(ref_out), host_bits(ref_inter), host_bits(ref_sum))
    for o, i, s in outs:
        assert np.array_equal(host_bits(o), want[0])
        assert np.array_equal(host_bits(i), want[1])
        assert np.array_equal(host_bits(s), want[2])


def test_calls_from_several_host_threads():
    """The entry points are re-entrant: host threads, each with its own stream
    and its own shapes (different kernel instances, so first calls fill the
    per-device caches at the same time), all match the oracle."""
    import threading
    cases = [inputs.random_fused("bf16", 8, 300, 5120, 1700), inputs.random_fused("fp16", 3, 270, 3072, 1701),
             inputs.random_fused("fp32", 6, 300, 2560, 1702), inputs.random_fused("bf16", 5, 260, 12288, 1703)]
    sums = [inputs.random_sum("fp16", 7, 300007, 1704), inputs.random_sum("fp32", 5, 200003, 1705)]
    jobs = []
    for w in cases:
        parts = [dev(p, w.dtype) for p in w.partials]
        bufs = (torch.empty_like(parts[0]), torch.empty_like(parts[0]))
        jobs.append(("fused", w, parts, bufs, (dev(w.weight, w.dtype), dev(w.bias, w.dtype), dev(w.residual, w.dtype))))
    for w in sums:
        parts = [dev(p, w.dtype) for p in w.partials]
        jobs.append(("sum", w, parts, (torch.empty_like(parts[0]),), None))
    torch.cuda.synchronize()
    errors = []

    def worker(job):
        try:
            kind, w, parts, bufs, extra = job
            stream = torch.cuda.Stream()
            for _ in range(5):
                if kind == "fused":
                    weight, bias, res = extra
                    ar.ar_residual_rmsnorm(parts, weight, w.eps, bufs[0], bufs[1], bias=bias, residual=res,
                                           stream=stream)
                else:
                    ar.ar_sum(parts, bufs[0], stream=stream)
            stream.synchronize()
        except Exception as e:  # reported by the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(j,)) for j in jobs]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=60)
    torch.cuda.synchronize()
    assert not errors, errors
    for kind, w, parts, bufs, extra in jobs:
        note(f"[parity] threads {kind} {w.name}")
        if kind == "fused":
            check_fused(w, host_bits(bufs[0]), host_bits(bufs[1]))
        else:
            assert_bitexact(host_bits(bufs[0]), ref_sum(w), w.dtype, f"threaded {w.name}")


# ------------------------------------------------------------ prepared calls
@pytest.mark.parametrize("name", [inputs.SUM_FP32_R2_4x256, inputs.SUM_FP16_R2_1000003, inputs.FUSED_FP16_R8_16x4096,
                                  inputs.fused_fp16_r2_5120_name(7)])
def test_prepared_calls_match_the_oracle_on_repeat(name):
    """A prepared call (argument block built once) run three times, on the
    current stream and on a side stream, gives the oracle's result each time;
    inputs are refreshed between calls so a stale launch would show."""
    note(f"[prepared] {name}")
    w = inputs.make(name)
    parts = [dev(p, w.dtype) for p in w.partials]
    out = Guarded(w.n, w.dtype)
    if w.op == "sum":
        call_ = ar.prepare_sum(parts, out.t)
        ref = ref_sum(w)
    else:
        inter = Guarded(w.n, w.dtype)
        call_ = ar.prepare_residual_rmsnorm(parts, dev(w.weight, w.dtype), w.eps, out.t, inter.t,
                                            bias=dev(w.bias, w.dtype), residual=dev(w.residual, w.dtype))
    side = torch.cuda.Stream()
    for k in range(3):
        out.t.zero_()
        if w.op != "sum":
            inter.t.zero_()
        torch.cuda.synchronize()
        if k == 2:
            side.wait_stream(torch.cuda.current_stream())
            call_(stream=side)
            torch.cuda.current_stream().wait_stream(side)
        else:
            call_()
        torch.cuda.synchronize()
        out.check_guards()
        if w.op == "sum":
            assert_bitexact(host_bits(out.t), bits(ref), w.dtype, f"prepared sum, call {k}")
        else:
            inter.check_guards()
            check_fused(w, host_bits(out.t), host_bits(inter.t))


def test_prepared_calls_replayed_from_a_graph():
    """Prepared calls captured into a HIP graph (through torch's CUDA graph)
    and replayed five times, with eager work between the replays (outputs
    filled with NaN; before the last two, new partials copied into the same
    buffers): every replay matches the oracle on the inputs it saw."""
    note("[prepared] graph replay")
    ws = [inputs.random_sum("bf16", 3, 70001, 1601), inputs.random_sum("bf16", 3, 70001, 1611)]
    wf = [inputs.random_fused("fp16", 8, 24, 4096, 1602, bias=True),
          inputs.random_fused("fp16", 8, 24, 4096, 1612, bias=True)]
    sp = [dev(p, "bf16") for p in ws[0].partials]
    fp = [dev(p, "fp16") for p in wf[0].partials]
    wt, b, q = dev(wf[0].weight, "fp16"), dev(wf[0].bias, "fp16"), dev(wf[0].residual, "fp16")
    so = torch.empty_like(sp[0])
    fo, fi = torch.empty_like(fp[0]), torch.empty_like(fp[0])
    calls = [ar.prepare_sum(sp, so), ar.prepare_residual_rmsnorm(fp, wt, wf[0].eps, fo, fi, bias=b, residual=q)]
    for c in calls:  # warm up outside the capture
        c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for c in calls:
                c()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(5):
        k = 0 if rep < 3 else 1
        if rep == 3:  # same buffers, new contents (weight, bias and residual stay)
            for t, p in zip(sp, ws[1].partials):
                t.copy_(dev(p, "bf16"))
            for t, p in zip(fp, wf[1].partials):
                t.copy_(dev(p, "fp16"))
        for t in (so, fo, fi):
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_bitexact(host_bits(so), bits(ref_sum(ws[k])), "bf16", f"graph replay {rep}: sum")
        w = inputs.Workload("graph-fused", "fused", "fp16", 8, wf[k].n, wf[k].hidden, wf[k].partials,
                            wf[0].bias, wf[0].residual, wf[0].weight, wf[0].eps)
        check_fused(w, host_bits(fo), host_bits(fi))


def test_prepared_call_reports_errors():
    """The C entry point's validation still runs on every prepared call."""
    # partial overlap of the output with a partial is rejected when the call runs
    base = torch.zeros(2048, device="cuda", dtype=torch.float16)
    c = ar.prepare_sum([base[:1024], base[1024:]], base[8:1032])
    with pytest.raises(ar.ArError, match="AR_ERR_ALIAS"):
        c()


@pytest.mark.parametrize("dtype", DTYPES)
def test_prepared_unfused_path_matches_plain_calls(dtype):
    """prepare_sum then prepare_rmsnorm (the unfused path, prepared) give
    bitwise what ar_sum then ar_rmsnorm give, with and without side streams."""
    note(f"[prepared] unfused {dtype}")
    w = inputs.random_fused(dtype, 4, 37, 2560, 77)
    parts = [dev(p, dtype) for p in w.partials]
    wt, b, q = dev(w.weight, dtype), dev(w.bias, dtype), dev(w.residual, dtype)
    x1, o1, s1 = (torch.empty_like(parts[0]) for _ in range(3))
    ar.ar_sum(parts, x1)
    ar.ar_rmsnorm(x1, wt, w.eps, o1, s1, bias=b, residual=q)
    x2, o2, s2 = (torch.zeros_like(parts[0]) for _ in range(3))
    ps, pn = ar.prepare_sum(parts, x2), ar.prepare_rmsnorm(x2, wt, w.eps, o2, s2, bias=b, residual=q)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    ps(side)
    pn(side)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for got, want, what in ((x2, x1, "sum"), (s2, s1, "intermediate"), (o2, o1, "output")):
        assert_bitexact(host_bits(got), host_bits(want), dtype, f"prepared unfused {what}")
