"""GPU parity past 2^31 elements (64-bit indexing) and under HIP graph replay.

Large cases: the partials are filled on the device from a counter-based
stream (element i depends only on the stream seed and i), so the host can
recompute any sampled element; the oracle then computes the sampled elements
(sum) or the sampled rows (fused op, rows are independent) and the GPU result
must match them by the usual rules.

Graphs: calls captured into a torch CUDA graph (a HIP graph) and replayed
several times, with eager work and synchronizations in between, must give the
eager result bit for bit on every replay.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_ar_amd as ar
from tensor_all_reduce_ar_amd import inputs

from gpu_util import TORCH_DT, assert_bitexact, assert_output_close, bits, dev, empty_host, host_bits, note

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

BIG = (1 << 31) + 1003  # elements: past the signed 32-bit range, not a multiple of a pack


def _sample_indices(n, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    idx = np.concatenate([np.arange(0, 4096), np.arange((1 << 31) - 4096, min(n, (1 << 31) + 4096)),
                          np.arange(n - 4096, n), rng.integers(0, n, 20000)])
    return np.unique(idx).astype(np.int64)


def _gather(t, idx):
    return host_bits(t[torch.from_numpy(idx).cuda()])


@pytest.mark.parametrize("offset", [0, 1])
def test_sum_past_2_31_elements(offset):
    """Vector path (aligned) and element path (one element of offset) on a
    bf16 sum of 2^31 + 1003 elements, sampled around the 2^31 boundary."""
    dtype, n = "bf16", BIG
    note(f"[large] sum bf16 n={n} offset={offset}")
    seeds = (7001, 7002)
    parts = []
    for s in seeds:
        full = inputs.counter_fill_device(s, n + offset, dtype)
        parts.append(full[offset:])
    out = torch.empty(n + offset, dtype=TORCH_DT[dtype], device="cuda")[offset:]
    ar.ar_sum(parts, out)
    torch.cuda.synchronize()
    idx = _sample_indices(n, 11 + offset)
    host_parts = [inputs.counter_values(s, idx + offset, dtype) for s in seeds]
    assert np.array_equal(_gather(parts[0], idx), host_parts[0].view(np.uint16))  # the two generators agree
    ref = empty_host(idx.size, dtype)
    oracle.ar_sum(dtype, host_parts, ref)
    assert_bitexact(_gather(out, idx), bits(ref), dtype, f"sum past 2^31, offset {offset}")
    del parts, out
    torch.cuda.empty_cache()


def test_fused_past_2_31_elements():
    """bf16, 2 ranks, hidden 8192, 262,147 rows (2^31 + 24,576 elements):
    sampled rows, including the ones that straddle the 2^31 boundary."""
    dtype, H, rows, R = "bf16", 8192, (1 << 18) + 3, 2
    n = rows * H
    note(f"[large] fused bf16 rows={rows} H={H}")
    seeds = (7101, 7102)
    parts = [inputs.counter_fill_device(s, n, dtype) for s in seeds]
    res = inputs.counter_fill_device(7103, n, dtype)
    weight_h = inputs.normal((H,), 7104, 1.0, 0.1, dtype)
    weight = dev(weight_h, dtype)
    out, inter = torch.empty_like(res), torch.empty_like(res)
    ar.ar_residual_rmsnorm(parts, weight, 1e-5, out, inter, residual=res)
    torch.cuda.synchronize()
    boundary_row = (1 << 31) // H
    rng = np.random.Generator(np.random.PCG64(13))
    sample_rows = np.unique(np.concatenate([[0, 1, boundary_row - 1, boundary_row, boundary_row + 1, rows - 1],
                                            rng.integers(0, rows, 24)]))
    idx = (sample_rows[:, None] * H + np.arange(H)[None, :]).ravel().astype(np.int64)
    hp = [inputs.counter_values(s, idx, dtype) for s in seeds]
    hq = inputs.counter_values(7103, idx, dtype)
    ref_out, ref_inter = empty_host(idx.size, dtype), empty_host(idx.size, dtype)
    oracle.ar_residual_rmsnorm(dtype, hp, H, weight_h, 1e-5, ref_out, ref_inter, residual=hq)
    assert_bitexact(_gather(inter, idx), bits(ref_inter), dtype, "fused past 2^31, intermediate")
    assert_output_close(_gather(out, idx), bits(ref_out), dtype, "fused past 2^31, output")
    del parts, res, out, inter
    torch.cuda.empty_cache()


# ------------------------------------------------------------- HIP graphs
def test_graph_replay_matches_eager():
    note("[graph] capture and replay")
    w = inputs.random_fused("bf16", 8, 64, 4096, 1500)
    s = inputs.random_sum("fp16", 4, 100003, 1501)
    one = inputs.random_sum("fp32", 1, 4099, 1502)
    parts = [dev(p, w.dtype) for p in w.partials]
    weight, res = dev(w.weight, w.dtype), dev(w.residual, w.dtype)
    sp = [dev(p, s.dtype) for p in s.partials]
    op = [dev(p, one.dtype) for p in one.partials]
    bufs = {k: torch.empty_like(parts[0]) for k in ("out", "inter", "x", "uo", "ui", "so", "sl")}
    bufs["s"] = torch.empty_like(sp[0])
    bufs["s8"] = torch.empty_like(sp[0])
    bufs["o1"] = torch.empty_like(op[0])

    def work():
        ar.ar_residual_rmsnorm(parts, weight, w.eps, bufs["out"], bufs["inter"], residual=res)
        ar.ar_sum(parts, bufs["x"])
        ar.ar_rmsnorm(bufs["x"], weight, w.eps, bufs["uo"], bufs["ui"], residual=res)
        for k in range(4):
            ar.ar_residual_rmsnorm_slice(parts, weight, w.eps, bufs["so"], bufs["sl"], k, 4, residual=res)
        ar.ar_sum(sp, bufs["s"])
        for k in range(8):
            ar.ar_sum_slice(sp, bufs["s8"], k, 8)
        ar.ar_sum(op, bufs["o1"])  # one rank: a device-to-device copy node

    work()
    torch.cuda.synchronize()
    eager = {k: host_bits(v) for k, v in bufs.items()}
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(5):
        for v in bufs.values():
            v.fill_(float("nan"))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in bufs.items():
            assert np.array_equal(host_bits(v), eager[k]), f"replay {rep}: {k} differs from the eager result"


def test_graph_replay_matches_eager_in_the_throughput_layouts():
    """More rows than CUs, so the captured calls run the throughput layouts:
    the wave-per-row kernel (1024), the multi-row kernel (4096), the
    pipelined walk full on 256 lanes (8192), ragged on 256 lanes (9216) and
    ragged on 512 lanes (20488). Every replay must match the eager result bit
    for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    calls = []
    for hidden in (1024, 4096, 8192, 9216, 20488):
        w = inputs.random_fused("bf16", 8, cus + 5, hidden, 1600 + hidden % 97)
        calls.append(dict(parts=[dev(p, w.dtype) for p in w.partials], weight=dev(w.weight, w.dtype),
                          bias=dev(w.bias, w.dtype), res=dev(w.residual, w.dtype), eps=w.eps))
    for c in calls:
        c["out"], c["inter"] = torch.empty_like(c["parts"][0]), torch.empty_like(c["parts"][0])
    note(f"[graph] throughput layouts, {cus + 5} rows")

    def work():
        for c in calls:
            ar.ar_residual_rmsnorm(c["parts"], c["weight"], c["eps"], c["out"], c["inter"], bias=c["bias"],
                                   residual=c["res"])

    work()
    torch.cuda.synchronize()
    eager = [(host_bits(c["out"]), host_bits(c["inter"])) for c in calls]
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            work()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(5):
        for c in calls:
            c["out"].fill_(float("nan"))  # eager work between replays
            c["inter"].fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, c in enumerate(calls):
            assert np.array_equal(host_bits(c["out"]), eager[i][0]), f"replay {rep}: output {i} differs"
            assert np.array_equal(host_bits(c["inter"]), eager[i][1]), f"replay {rep}: intermediate {i} differs"
