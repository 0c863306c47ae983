"""Benchmark of the fused all-reduce core on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step = one ar_residual_rmsnorm call on the large fused workload: 8 bf16
rank partials of [2048 tokens, 8192 hidden] summed in fp32, plus residual, then
RMSNorm (eps 1e-5, no bias), writing the pre-norm sum and the normed output.
Inputs are seeded synthetic data already resident in HBM. The partials sit
where the all-reduce keeps them: in one allocation from allocate_workspace
(the slots of ar_partials_layout, the counterpart of the comm-buffer workspace
the pages' kernels read); --partials separate puts each in its own torch
allocation instead, and the line reports that layout beside the headline.
The large sum and the fp16 2-rank fused workload take the same layout. Steps rotate over
enough copies of the inputs and outputs (at least 4x the 256 MB last-level
cache in all, the outputs alone at least 2x) that each call streams from and
to HBM rather than the cache.

Prints ONE JSON line: effective HBM GB/s (algorithmic bytes / time), the
roofline of the fused kernel against the 8 TB/s HBM peak, the standalone sum
on its large workload, the fused op on 4096 fp16 rows of 5120 (2 ranks, with
bias), the unfused path and one two-shot share, the per-call latency of the
small workloads, and the CPU oracle timed on the host (its own baseline). Each
large workload also reports the streaming ceiling on its own buffers: the
in-repo streaming kernel (libstream_ceiling.so) reading and writing exactly the
same buffers once, with no other work; copy and read rates over 1 GiB are
reported too.
"""
from __future__ import annotations

import argparse
import gc
import hashlib
import json
import os
import platform
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "effective HBM GB/s and % of peak, fused AR+residual+RMSNorm, 1 MI355X"
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published peak
LLC_BYTES = 256 << 20   # MI355X Infinity Cache
MIN_TIMED_CALLS = 20    # every timed configuration is timed over at least this many calls
FUSED_KERNEL = "ar_rmsnorm_pack_kernel"
SUM_KERNEL = "ar_sum_pack_kernel"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None, help="fused workload name (default: the large bf16 one)")
    ap.add_argument("--no-sum", action="store_true", help="skip the standalone-sum line item")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-next", action="store_true", help="skip the unfused and two-shot line items")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle budget (repeats the sample)")
    ap.add_argument("--partials", choices=("workspace", "separate"), default="workspace",
                    help="where the headline's rank partials live: one allocation from allocate_workspace (the "
                         "all-reduce workspace layout) or one torch allocation each")
    ap.add_argument("--min-calls", type=int, default=MIN_TIMED_CALLS,
                    help="calls timed for every workload but the headline (which takes --steps)")
    return ap.parse_args()


def source_hash(texts=None) -> str:
    """Hash of the kernel source (csrc/ar.hip, csrc/fused_geometry.h,
    include/ar.h) with comments and whitespace removed, so that it changes
    when the code does and not when only a comment does."""
    import re
    if texts is None:
        texts = []
        for rel in ("tensor_all_reduce_ar_amd/csrc/ar.hip", "tensor_all_reduce_ar_amd/csrc/fused_geometry.h",
                    "include/ar.h"):
            with open(os.path.join(ROOT, rel)) as f:
                texts.append(f.read())
    h = hashlib.sha256()
    for t in texts:
        t = re.sub(r"/\*.*?\*/", " ", t, flags=re.S)
        t = re.sub(r"//[^\n]*", " ", t)
        h.update(" ".join(t.split()).encode())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(f"{kernel}:{workload}")
    if not entry or entry.get("source_hash") != source_hash():
        return None
    return entry.get("bytes_per_launch")


def rotation_sets(bytes_per_set: int, out_bytes_per_set: int) -> int:
    """Copies of the inputs/outputs to cycle through: the whole cycle is at
    least 4x the last-level cache and the outputs alone at least 2x, so that
    neither inputs nor earlier outputs are served from cache."""
    return max(2, -(-4 * LLC_BYTES // bytes_per_set), -(-2 * LLC_BYTES // out_bytes_per_set))


LEAD_IN_MAX = 8  # untimed launches queued right before a timed region


def time_launches(torch, launch, nsets, steps, warmup, stream):
    """Whole-region timing (ms per step over `steps` back-to-back launches) and
    per-launch timing (a list of `steps` kernel durations in ms, each between
    two events around one launch), both with HIP events on the launch stream.
    After the warmup, a lead-in of untimed launches (one rotation cycle, at
    most LEAD_IN_MAX) is queued just before the start event, so that the
    device is already busy and the host well ahead when the region starts: a
    host pause early in the region then finds kernels queued instead of an
    idle device. The start event fires when the lead-in has finished, so the
    region holds exactly the `steps` timed launches."""
    for i in range(warmup):
        launch(i % nsets)
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    lead = min(nsets, LEAD_IN_MAX)
    gc_was_on = gc.isenabled()
    gc.disable()  # no collector pause while the host queues a timed region
    try:
        for i in range(lead):
            launch((nsets - lead + i) % nsets)
        start.record(stream)
        for i in range(steps):
            launch(i % nsets)
        stop.record(stream)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(evs):
            a.record(stream)
            launch(i % nsets)
            b.record(stream)
        torch.cuda.synchronize()
    finally:
        if gc_was_on:
            gc.enable()
    return start.elapsed_time(stop) / steps, [a.elapsed_time(b) for a, b in evs]


OUTLIER_FACTOR = 1.5


def launch_stats(per_ms):
    """Median / min / max / mean of per-launch durations (us), and the
    launches slower than OUTLIER_FACTOR x the median, flagged by index."""
    us = [x * 1e3 for x in per_ms]
    med = statistics.median(us)
    out = [(i, round(x, 2)) for i, x in enumerate(us) if x > OUTLIER_FACTOR * med]
    return {"launches": len(us), "median": round(med, 2), "min": round(min(us), 2), "max": round(max(us), 2),
            "mean": round(statistics.mean(us), 2), "mean_without_outliers":
                round(statistics.mean([x for x in us if x <= OUTLIER_FACTOR * med]), 2),
            "outliers": {"rule": f"> {OUTLIER_FACTOR} x median", "count": len(out), "index_us": out}}


def dev(torch, a, dtype):
    import numpy as np
    a = np.ascontiguousarray(a)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(a).cuda()


def slab_copies(torch, ar, parts):
    """Copies of the device partials in one allocation from
    ar.allocate_workspace (the slots of ar_partials_layout); returns
    (allocation, views)."""
    ws = ar.allocate_workspace(parts[0].numel(), parts[0].dtype, len(parts))
    for v, p in zip(ws.partials, parts):
        v.copy_(p)
    return ws.buffer, ws.partials


def partial_sets(torch, ar, base, nsets, layout):
    """`nsets` copies of the device partials `base` (set 0 may be `base`
    itself): one allocation per partial ("separate"), or all partials of a set
    in one allocation from allocate_workspace ("slab"). Returns the sets and
    the allocations to keep alive."""
    sets, keep = [], []
    for k in range(nsets):
        if layout == "slab":
            slab, parts = slab_copies(torch, ar, base)
            keep.append(slab)
        else:
            parts = base if k == 0 else [p.clone() for p in base]
        sets.append(parts)
    return sets, keep


def bench_fused(torch, ar, w, args, stream, layout="separate"):
    """layout: "separate" (one allocation per partial) or "slab" (the partials
    of a set in one allocation at ar_partials_layout's slots)."""
    nb = w.algorithmic_bytes()
    nsets = rotation_sets(nb, 2 * w.n * w.itemsize)
    base = [dev(torch, p, w.dtype) for p in w.partials]
    res0 = dev(torch, w.residual, w.dtype)
    weight = dev(torch, w.weight, w.dtype)
    bias = dev(torch, w.bias, w.dtype) if w.bias is not None else None
    psets, keep = partial_sets(torch, ar, base, nsets, layout)
    sets = []
    for k in range(nsets):
        res = res0 if k == 0 else res0.clone()
        sets.append((psets[k], res, torch.empty_like(res0), torch.empty_like(res0)))
    del base

    # prepared calls: the host queues each launch in a few microseconds, far
    # ahead of the device, so the timed region measures the kernels
    preps = [ar.prepare_residual_rmsnorm(parts, weight, w.eps, out, inter, bias=bias, residual=res)
             for parts, res, out, inter in sets]

    def launch(k):
        preps[k](stream)

    ms_step, per = time_launches(torch, launch, nsets, args.steps, args.warmup, stream)
    out_bits, inter_bits = host_bits(torch, sets[0][2]), host_bits(torch, sets[0][3])

    # The practical ceiling on the same buffers: every partial and the
    # residual read once, S and the output written once, nothing else.
    def streams(k):
        parts, res, out, inter = sets[k]
        return list(parts) + ([res] if w.residual is not None else []), [inter, out]

    ceil_bytes = (w.ranks + (w.residual is not None) + 2) * w.n * w.itemsize
    ceil = stream_ceiling_on(torch, streams, nsets, ceil_bytes, args.steps, args.warmup, stream)
    return dict(bytes=nb, nsets=nsets, ms_step=ms_step, per=launch_stats(per), steps=args.steps,
                out_bits=out_bits, inter_bits=inter_bits, ceil=ceil)


def bench_sum(torch, ar, w, args, stream, layout="separate"):
    """layout as for bench_fused."""
    nb = w.algorithmic_bytes()
    nsets = rotation_sets(nb, w.n * w.itemsize)
    base = [dev(torch, p, w.dtype) for p in w.partials]
    psets, keep = partial_sets(torch, ar, base, nsets, layout)
    sets = [(psets[k], torch.empty_like(base[0])) for k in range(nsets)]
    del base

    preps = [ar.prepare_sum(parts, out) for parts, out in sets]

    def launch(k):
        preps[k](stream)

    steps = max(args.min_calls, args.steps)
    ms_step, per = time_launches(torch, launch, nsets, steps, max(2, args.warmup // 2), stream)
    out_bits = host_bits(torch, sets[0][1])

    # the same buffers, read and written once, nothing else
    ceil = stream_ceiling_on(torch, lambda k: (sets[k][0], [sets[k][1]]), nsets, nb, steps,
                             max(2, args.warmup // 2), stream)
    return dict(bytes=nb, nsets=nsets, ms_step=ms_step, per=launch_stats(per), steps=steps, out_bits=out_bits,
                ceil=ceil)


def bench_unfused(torch, ar, w, args, stream, layout="separate"):
    """The unfused path on the fused workload: ar_sum into a buffer X, then
    ar_rmsnorm (residual, bias, norm) on X. Bytes: the sum's (R+1)*N*s, the
    norm's (X + residual + S + out)*N*s plus weight (and bias)."""
    s = w.itemsize
    nb = (w.ranks + 1) * w.n * s + (1 + (w.residual is not None) + 2) * w.n * s \
        + (1 + (w.bias is not None)) * w.hidden * s
    nsets = rotation_sets(nb, 3 * w.n * s)
    base = [dev(torch, p, w.dtype) for p in w.partials]
    res0 = dev(torch, w.residual, w.dtype)
    weight = dev(torch, w.weight, w.dtype)
    bias = dev(torch, w.bias, w.dtype) if w.bias is not None else None
    psets, keep = partial_sets(torch, ar, base, nsets, layout)
    sets = []
    for k in range(nsets):
        res = res0 if k == 0 else res0.clone()
        sets.append((psets[k], res, torch.empty_like(res0), torch.empty_like(res0), torch.empty_like(res0)))

    preps = [(ar.prepare_sum(parts, x), ar.prepare_rmsnorm(x, weight, w.eps, out, inter, bias=bias, residual=res))
             for parts, res, x, out, inter in sets]

    def launch(k):
        preps[k][0](stream)
        preps[k][1](stream)

    steps = max(args.min_calls, args.steps)
    ms_step, _ = time_launches(torch, launch, nsets, steps, max(2, args.warmup // 2), stream)
    return dict(bytes=nb, nsets=nsets, ms_step=ms_step, steps=steps)


def bench_slice(torch, ar, w, args, stream, num, layout="separate"):
    """One rank's share (slice 0 of `num`) of the two-shot split."""
    s = w.itemsize
    base = [dev(torch, p, w.dtype) for p in w.partials]
    res0 = dev(torch, w.residual, w.dtype) if w.residual is not None else None
    weight = dev(torch, w.weight, w.dtype) if w.weight is not None else None
    out0, inter0 = torch.empty_like(base[0]), torch.empty_like(base[0])
    params = ar.make_params(w.n, w.ranks, {"fp32": 0, "fp16": 1, "bf16": 2}[w.dtype], [t.data_ptr() for t in base],
                            out0.data_ptr(), hidden_size=w.hidden,
                            weight=weight.data_ptr() if weight is not None else 0,
                            intermediate=inter0.data_ptr(), residual=res0.data_ptr() if res0 is not None else 0)
    op = ar.AR_FUSION_NONE if w.op == "sum" else ar.AR_FUSION_RESIDUAL_RMS_NORM
    st, b, e = ar.ar_slice_range(params, op, 0, num)
    assert st == 0, ar.ar_status_string(st)
    m = e - b
    if w.op == "sum":
        nb = (w.ranks + 1) * m * s
    else:
        nb = (w.ranks + 2 + (w.residual is not None)) * m * s + (1 + (w.bias is not None)) * w.hidden * s
    # rotate by the bytes the share itself touches (inputs and outputs), so
    # that its sets, not just the full buffers, exceed the cache as required
    nsets = rotation_sets(nb, (1 if w.op == "sum" else 2) * m * s)
    psets, keep = partial_sets(torch, ar, base, nsets, layout)
    sets = [(psets[0], res0, out0, inter0)]
    for k in range(1, nsets):
        sets.append((psets[k], res0.clone() if res0 is not None else None,
                     torch.empty_like(base[0]), torch.empty_like(base[0])))

    # prepared calls, as for the other timed loops: the host stays ahead
    if w.op == "sum":
        preps = [ar.prepare_sum_slice(parts, out, 0, num) for parts, res, out, inter in sets]
    else:
        preps = [ar.prepare_residual_rmsnorm_slice(parts, weight, w.eps, out, inter, 0, num, residual=res)
                 for parts, res, out, inter in sets]

    def launch(k, on=None):
        preps[k](on if on is not None else stream)

    steps = max(args.min_calls, args.steps)
    ms_step, _ = time_launches(torch, launch, nsets, steps, max(2, args.warmup // 2), stream)

    # The same calls replayed from a HIP graph (one call per rotating set),
    # which takes the host's launch cost out of a call this small.
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for k in range(nsets):
                launch(k, on=side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    reps = max(2, steps // nsets)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        g.replay()
    b.record(stream)
    torch.cuda.synchronize()
    graph_ms = a.elapsed_time(b) / (reps * nsets)
    del g
    return dict(bytes=nb, elements=m, nsets=nsets, ms_step=ms_step, steps=steps, graph_ms=graph_ms)


def bench_small(torch, ar, w, stream, calls=20, reps=20):
    """A launch-bound workload on one set of buffers (warm in cache, as right
    after the GEMMs that produce the partials): per-call time of eager
    back-to-back launches through the binding (each call marshalling its
    arguments, and through a prepared call), and of a HIP graph of `calls`
    back-to-back calls replayed `reps` times (one per-call figure per replay),
    which takes the host's launch cost out. Returns the outputs of the last
    call as raw bits."""
    parts = [dev(torch, p, w.dtype) for p in w.partials]
    out = torch.empty_like(parts[0])
    inter = None
    if w.op == "sum":
        def call(st=None):
            ar.ar_sum(parts, out, stream=st)
    else:
        inter = torch.empty_like(parts[0])
        weight, res = dev(torch, w.weight, w.dtype), dev(torch, w.residual, w.dtype)
        bias = dev(torch, w.bias, w.dtype) if w.bias is not None else None

        def call(st=None):
            ar.ar_residual_rmsnorm(parts, weight, w.eps, out, inter, bias=bias, residual=res, stream=st)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(calls * reps):
        call()
    b.record(stream)
    torch.cuda.synchronize()
    eager = a.elapsed_time(b) * 1e3 / (calls * reps)
    # the same, through a prepared call (argument block built once)
    if w.op == "sum":
        prep = ar.prepare_sum(parts, out)
    else:
        prep = ar.prepare_residual_rmsnorm(parts, weight, w.eps, out, inter, bias=bias, residual=res)
    prep()
    torch.cuda.synchronize()
    a.record(stream)
    for _ in range(calls * reps):
        prep()
    b.record(stream)
    torch.cuda.synchronize()
    eager_prepared = a.elapsed_time(b) * 1e3 / (calls * reps)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            for _ in range(calls):
                call(side)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for x, y in evs:
        x.record(stream)
        g.replay()
        y.record(stream)
    torch.cuda.synchronize()
    per_call = [x.elapsed_time(y) / calls for x, y in evs]  # ms
    del g
    return dict(eager_us=eager, eager_prepared_us=eager_prepared, per_call=per_call, calls=calls, reps=reps,
                out_bits=host_bits(torch, out),
                inter_bits=host_bits(torch, inter) if inter is not None else None)


def stream_ceiling_on(torch, streams, nsets, nbytes, steps, warmup, stream):
    """The in-repo streaming kernel in each of its workgroup shapes on the
    rotating sets' own buffers (`streams(k)` -> (inputs, outputs)); the
    fastest shape is the practical ceiling. GB/s of bytes moved."""
    from tensor_all_reduce_ar_amd import stream_ceiling as sc
    per = {}
    for shape, label in sc.SHAPES.items():
        def launch(k, shape=shape):
            ins, outs = streams(k)
            sc.sc_stream(ins, outs, shape, stream=stream)
        ms, _ = time_launches(torch, launch, nsets, steps, warmup, stream)
        per[label] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    best = max(per, key=per.get)
    return {"gbps": per[best], "shape": best, "per_shape_gbps": per}


def stream_ceilings(torch, stream):
    """Streaming rates over 1 GiB buffers: the in-repo streaming kernel as a
    copy (1 read + 1 write stream) and as a pure read, and torch's own device
    copy. GB/s of bytes moved."""
    from tensor_all_reduce_ar_amd import stream_ceiling as sc
    n = 1 << 28  # fp32 elements, 1 GiB
    # random contents: constant data streams measurably faster than real data
    gen = torch.Generator(device="cuda")
    gen.manual_seed(1)
    src = torch.randn(n, dtype=torch.float32, device="cuda", generator=gen)
    dst = torch.empty_like(src)

    def rate(fn, nbytes, reps=10):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return nbytes / (a.elapsed_time(b) / reps * 1e-3) / 1e9

    out = {
        "copy_gbps": max(rate(lambda: sc.sc_stream([src], [dst], k, stream=stream), 2 * n * 4) for k in sc.SHAPES),
        "read_gbps": max(rate(lambda: sc.sc_stream([src], [], k, stream=stream), n * 4) for k in sc.SHAPES),
        "torch_copy_gbps": rate(lambda: dst.copy_(src), 2 * n * 4),
    }
    del src, dst
    return {k: round(v, 1) for k, v in out.items()}


def oracle_call(w, lo=0, hi=None, out=None, inter=None):
    """The CPU oracle on rows [lo, hi) of a fused workload, or on elements
    [lo, hi) of a sum, writing into `out` (and `inter`) at the same places."""
    import numpy as np

    import oracle
    if w.op == "sum":
        hi = w.n if hi is None else hi
        oracle.ar_sum(w.dtype, [p[lo:hi] for p in w.partials], out[lo:hi])
        return
    hi = w.rows if hi is None else hi
    H = w.hidden
    sl = slice(lo * H, hi * H)
    oracle.ar_residual_rmsnorm(w.dtype, [p[sl] for p in w.partials], H, w.weight, w.eps, out[sl], inter[sl],
                               bias=w.bias, residual=w.residual[sl] if w.residual is not None else None)


def host_threads() -> int:
    """Host threads the all-core oracle uses: the CPUs this process may run
    on (at most 16, the GPU host's share)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


def oracle_timed(w, runs_1t, runs_nt, seconds):
    """The oracle as it stands, on 1 thread and on every host core at once
    (contiguous blocks of rows, or of elements for the sum; the ctypes call
    releases the GIL). Each leg repeats until `runs` runs or `seconds` have
    passed, at least once. Returns the 1-thread result arrays, both medians
    (s), run counts, threads, and whether the all-core result is bitwise the
    1-thread one."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np
    dt = w.partials[0].dtype
    out, inter = np.zeros(w.n, dt), (np.zeros(w.n, dt) if w.op == "fused" else None)

    def repeat(fn, runs):
        times, t_end = [], time.perf_counter() + seconds
        while True:
            t0 = time.perf_counter()
            fn()
            times.append(time.perf_counter() - t0)
            if len(times) >= runs or time.perf_counter() >= t_end:
                return statistics.median(times), len(times)

    t1, n1 = repeat(lambda: oracle_call(w, out=out, inter=inter), runs_1t)
    units = w.n if w.op == "sum" else w.rows
    threads = max(1, min(host_threads(), units))
    blocks = [(units * k // threads, units * (k + 1) // threads) for k in range(threads)]
    m_out, m_inter = np.zeros_like(out), (np.zeros_like(inter) if inter is not None else None)
    with ThreadPoolExecutor(threads) as ex:
        tn, nn = repeat(lambda: list(ex.map(lambda b: oracle_call(w, b[0], b[1], m_out, m_inter), blocks)), runs_nt)
    same = bool(np.array_equal(m_out, out) and (inter is None or np.array_equal(m_inter, inter)))
    return dict(out=out, inter=inter, t1=t1, n1=n1, tn=tn, nn=nn, threads=threads, nt_bitexact=same)


def compare_to_oracle(w, gpu_out, gpu_inter, ref_out, ref_inter):
    """The comparison rules: sums and pre-norm sums bitwise (NaN == NaN);
    normed outputs within 2 ulp (fp16/bf16: the distance between
    order-preserving integer encodings, +0 == -0) or 1e-5 relative (fp32).
    Also reported: the largest relative error |gpu - ref| / |ref| over the
    elements whose reference is finite, with |ref| floored at the type's
    smallest normal so that zeros do not divide."""
    import numpy as np

    def bits(a):
        return a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint16)

    def ordered(b):
        b = b.astype(np.int64)
        sign = 0x80000000 if w.dtype == "fp32" else 0x8000
        return np.where(b & sign, sign - b, b)

    def values(b):
        if w.dtype == "fp32":
            return b.view(np.float32).astype(np.float64)
        if w.dtype == "fp16":
            return b.view(np.float16).astype(np.float64)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)

    def max_rel(g_bits, r_bits):
        g, r = values(g_bits), values(r_bits)
        ok = np.isfinite(r)
        if not ok.any():
            return 0.0
        tiny = float(np.finfo(np.float16 if w.dtype == "fp16" else np.float32).tiny)
        return float(np.max(np.abs(g[ok] - r[ok]) / np.maximum(np.abs(r[ok]), tiny)))

    rec = {}
    if w.op == "sum":
        rec["bitexact"] = bool(np.array_equal(gpu_out, bits(ref_out)))
        rec["max_ulp"] = int(np.abs(ordered(gpu_out) - ordered(bits(ref_out))).max())
        rec["max_rel"] = max_rel(gpu_out, bits(ref_out))
        return rec
    rec["intermediate_bitexact"] = bool(np.array_equal(gpu_inter, bits(ref_inter)))
    rec["output_max_ulp"] = int(np.abs(ordered(gpu_out) - ordered(bits(ref_out))).max())
    rec["output_max_rel"] = max_rel(gpu_out, bits(ref_out))
    if w.dtype == "fp32":
        rec["within_tolerance"] = bool(rec["intermediate_bitexact"] and rec["output_max_rel"] <= 1e-5)
    else:
        rec["within_tolerance"] = bool(rec["intermediate_bitexact"] and rec["output_max_ulp"] <= 2)
    return rec


def host_cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_bits(torch, t):
    import numpy as np
    t = t.cpu()
    if t.element_size() == 4:
        return t.view(torch.int32).numpy().view(np.uint32)
    return t.view(torch.int16).numpy().view(np.uint16)


def workload_record(w, nbytes, timing, stats, extra=None):
    """One workload's GPU figures: per-call median / min / max (us), GB/s and
    fraction of the HBM peak at the median, and how they were timed."""
    rec = {"op": "sum" if w.op == "sum" else "fused", "ranks": w.ranks, "dtype": w.dtype,
           "shape": [w.n] if w.op == "sum" else [w.rows, w.hidden], "bias": w.bias is not None,
           "seeds": w.seeds, "distribution": w.distribution, "bytes": nbytes, "timing": timing,
           "gpu_us_median": stats["median"], "gpu_us_min": stats["min"], "gpu_us_max": stats["max"],
           "gbps_at_median": round(nbytes / (stats["median"] * 1e-6) / 1e9, 1),
           "pct_of_peak_at_median": round(100 * nbytes / (stats["median"] * 1e-6) / 1e9 / HBM_PEAK_GBPS, 2),
           "per_call_us": stats}
    rec.update(extra or {})
    return rec


COLD = "cold: rotating input sets (whole cycle >= 4x the 256 MB cache), HIP events around each launch"
WARM = "warm: one set of buffers, a HIP graph of 20 back-to-back calls replayed 20 times (one figure per replay)"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus > 1 or world > 1:
        print(f"bench.py runs on one GPU only: the all-reduce core here is one GPU's share of the work "
              f"(all rank partials in local HBM); --gpus {max(args.gpus, world)} is not supported.",
              file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import tensor_all_reduce_ar_amd as ar
    from tensor_all_reduce_ar_amd import inputs

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    name = args.workload or inputs.FUSED_BF16_R8_2048x8192
    t0 = time.time()
    w = inputs.make(name)
    if w.op != "fused":
        raise SystemExit("--workload must name a fused workload")
    print(f"[bench] inputs for {name} ready in {time.time() - t0:.1f}s", file=sys.stderr, flush=True)

    # The rank partials of the headline live where the all-reduce's own
    # workspace puts them (allocate_workspace, the counterpart of the comm
    # buffers the kernels read), unless --partials separate.
    head_layout = "slab" if args.partials == "workspace" else "separate"
    other_layout = "separate" if head_layout == "slab" else "slab"
    f = bench_fused(torch, ar, w, args, stream, layout=head_layout)
    gbps = f["bytes"] / (f["ms_step"] * 1e-3) / 1e9
    # One launch per step, back to back on one stream (no gaps between them):
    # the region time per step is the average launch duration.
    achieved = gbps
    print(f"[bench] fused ({args.partials} partials): {f['ms_step'] * 1e3:.1f} us/step ({achieved:.0f} GB/s); "
          f"isolated launches median "
          f"{f['per']['median']:.1f} us; streaming ceiling on the same buffers {f['ceil']['gbps']:.0f} GB/s",
          file=sys.stderr, flush=True)
    gpu = {name: (w, f.pop("out_bits"), f.pop("inter_bits"))}  # outputs to check against the oracle
    records = {name: workload_record(w, f["bytes"], COLD, f["per"], {
        "us_per_call_back_to_back": round(f["ms_step"] * 1e3, 2), "rotating_input_sets": f["nsets"],
        "stream_ceiling_same_buffers_gbps": f["ceil"]["gbps"], "partials": args.partials})}

    result = {
        "metric": METRIC,
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["ms_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": name, "op": "RESIDUAL_RMS_NORM", "ranks": w.ranks, "tokens": w.rows,
            "hidden": w.hidden, "bias": w.bias is not None, "residual": w.residual is not None, "eps": w.eps,
            "bytes_per_step": f["bytes"], "rotating_input_sets": f["nsets"], "seeds": w.seeds,
            "partials": ("one allocation per set from allocate_workspace (ar_partials_layout's staggered slots)"
                         if head_layout == "slab" else "one torch allocation per partial"),
            "distribution": w.distribution,
        },
        "pct_of_peak": round(100 * gbps / HBM_PEAK_GBPS, 2),
        "roofline": {
            "kernel": FUSED_KERNEL, "bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": measured_traffic(FUSED_KERNEL, name),
            "stream_ceiling_same_buffers": f["ceil"],
            "frac_of_stream_ceiling": round(achieved / f["ceil"]["gbps"], 4),
            "launch_us": round(f["ms_step"] * 1e3, 2), "algorithmic_bytes_per_launch": f["bytes"],
            "isolated_launch_us": f["per"],
        },
    }

    if not args.no_sum:
        sw = inputs.make(inputs.SUM_BF16_R4_8192x8192)
        s = bench_sum(torch, ar, sw, args, stream, layout=head_layout)
        s_ach = s["bytes"] / (s["ms_step"] * 1e-3) / 1e9
        result["standalone_sum"] = {
            "workload": sw.name, "kernel": SUM_KERNEL, "bytes_per_call": s["bytes"], "partials": args.partials,
            "us_per_call": round(s["ms_step"] * 1e3, 2), "isolated_launch_us": s["per"],
            "gbps": round(s_ach, 1), "achieved": round(s_ach, 1),
            "frac": round(s_ach / HBM_PEAK_GBPS, 4), "steps": s["steps"], "rotating_input_sets": s["nsets"],
            "traffic": measured_traffic(SUM_KERNEL, sw.name),
            "stream_ceiling_same_buffers": s["ceil"],
            "frac_of_stream_ceiling": round(s_ach / s["ceil"]["gbps"], 4),
        }
        gpu[sw.name] = (sw, s.pop("out_bits"), None)
        if not args.no_next:
            sl = bench_sum(torch, ar, sw, args, stream, layout=other_layout)
            sl_gbps = sl["bytes"] / (sl["ms_step"] * 1e-3) / 1e9
            result["standalone_sum"]["other_partials_layout"] = {
                "what": ("the same sum with one torch allocation per partial" if other_layout == "separate" else
                         "the same sum with each set's partials in one allocation from allocate_workspace"),
                "us_per_call": round(sl["ms_step"] * 1e3, 2), "gbps": round(sl_gbps, 1),
                "frac": round(sl_gbps / HBM_PEAK_GBPS, 4), "stream_ceiling_same_buffers": sl["ceil"],
                "frac_of_stream_ceiling": round(sl_gbps / sl["ceil"]["gbps"], 4),
                "gpu_matches_headline_layout": bool(np.array_equal(sl["out_bits"], gpu[sw.name][1])),
            }
            del sl
        records[sw.name] = workload_record(sw, s["bytes"], COLD, s["per"], {
            "us_per_call_back_to_back": round(s["ms_step"] * 1e3, 2), "rotating_input_sets": s["nsets"],
            "stream_ceiling_same_buffers_gbps": s["ceil"]["gbps"], "partials": args.partials})
        print(f"[bench] sum: {s['ms_step'] * 1e3:.1f} us/call ({s_ach:.0f} GB/s)", file=sys.stderr, flush=True)

    if not args.no_next:
        u = bench_unfused(torch, ar, w, args, stream, layout=head_layout)
        result["unfused_baseline"] = {
            "what": "ar_sum into a buffer, then ar_rmsnorm on it (two launches), partials laid out as the headline's",
            "us_per_call": round(u["ms_step"] * 1e3, 2), "bytes_per_call": u["bytes"], "steps": u["steps"],
            "gbps": round(u["bytes"] / (u["ms_step"] * 1e-3) / 1e9, 1),
            "fused_us_per_call": round(f["ms_step"] * 1e3, 2),
            "time_saved_by_fusion": round(1 - f["ms_step"] / u["ms_step"], 4),
        }
        print(f"[bench] unfused: {u['ms_step'] * 1e3:.1f} us/call", file=sys.stderr, flush=True)
        sl = bench_slice(torch, ar, w, args, stream, w.ranks, layout=head_layout)
        result["two_shot_share"] = {
            "what": f"slice 0 of {w.ranks} of the fused op (one rank's share of a two-shot split)",
            "elements": sl["elements"], "bytes_per_call": sl["bytes"], "us_per_call": round(sl["ms_step"] * 1e3, 2),
            "gbps": round(sl["bytes"] / (sl["ms_step"] * 1e-3) / 1e9, 1), "steps": sl["steps"],
            "graph_us_per_call": round(sl["graph_ms"] * 1e3, 2),
            "graph_gbps": round(sl["bytes"] / (sl["graph_ms"] * 1e-3) / 1e9, 1),
        }
        print(f"[bench] two-shot share: {sl['ms_step'] * 1e3:.1f} us/call eager, {sl['graph_ms'] * 1e3:.1f} us/call "
              f"from a HIP graph", file=sys.stderr, flush=True)

        gpu_out, gpu_inter = gpu[name][1], gpu[name][2]
        sl = bench_fused(torch, ar, w, args, stream, layout=other_layout)
        sl_gbps = sl["bytes"] / (sl["ms_step"] * 1e-3) / 1e9
        key = "fused_partials_separate" if other_layout == "separate" else "fused_partials_in_layout"
        result[key] = {
            "what": ("the same fused workload with one torch allocation per partial" if other_layout == "separate"
                     else "the same fused workload with each set's partials in one allocation from "
                          "allocate_workspace (the slots of ar_partials_layout: 4 KiB more stagger per partial)"),
            "us_per_call": round(sl["ms_step"] * 1e3, 2), "gbps": round(sl_gbps, 1),
            "frac": round(sl_gbps / HBM_PEAK_GBPS, 4), "isolated_launch_us": sl["per"],
            "stream_ceiling_same_buffers": sl["ceil"],
            "frac_of_stream_ceiling": round(sl_gbps / sl["ceil"]["gbps"], 4),
            "gpu_matches_headline_layout": bool(np.array_equal(sl["out_bits"], gpu_out) and
                                                np.array_equal(sl["inter_bits"], gpu_inter)),
        }
        print(f"[bench] fused, partials {other_layout}: {sl['ms_step'] * 1e3:.1f} us/call "
              f"({sl_gbps:.0f} GB/s)", file=sys.stderr, flush=True)
        del sl
        mw = inputs.make(inputs.fused_fp16_r2_5120_name(4096))
        m = bench_fused(torch, ar, mw, args, stream, layout=head_layout)
        m_gbps = m["bytes"] / (m["ms_step"] * 1e-3) / 1e9
        result["fused_fp16_r2_4096x5120"] = {
            "workload": mw.name, "kernel": FUSED_KERNEL, "bytes_per_call": m["bytes"], "partials": args.partials,
            "us_per_call": round(m["ms_step"] * 1e3, 2), "gbps": round(m_gbps, 1),
            "frac": round(m_gbps / HBM_PEAK_GBPS, 4), "rotating_input_sets": m["nsets"],
            "isolated_launch_us": m["per"], "traffic": measured_traffic(FUSED_KERNEL, mw.name),
            "stream_ceiling_same_buffers": m["ceil"],
            "frac_of_stream_ceiling": round(m_gbps / m["ceil"]["gbps"], 4),
        }
        gpu[mw.name] = (mw, m.pop("out_bits"), m.pop("inter_bits"))
        records[mw.name] = workload_record(mw, m["bytes"], COLD, m["per"], {
            "us_per_call_back_to_back": round(m["ms_step"] * 1e3, 2), "rotating_input_sets": m["nsets"],
            "stream_ceiling_same_buffers_gbps": m["ceil"]["gbps"], "partials": args.partials})
        print(f"[bench] fused fp16 R=2 4096x5120: {m['ms_step'] * 1e3:.1f} us/call ({m_gbps:.0f} GB/s)",
              file=sys.stderr, flush=True)

        small = [inputs.SUM_FP32_R2_4x256, inputs.FUSED_FP16_R8_16x4096, inputs.SUM_FP16_R2_1000003] + \
            [inputs.fused_fp16_r2_5120_name(t) for t in (1, 7, 64)]
        for nm in small:
            sw_ = inputs.make(nm)
            r = bench_small(torch, ar, sw_, stream)
            stats = launch_stats(r["per_call"])
            stats["launches"] = r["calls"] * r["reps"]
            records[nm] = workload_record(sw_, sw_.algorithmic_bytes(), WARM, stats, {
                "eager_us_per_call": round(r["eager_us"], 2),
                "eager_prepared_us_per_call": round(r["eager_prepared_us"], 2), "graph_replays": r["reps"]})
            gpu[nm] = (sw_, r["out_bits"], r["inter_bits"])
        print("[bench] launch-bound workloads done", file=sys.stderr, flush=True)

    ceilings = stream_ceilings(torch, stream)
    result["copy_ceiling_gbps"] = ceilings["copy_gbps"]
    result["stream_ceilings_1gib"] = ceilings

    if not args.no_cpu_baseline:
        # The oracle on the host, on the same inputs, checked against this run's
        # GPU outputs: every workload on 1 thread and on every core; the
        # headline workload's 1-thread rate is the reported CPU baseline.
        for nm, (wk, g_out, g_inter) in gpu.items():
            big = wk.algorithmic_bytes() > (64 << 20)
            secs = args.cpu_seconds if nm == name else (8.0 if big else 2.0)
            # the headline's 1-thread leg (the reported baseline) repeats until
            # its time budget is spent; the others stop at a few runs
            runs_1t = 1000 if nm == name else (3 if big else 20)
            o = oracle_timed(wk, runs_1t, 3 if big else 20, secs)
            rec = records[nm]
            rec["vs_oracle"] = compare_to_oracle(wk, g_out, g_inter, o["out"], o["inter"])
            rec.update({"oracle_1t_ms": round(o["t1"] * 1e3, 3), "oracle_1t_runs": o["n1"],
                        "oracle_nt_ms": round(o["tn"] * 1e3, 3), "oracle_nt_runs": o["nn"],
                        "oracle_threads": o["threads"], "oracle_nt_bitexact_vs_1t": o["nt_bitexact"],
                        "oracle_1t_gbps": round(wk.algorithmic_bytes() / o["t1"] / 1e9, 4),
                        "oracle_nt_gbps": round(wk.algorithmic_bytes() / o["tn"] / 1e9, 4)})
            if nm == name:
                result["cpu_baseline"] = {
                    "value": rec["oracle_1t_gbps"], "unit": "GB/s", "cores": 1, "kind": "oracle",
                    "sample": f"the whole {name} call ({wk.rows} rows), {o['n1']} run(s), median {o['t1']:.2f} s",
                    "host_cpu": host_cpu_model(), "host_logical_cpus": os.cpu_count(),
                    "gpu_vs_oracle": rec["vs_oracle"],
                    "all_cores": {
                        "value": rec["oracle_nt_gbps"], "unit": "GB/s", "cores": o["threads"],
                        "sample": f"the same call split into {o['threads']} row blocks, one thread each, "
                                  f"{o['nn']} run(s), median {o['tn']:.3f} s",
                        "bitexact_vs_one_thread": o["nt_bitexact"],
                    },
                }
            print(f"[bench] oracle {nm}: {o['t1'] * 1e3:.1f} ms on 1 thread, {o['tn'] * 1e3:.1f} ms on "
                  f"{o['threads']}; GPU vs oracle {rec['vs_oracle']}", file=sys.stderr, flush=True)
    result["per_workload"] = records
    result["host"] = {"cpu": host_cpu_model(), "logical_cpus": os.cpu_count(), "oracle_threads": host_threads()}
    result["versions"] = {"torch": torch.__version__, "hip": getattr(torch.version, "hip", None),
                          "source_hash": source_hash()}
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
