"""Randomized GPU parity: seeded cases that combine what the other GPU tests
vary one at a time. Each case draws the op (sum or fused), element type, rank
count, size (row width and row count for the fused op, element count for the
sum), whether bias and residual are present, an aliasing mode the ABI allows
(output = a partial, intermediate = the residual or a partial), and element
offsets that move pointers off 16-byte alignment, and is compared with the
oracle on the same inputs: sums and pre-norm sums bit for bit, normed outputs
within 1e-5 relative (fp32) or 2 ulp (fp16/bf16). Outputs that are not aliased
to an input carry canaries on both sides. A second set draws fused cases with
rows wider than 2048 packs (the 512-lane, two-pass and chunked paths).
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_all_reduce_ar_amd as ar
from tensor_all_reduce_ar_amd import inputs

from gpu_util import TORCH_DT, Guarded, assert_bitexact, assert_output_close, bits, dev, empty_host, host_bits, note


DTYPES = ("fp32", "fp16", "bf16")
CASES = 600
MAX_ELEMS = 1 << 21
WIDE_CASES = 150
WIDE_MAX_ELEMS = 1 << 23


def draw(case):
    """The parameters of one case (deterministic in `case`)."""
    rng = np.random.Generator(np.random.PCG64(20_000 + case))
    c = {"op": "sum" if rng.random() < 0.4 else "fused", "dtype": DTYPES[rng.integers(3)],
         "ranks": int(rng.integers(1, 9)), "seed": 30_000 + case}
    v = 4 if c["dtype"] == "fp32" else 8
    if c["op"] == "sum":
        c["n"] = int(np.exp(rng.uniform(0, np.log(MAX_ELEMS))))
        c["alias"] = "out=partial" if rng.random() < 0.3 else "none"
    else:
        if rng.random() < 0.6:
            hidden = int(rng.integers(1, 2600)) * v        # 16-byte rows: the vector kernels
        else:
            hidden = int(rng.integers(1, 9000))            # any width: often the element-wise kernel
        rows = int(rng.choice([1, 2, 3, 7, 64, int(rng.integers(1, 400))]))
        rows = max(1, min(rows, MAX_ELEMS // hidden))
        c.update(hidden=hidden, rows=rows, n=hidden * rows, bias=bool(rng.random() < 0.5),
                 residual=bool(rng.random() < 0.7))
        modes = ["none", "out=partial", "inter=partial"] + (["inter=residual"] if c["residual"] else [])
        c["alias"] = modes[rng.integers(len(modes))]
    c["alias_rank"] = int(rng.integers(c["ranks"]))
    # element offsets of each partial and of the first output (0 keeps 16-byte alignment)
    c["offsets"] = [int(rng.integers(1, v)) if rng.random() < 0.2 else 0 for _ in range(c["ranks"] + 2)]
    return c


def device_with_offset(a, dtype, off):
    t = torch.empty(a.size + off, dtype=TORCH_DT[dtype], device="cuda")
    t[off:].copy_(dev(a, dtype))
    return t[off:]


def draw_wide(case):
    """A fused case with rows of 2049..9000 16-byte packs - the 512-lane
    register path (fp32 up to 2 ranks, 16-bit types up to 4096 packs), the
    two-pass kernel (fp32 rows of up to 4096 packs from 3 ranks) and the
    chunked path (more than 4096 packs) - at 1..WIDE_MAX_ELEMS elements."""
    rng = np.random.Generator(np.random.PCG64(50_000 + case))
    c = {"op": "fused", "dtype": DTYPES[rng.integers(3)], "ranks": int(rng.integers(1, 9)), "seed": 60_000 + case}
    v = 4 if c["dtype"] == "fp32" else 8
    hidden = int(rng.integers(2049, 9001)) * v
    top = WIDE_MAX_ELEMS // hidden
    rows = int(rng.choice([1, 2, int(rng.integers(1, 129)), int(rng.integers(1, top + 1))]))
    rows = max(1, min(rows, top))
    c.update(hidden=hidden, rows=rows, n=hidden * rows, bias=bool(rng.random() < 0.5),
             residual=bool(rng.random() < 0.7))
    modes = ["none", "out=partial", "inter=partial"] + (["inter=residual"] if c["residual"] else [])
    c["alias"] = modes[rng.integers(len(modes))]
    c["alias_rank"] = int(rng.integers(c["ranks"]))
    c["offsets"] = [0] * (c["ranks"] + 2)
    return c


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("case", range(CASES))
def test_random_case_matches_oracle(case):
    c = draw(case)
    note(f"[random] case {case}: {c}")
    run_case(c, f"random case {case}")


@pytest.mark.gpu
@pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")
@pytest.mark.parametrize("case", range(WIDE_CASES))
def test_random_wide_row_case_matches_oracle(case):
    c = draw_wide(case)
    note(f"[random] wide case {case}: {c}")
    run_case(c, f"random wide case {case}")


def run_case(c, label):
    """Runs one drawn case on the GPU and compares it with the oracle."""
    dt, R = c["dtype"], c["ranks"]
    if c["op"] == "sum":
        w = inputs.random_sum(dt, R, c["n"], c["seed"])
    else:
        w = inputs.random_fused(dt, R, c["rows"], c["hidden"], c["seed"], bias=c["bias"], residual=c["residual"])
    parts = [device_with_offset(p, dt, off) for p, off in zip(w.partials, c["offsets"])]
    guarded = []
    if c["alias"] == "out=partial":
        out = parts[c["alias_rank"]]
    else:
        g = Guarded(w.n, dt, c["offsets"][R])
        guarded.append(g)
        out = g.t

    if c["op"] == "sum":
        ar.ar_sum(parts, out)
        torch.cuda.synchronize()
        for g in guarded:
            g.check_guards()
        ref = empty_host(w.n, dt)
        oracle.ar_sum(dt, w.partials, ref)
        assert_bitexact(host_bits(out), bits(ref), dt, f"{label}: sum")
        return

    residual = device_with_offset(w.residual, dt, c["offsets"][R + 1]) if w.residual is not None else None
    if c["alias"] == "inter=residual":
        inter = residual
    elif c["alias"] == "inter=partial":
        inter = parts[c["alias_rank"]]
    else:
        g = Guarded(w.n, dt)
        guarded.append(g)
        inter = g.t
    bias = dev(w.bias, dt) if w.bias is not None else None
    ar.ar_residual_rmsnorm(parts, dev(w.weight, dt), w.eps, out, inter, bias=bias, residual=residual,
                           hidden_size=w.hidden)
    torch.cuda.synchronize()
    for g in guarded:
        g.check_guards()
    ref_out, ref_inter = empty_host(w.n, dt), empty_host(w.n, dt)
    oracle.ar_residual_rmsnorm(dt, w.partials, w.hidden, w.weight, w.eps, ref_out, ref_inter, bias=w.bias,
                               residual=w.residual)
    assert_bitexact(host_bits(inter), bits(ref_inter), dt, f"{label}: intermediate")
    assert_output_close(host_bits(out), bits(ref_out), dt, f"{label}: output")


def test_random_cases_cover_every_dimension():
    """Host only. The draw reaches every op, type, rank count, aliasing mode,
    the optional terms both ways, misaligned pointers, non-16-byte rows and
    one-row calls."""
    cs = [draw(k) for k in range(CASES)]
    assert {c["op"] for c in cs} == {"sum", "fused"}
    assert {c["dtype"] for c in cs} == set(DTYPES)
    assert {c["ranks"] for c in cs} == set(range(1, 9))
    fused = [c for c in cs if c["op"] == "fused"]
    assert {c["alias"] for c in fused} == {"none", "out=partial", "inter=partial", "inter=residual"}
    assert {c["bias"] for c in fused} == {True, False} and {c["residual"] for c in fused} == {True, False}
    assert any(any(o for o in c["offsets"]) for c in cs)
    assert any(c["hidden"] * (4 if c["dtype"] == "fp32" else 2) % 16 for c in fused)
    assert any(c["rows"] == 1 for c in fused)
    assert any(c["alias"] == "out=partial" for c in cs if c["op"] == "sum")


def test_random_wide_cases_cover_every_path():
    """Host only. The wide-row draw reaches every type and rank count, rows
    of 2049..4096 packs (fp32 from 3 ranks among them) and of more, one row,
    and rows wider than 4096 packs at more and fewer than 128 rows."""
    cs = [draw_wide(k) for k in range(WIDE_CASES)]
    assert {c["dtype"] for c in cs} == set(DTYPES)
    assert {c["ranks"] for c in cs} == set(range(1, 9))
    packs = [c["hidden"] * (4 if c["dtype"] == "fp32" else 2) // 16 for c in cs]
    assert any(p <= 4096 for p in packs) and any(p > 4096 for p in packs)
    assert any(p <= 4096 and c["dtype"] == "fp32" and c["ranks"] >= 3 for c, p in zip(cs, packs))
    assert any(c["rows"] == 1 for c in cs)
    wide = [c for c, p in zip(cs, packs) if p > 4096]
    assert any(c["rows"] <= 128 for c in wide) and any(c["rows"] > 128 for c in wide)
    assert {c["alias"] for c in cs} >= {"none", "out=partial", "inter=partial"}
