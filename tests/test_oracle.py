"""Pins for the CPU oracle (no GPU).

The pages print no numbers, so every pin here is a closed form, an exact
special case, an invariant, a library routine the oracle does not use, or
brute force on tiny inputs. Each is chosen so that a plausible slip in the
oracle (a dropped or repeated term, a wrong index, a wrong order of adds, the
wrong divisor, eps outside the root, norming the unrounded sum, accumulating in
the wrong precision) fails at least one of them.

Sources of what is pinned: "All Reduce Plugin" page (all-reduce is a SUM over
tensor-parallel ranks; one rank is a passthrough); "type.d2" page
(AllReduceFusionParams: bias_buffer is the GEMM bias, residual_buffer, RMSNorm
over hidden_size with weight_buffer and eps, intermediate_buffer); "allreduce.d2"
page (fused branch ... -> rms_norm; unfused branch: all-reduce then
rms_norm_kernel, which must compute the same function).
"""
import functools
import hashlib
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as orc
from tensor_all_reduce_ar_amd import inputs

DTYPES = ("fp32", "fp16", "bf16")
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "oracle_small.json")


# ---------------------------------------------------------------- helpers
def enc(vals, dtype):
    """Exactly representable values -> array of the type (numpy/torch rounding)."""
    return inputs.to_dtype(np.asarray(vals, dtype=np.float32), dtype)


def dec(a, dtype):
    """Array of the type -> float64 values (numpy/torch widening)."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).double().numpy()
    return np.asarray(a).astype(np.float64)


def bits(a):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32 if a.dtype.itemsize == 4 else np.uint16)


def empty(n, dtype):
    return np.zeros(n, dtype={"fp32": np.float32, "fp16": np.float16, "bf16": np.uint16}[dtype])


def osum(dtype, parts):
    out = empty(parts[0].size, dtype)
    orc.ar_sum(dtype, parts, out)
    return out


def ofused(dtype, parts, hidden, weight, eps, bias=None, residual=None):
    n = parts[0].size
    out, inter = empty(n, dtype), empty(n, dtype)
    orc.ar_residual_rmsnorm(dtype, parts, hidden, weight, eps, out, inter, bias=bias, residual=residual)
    return out, inter


def onorm(dtype, x, weight, eps, hidden):
    out = empty(x.size, dtype)
    orc.rmsnorm(dtype, x, weight, eps, out, hidden)
    return out


def ulp_at(v, dtype):
    """Spacing of the type's numbers at |v| (for bounds only)."""
    p, emin = {"fp32": (24, -126), "fp16": (11, -14), "bf16": (8, -126)}[dtype]
    e = max(math.frexp(abs(v))[1] - 1, emin) if v != 0 else emin
    return 2.0 ** (e - p + 1)


# --------------------------------------------------- converters (rounding)
def test_decode_fp16_exhaustive_vs_numpy():
    allbits = np.arange(65536, dtype=np.uint16)
    ref = allbits.view(np.float16).astype(np.float64)
    got = np.array([orc.f64_from_f16(int(h)) for h in allbits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_decode_bf16_exhaustive_vs_torch():
    allbits = np.arange(65536, dtype=np.uint16)
    ref = dec(allbits, "bf16")
    got = np.array([orc.f64_from_bf16(int(h)) for h in allbits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def _f32_samples(seed, lo_exp, hi_exp, count):
    rng = np.random.Generator(np.random.PCG64(seed))
    mant = rng.integers(0, 1 << 23, size=count, dtype=np.uint32)
    expo = rng.integers(lo_exp + 127, hi_exp + 127, size=count, dtype=np.uint32)
    sign = rng.integers(0, 2, size=count, dtype=np.uint32) << 31
    return (sign | (expo << 23) | mant).view(np.float32)


def _midpoints16(dtype, seed, count):
    """Exact midpoints between neighbouring finite 16-bit values (the ties)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    hb = rng.integers(0, 0x7BFF if dtype == "fp16" else 0x7F7F, size=count, dtype=np.uint16)
    lo, hi = dec(hb, dtype), dec(hb + 1, dtype)
    mid = (lo + hi) / 2
    sign = np.where(rng.integers(0, 2, size=count) == 1, -1.0, 1.0)
    return (mid * sign).astype(np.float32)  # exact: the midpoint has <= p+1 significant bits


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_encode_from_fp32_vs_library(dtype):
    lo, hi = (-26, 17) if dtype == "fp16" else (-127, 128)
    x = np.concatenate([
        _f32_samples(11, lo, hi, 20000),
        _midpoints16(dtype, 12, 5000),
        np.array([0.0, -0.0, np.inf, -np.inf, 65504, 65519.996, 65520, -65520, 2.0 ** -24, 2.0 ** -25,
                  3 * 2.0 ** -26, 2.0 ** -133, 2.0 ** -134, 3.0e38, 3.4028235e38], dtype=np.float32),
    ])
    ref = bits(enc(x, dtype))  # numpy (fp16) / torch (bf16) fp32 -> 16-bit conversion
    conv = orc.f16_from_f64 if dtype == "fp16" else orc.bf16_from_f64
    got = np.array([conv(float(v)) for v in x], dtype=np.uint16)
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("dtype", ["fp16", "bf16"])
def test_encode_from_fp64_is_nearest_even(dtype):
    """Brute force: the encoding of a double is the nearest neighbour, ties to
    even, checked against both adjacent encodings."""
    conv = orc.f16_from_f64 if dtype == "fp16" else orc.bf16_from_f64
    decode = orc.f64_from_f16 if dtype == "fp16" else orc.f64_from_bf16
    rng = np.random.Generator(np.random.PCG64(7))
    top = 65504.0 if dtype == "fp16" else 3.3e38
    xs = list(rng.uniform(-1, 1, 3000) * np.exp2(rng.integers(-30 if dtype == "fp16" else -140,
                                                              16 if dtype == "fp16" else 127, 3000)))
    xs = [x for x in xs if abs(x) <= top]
    for x in xs:
        e = conv(x)
        v = decode(e)
        mag = e & 0x7FFF
        for nb in (mag - 1, mag + 1):
            if nb < 0 or nb >= (0x7C00 if dtype == "fp16" else 0x7F80):
                continue
            w = decode((e & 0x8000) | nb)
            assert abs(v - x) <= abs(w - x), (x, hex(e))
            if abs(v - x) == abs(w - x):
                assert mag % 2 == 0, (x, hex(e))


def test_encode_worked_ties():
    # bf16 (7 fraction bits): ties go to the even significand
    assert orc.bf16_from_f64(1 + 2 ** -8) == 0x3F80
    assert orc.bf16_from_f64(1 + 3 * 2 ** -8) == 0x3F82
    assert orc.bf16_from_f64(-(1 + 2 ** -8)) == 0xBF80
    # fp16 (10 fraction bits)
    assert orc.f16_from_f64(1 + 2 ** -11) == 0x3C00
    assert orc.f16_from_f64(1 + 3 * 2 ** -11) == 0x3C02
    assert orc.f16_from_f64(65504 + 15) == 0x7BFF
    assert orc.f16_from_f64(65504 + 16) == 0x7C00  # 65520 rounds up, out of range -> +Inf
    assert orc.f16_from_f64(-65520.0) == 0xFC00
    assert orc.f16_from_f64(2.0 ** -25) == 0x0000  # tie between 0 and the smallest subnormal
    assert orc.f16_from_f64(3 * 2.0 ** -25) == 0x0002
    assert orc.f16_from_f64(-0.0) == 0x8000
    assert orc.f16_from_f64(float("nan")) & 0x7C00 == 0x7C00 and orc.f16_from_f64(float("nan")) & 0x3FF


# ------------------------------------------------------------ the sum
@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_one_rank_is_passthrough(dtype):
    """One rank: the all-reduce returns its input unchanged ("All Reduce
    Plugin": passthrough for tpSize=1), bit for bit, signed zero, infinities
    and subnormals included."""
    tiny = {"fp32": 2.0 ** -149, "fp16": 2.0 ** -24, "bf16": 2.0 ** -133}[dtype]
    big = {"fp32": 3.4028234e38, "fp16": 65504.0, "bf16": 3.3895314e38}[dtype]
    vals = [0.0, -0.0, np.inf, -np.inf, tiny, -tiny, 3 * tiny, big, -big, 1.0, -2.5]
    p = np.concatenate([enc(vals, dtype), inputs.normal((1000,), 99, 0.0, 1.0, dtype)])
    assert np.array_equal(bits(osum(dtype, [p])), bits(p))
    pn = enc([np.nan, 1.0], dtype)
    assert np.isnan(dec(osum(dtype, [pn]), dtype)[0])


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", range(1, 9))
def test_sum_of_constants(dtype, ranks):
    for c in (0.375, -1.25, 3.0, 0.0):
        p = [enc(np.full(37, c), dtype) for _ in range(ranks)]
        assert np.array_equal(dec(osum(dtype, p), dtype), np.full(37, ranks * c))


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_integer_partials_exact_and_order_free(dtype):
    rng = np.random.Generator(np.random.PCG64(3))
    ints = rng.integers(-64, 65, size=(8, 513))
    p = [enc(ints[r], dtype) for r in range(8)]
    o = osum(dtype, p)
    # the fp32 sum of integers below 2^24 is exact in any order; the result is that
    # exact sum rounded once to the type (bf16 keeps 8 significant bits)
    assert np.array_equal(bits(o), bits(enc(ints.sum(axis=0), dtype)))
    for perm in ([7, 6, 5, 4, 3, 2, 1, 0], [3, 0, 6, 1, 7, 2, 5, 4]):
        assert np.array_equal(bits(osum(dtype, [p[i] for i in perm])), bits(o))


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", [2, 3, 8])
def test_sum_within_recursive_summation_bound(dtype, ranks):
    """|fl32 recursive sum - exact| <= (R-1) * 2^-24 * sum|P_r| (Higham,
    recursive summation), plus half a unit of the type for the final rounding."""
    w = inputs.random_sum(dtype, ranks, 4099, 40 + ranks)
    o = dec(osum(dtype, w.partials), dtype)
    P = np.stack([dec(p, dtype) for p in w.partials])
    exact = P.sum(axis=0)  # fp64 sums of <= 8 fp32-representable values of similar scale are exact enough
    bound = (ranks - 1) * 2.0 ** -24 * np.abs(P).sum(axis=0)
    half_ulp = np.array([0.5 * ulp_at(v, dtype) for v in o]) if dtype != "fp32" else 0.0
    assert np.all(np.abs(o - exact) <= bound + half_ulp + 1e-300)


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", [1, 2, 5, 8])
def test_sum_bitwise_equals_torch_sequential_fp32(dtype, ranks):
    """Library pin: torch CPU elementwise fp32 adds in rank order, then
    torch's round-to-nearest-even cast."""
    w = inputs.random_sum(dtype, ranks, 2053, 60 + ranks)
    tt = {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]
    tp = [torch.from_numpy(p.view(np.int16) if dtype == "bf16" else p) for p in w.partials]
    if dtype == "bf16":
        tp = [t.view(torch.bfloat16) for t in tp]
    ref = functools.reduce(torch.add, [t.float() for t in tp]).to(tt)
    ref_bits = ref.view(torch.int16 if dtype != "fp32" else torch.int32).numpy()
    assert np.array_equal(bits(osum(dtype, w.partials)), ref_bits.view(bits(ref_bits).dtype))


def test_sum_accumulates_in_fp32_in_rank_order():
    # fp32: 1 + 2^-24 is a tie and rounds to 1, twice; the other order gives 1 + 2^-23
    t = 2.0 ** -24
    a = osum("fp32", [enc([1.0], "fp32"), enc([t], "fp32"), enc([t], "fp32")])
    b = osum("fp32", [enc([t], "fp32"), enc([t], "fp32"), enc([1.0], "fp32")])
    assert dec(a, "fp32")[0] == 1.0
    assert dec(b, "fp32")[0] == 1.0 + 2.0 ** -23
    # bf16: three 2^-9 on top of 1 are kept in fp32 (1 + 3*2^-9) and rounded once to 1 + 2^-7;
    # rounding to bf16 after each add would leave 1
    q = 2.0 ** -9
    c = osum("bf16", [enc([1.0], "bf16")] + [enc([q], "bf16")] * 3)
    assert dec(c, "bf16")[0] == 1.0 + 2.0 ** -7
    # fp16 range: 65504 + 16 = 65520 -> +Inf; 65504 + 15 -> 65504
    assert dec(osum("fp16", [enc([65504.0], "fp16"), enc([16.0], "fp16")]), "fp16")[0] == np.inf
    assert dec(osum("fp16", [enc([65504.0], "fp16"), enc([15.0], "fp16")]), "fp16")[0] == 65504.0


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_starts_from_rank0_value(dtype):
    """-0 + -0 = -0; an accumulator started at +0 would give +0."""
    o = osum(dtype, [enc([-0.0], dtype), enc([-0.0], dtype)])
    assert np.signbit(dec(o, dtype)[0]) and dec(o, dtype)[0] == 0.0


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_special_values(dtype):
    p0 = enc([np.inf, np.inf, np.nan, 1.0, -np.inf], dtype)
    p1 = enc([-np.inf, 1.0, 1.0, np.nan, -1.0], dtype)
    o = dec(osum(dtype, [p0, p1]), dtype)
    assert np.isnan(o[0]) and o[1] == np.inf and np.isnan(o[2]) and np.isnan(o[3]) and o[4] == -np.inf


def test_sum_fp32_subnormals_kept():
    s = 2.0 ** -149
    o = osum("fp32", [enc([s, 3 * s, 2.0 ** -126], "fp32"), enc([s, -s, -s], "fp32")])
    assert list(dec(o, "fp32")) == [2 * s, 2 * s, 2.0 ** -126 - s]


@pytest.mark.parametrize("dtype", DTYPES)
def test_sum_in_place_and_empty(dtype):
    w = inputs.random_sum(dtype, 3, 300, 5)
    ref = osum(dtype, w.partials)
    p0 = w.partials[0].copy()
    orc.ar_sum(dtype, [p0, w.partials[1], w.partials[2]], p0)
    assert np.array_equal(bits(p0), bits(ref))
    orc.ar_sum(dtype, [empty(0, dtype)], empty(0, dtype))


# ------------------------------------------------------------- RMSNorm
@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_exact_closed_form(dtype):
    """S = [5,-2,1,-1,1,0,0,0]: sum of squares 32, mean 4, rstd 1/2 exactly,
    so y = S/2 * W is exact in every type."""
    S = enc([5, -2, 1, -1, 1, 0, 0, 0], dtype)
    W = enc([1, 0.5, 2, -1, 1, 1, 1, 1], dtype)
    out = onorm(dtype, S, W, 0.0, 8)
    assert list(dec(out, dtype)) == [2.5, -0.5, 1.0, 0.5, 0.5, 0.0, 0.0, 0.0]


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_eps_inside_root_and_divisor_is_hidden(dtype):
    """S = [3,4]: mean of squares 25/2 (divisor H, not H-1); + eps 3.5 = 16;
    rstd = 1/4 exactly -> y = [0.75, 1]. eps outside the root, or H-1, or
    no eps, all give other values."""
    out = onorm(dtype, enc([3, 4], dtype), enc([1, 1], dtype), 3.5, 2)
    assert list(dec(out, dtype)) == [0.75, 1.0]
    out2 = onorm(dtype, enc([3, 4, 3, 4], dtype), enc([1, 2], dtype), 3.5, 2)  # two rows, weight per column
    assert list(dec(out2, dtype)) == [0.75, 2.0, 0.75, 2.0]


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_irrational_within_half_ulp(dtype):
    """S = [1,2,3,4], W = 1, eps = 0: y = S / sqrt(7.5); correctly rounded."""
    out = dec(onorm(dtype, enc([1, 2, 3, 4], dtype), enc([1, 1, 1, 1], dtype), 0.0, 4), dtype)
    for s, y in zip([1, 2, 3, 4], out):
        exact = s / math.sqrt(7.5)
        assert abs(y - exact) <= 0.5 * ulp_at(exact, dtype)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_unit_rms_after_norm(dtype):
    """With W = 1: sqrt(mean(y^2)) = sqrt(ms / (ms + eps)) ~ 1."""
    H, rows, eps = 1024, 6, 1e-5
    x = inputs.normal((rows * H,), 17, 0.0, 1.0, dtype)
    out = dec(onorm(dtype, x, enc(np.ones(H), dtype), eps, H), dtype).reshape(rows, H)
    X = dec(x, dtype).reshape(rows, H)
    ms = (X ** 2).mean(axis=1)
    rms_out = np.sqrt((out ** 2).mean(axis=1))
    rel = {"fp32": 1e-6, "fp16": 2.0 ** -10, "bf16": 2.0 ** -7}[dtype]
    assert np.all(np.abs(rms_out - np.sqrt(ms / (ms + eps))) <= rel)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_power_of_two_scale_invariance(dtype):
    H = 96
    x = inputs.normal((2 * H,), 21, 0.0, 1.0, dtype)
    W = inputs.normal((H,), 22, 1.0, 0.1, dtype)
    base = bits(onorm(dtype, x, W, 0.0, H))
    for k in (-3, -1, 2, 5):
        xs = enc(dec(x, dtype) * 2.0 ** k, dtype)  # exact scaling
        assert np.array_equal(bits(onorm(dtype, xs, W, 0.0, H)), base)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_special_rows(dtype):
    H = 64
    W = inputs.normal((H,), 31, 1.0, 0.1, dtype)
    Wd = dec(W, dtype)
    # constant row c with eps = 0: y = sign(c) * W
    out = dec(onorm(dtype, enc(np.full(H, -0.75), dtype), W, 0.0, H), dtype)
    assert np.array_equal(out, -Wd)
    # zero row with eps > 0: y = 0
    out = dec(onorm(dtype, enc(np.zeros(H), dtype), W, 1e-6, H), dtype)
    assert np.all(out == 0.0)
    # one nonzero x, eps = 0: y = sign(x) * sqrt(H) * W there (sqrt(64) = 8, exact), 0 elsewhere
    row = np.zeros(H)
    row[13] = -2.5
    out = dec(onorm(dtype, enc(row, dtype), W, 0.0, H), dtype)
    expect = np.zeros(H)
    expect[13] = dec(enc([-8.0 * Wd[13]], dtype), dtype)[0]
    assert np.array_equal(out, expect)


@pytest.mark.parametrize("dtype", DTYPES)
def test_rmsnorm_vs_torch_rms_norm_fp64(dtype):
    """Library pin: torch.nn.functional.rms_norm in fp64, rounded to the type
    (torch rounds fp64 -> bf16 through fp32, so allow one unit at ties)."""
    H, rows, eps = 320, 5, 1e-5
    x = inputs.normal((rows * H,), 41, 0.0, 1.0, dtype)
    W = inputs.normal((H,), 42, 1.0, 0.1, dtype)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(dec(x, dtype)).view(rows, H), (H,),
                                       torch.from_numpy(dec(W, dtype)), eps).numpy().ravel()
    got = dec(onorm(dtype, x, W, eps, H), dtype)
    err = np.abs(got - ref)
    tol = np.array([ulp_at(v, dtype) for v in ref]) * (0.5 if dtype == "fp32" else 1.0)
    assert np.all(err <= tol)


# ---------------------------------------------------------- fused op
@pytest.mark.parametrize("dtype", DTYPES)
def test_fused_bias_added_once_per_column(dtype):
    """Zero partials on 8 ranks and a bias b: S = b (the GEMM bias is added
    once, not once per rank), broadcast over rows by column index."""
    H, rows = 16, 3
    b = enc(np.arange(H) * 0.25 - 2.0, dtype)
    parts = [enc(np.zeros(rows * H), dtype) for _ in range(8)]
    W = enc(np.ones(H), dtype)
    out, inter = ofused(dtype, parts, H, W, 1e-6, bias=b)
    assert np.array_equal(dec(inter, dtype), np.tile(dec(b, dtype), rows))
    assert np.array_equal(bits(out), bits(onorm(dtype, inter, W, 1e-6, H)))


@pytest.mark.parametrize("dtype", DTYPES)
def test_fused_terms_and_indices_exact(dtype):
    """Small dyadic values make every add exact, so S must equal
    sum_r P_r[t,h] + B[h] + Q[t,h] exactly: catches a dropped term, a term
    counted twice, a bias indexed by row, a residual indexed by column."""
    H, rows, R = 8, 3, 3
    rng = np.random.Generator(np.random.PCG64(77))
    P = rng.integers(-8, 9, size=(R, rows * H)) * 0.25
    B = rng.integers(-8, 9, size=H) * 0.5
    Q = rng.integers(-16, 17, size=rows * H) * 0.125
    parts = [enc(P[r], dtype) for r in range(R)]
    W = enc(np.ones(H), dtype)
    out, inter = ofused(dtype, parts, H, W, 0.0, bias=enc(B, dtype), residual=enc(Q, dtype))
    expect = P.sum(axis=0) + np.tile(B, rows) + Q
    assert np.array_equal(dec(inter, dtype), expect)
    # without residual / without bias
    _, i2 = ofused(dtype, parts, H, W, 0.0, bias=enc(B, dtype))
    assert np.array_equal(dec(i2, dtype), P.sum(axis=0) + np.tile(B, rows))
    _, i3 = ofused(dtype, parts, H, W, 0.0, residual=enc(Q, dtype))
    assert np.array_equal(dec(i3, dtype), P.sum(axis=0) + Q)


def test_fused_order_of_adds():
    """((sum over ranks) + bias) + residual, in fp32."""
    t = 2.0 ** -24
    W, f = enc([1.0], "fp32"), "fp32"
    # bias after the residual would give 2^-24; bias before: (1 + 2^-24) = 1, then 1 - 1 = 0
    _, s = ofused(f, [enc([1.0], f)], 1, W, 1.0, bias=enc([t], f), residual=enc([-1.0], f))
    assert dec(s, f)[0] == 0.0
    # bias after the whole rank sum: (1 - 1) + 2^-24; bias folded into rank 0 would give 0
    _, s = ofused(f, [enc([1.0], f), enc([-1.0], f)], 1, W, 1.0, bias=enc([t], f))
    assert dec(s, f)[0] == t


def test_fused_norm_reads_the_rounded_sum():
    """fp16, three ranks: P0 + P1 + P2 = 5 + 2^-9 in fp32, a tie that rounds
    to S = 5 in fp16. Normalizing S = [5,-2,1,-1,1,0,0,0] gives exactly
    [2.5,-1,0.5,-0.5,0.5,0,0,0]; normalizing the unrounded 5 + 2^-9 would make
    the second output -0.99951171875 instead of -1."""
    d = "fp16"
    P0 = enc([4, -2, 1, -1, 1, 0, 0, 0], d)
    P1 = enc([1, 0, 0, 0, 0, 0, 0, 0], d)
    P2 = enc([2.0 ** -9, 0, 0, 0, 0, 0, 0, 0], d)
    out, inter = ofused(d, [P0, P1, P2], 8, enc(np.ones(8), d), 0.0)
    assert list(dec(inter, d)) == [5, -2, 1, -1, 1, 0, 0, 0]
    assert list(dec(out, d)) == [2.5, -1, 0.5, -0.5, 0.5, 0, 0, 0]
    s0 = 5 + 2.0 ** -9  # precondition: the other reading really differs
    alt = -2 / math.sqrt((s0 * s0 + 7) / 8)
    assert dec(enc([alt], d), d)[0] != -1.0


@pytest.mark.parametrize("dtype", DTYPES)
@pytest.mark.parametrize("ranks", [1, 2, 8])
def test_fused_equals_sum_then_norm_without_bias_residual(dtype, ranks):
    """"allreduce.d2": the fused branch and the unfused branch (all-reduce,
    then rms_norm_kernel) compute the same function, bit for bit here."""
    w = inputs.random_fused(dtype, ranks, 4, 256, 90 + ranks, bias=False, residual=False)
    out, inter = ofused(dtype, w.partials, w.hidden, w.weight, w.eps)
    s = osum(dtype, w.partials)
    assert np.array_equal(bits(inter), bits(s))
    assert np.array_equal(bits(out), bits(onorm(dtype, s, w.weight, w.eps, w.hidden)))


@pytest.mark.parametrize("dtype", DTYPES)
def test_fused_intermediate_may_alias_residual(dtype):
    w = inputs.random_fused(dtype, 4, 3, 128, 123)
    out, inter = ofused(dtype, w.partials, w.hidden, w.weight, w.eps, bias=w.bias, residual=w.residual)
    q = w.residual.copy()
    out2 = empty(w.n, dtype)
    orc.ar_residual_rmsnorm(dtype, w.partials, w.hidden, w.weight, w.eps, out2, q, bias=w.bias, residual=q)
    assert np.array_equal(bits(q), bits(inter)) and np.array_equal(bits(out2), bits(out))


def test_fused_rejects_ragged_rows():
    p = [enc(np.ones(10), "fp32")]
    with pytest.raises(ValueError):
        ofused("fp32", p, 3, enc(np.ones(3), "fp32"), 0.0)


# ------------------------------------------------------------- golden
def _digest(a):
    return hashlib.sha256(bits(a).tobytes()).hexdigest()


def test_oracle_reproduces_golden_digests():
    """Regression pin: tests/golden/oracle_small.json was written by
    tests/golden/make_golden.py, which calls only the oracle. A change in the
    oracle's arithmetic shows up here."""
    with open(GOLDEN) as f:
        gold = json.load(f)
    for name, g in gold["workloads"].items():
        w = inputs.make(name)
        if w.op == "sum":
            out = osum(w.dtype, w.partials)
            assert _digest(out) == g["out_sha256"], name
        else:
            out, inter = ofused(w.dtype, w.partials, w.hidden, w.weight, w.eps, bias=w.bias, residual=w.residual)
            assert _digest(out) == g["out_sha256"], name
            assert _digest(inter) == g["intermediate_sha256"], name
        for i, hx in g["out_samples"]:
            assert int(bits(out)[i]) == int(hx, 16), (name, i)
