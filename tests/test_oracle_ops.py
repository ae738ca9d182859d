"""Pins for the oracle's extra element types and reductions (CPU only).

* Rounding of sums, pre-divided quotients and wide-to-narrow conversions is
  checked against a first-principles rounder: the exact rational result
  (``fractions.Fraction``) rounded to nearest, ties to even, in the target
  format's precision and exponent range.  It shares nothing with the oracle.
* int64 wrapping against Python integers modulo 2**64.
* max against ``numpy.maximum`` (a library routine) away from signed-zero ties,
  and hand cases for +-0 and NaN.
* Ring-order sensitivity, pre-division and wide accumulation on hand-derived
  cases whose results are worked out in the comments.
"""

import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import arith
from ring_all_reduce_schedule_amd import inputs

# (significand bits incl. the implicit one, exponent of the smallest normal, largest exponent)
FORMATS = {"float16": (11, -14, 15), "bfloat16": (8, -126, 127),
           "float32": (24, -126, 127), "float64": (53, -1022, 1023)}


def round_to_format(x, fmt):
    """Exact rational x rounded to nearest even in ``fmt``; +-inf on overflow."""
    q, emin, emax = FORMATS[fmt]
    if x == 0:
        return 0.0
    sign = -1 if x < 0 else 1
    a = abs(Fraction(x))
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, emin)                        # below the normals the quantum is fixed
    quantum = Fraction(2) ** (e - q + 1)
    m = a / quantum
    fl = math.floor(m)
    r = m - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    res = fl * quantum
    if res >= Fraction(2) ** (emax + 1):
        return sign * math.inf
    return sign * float(res)


def random_values(dtype, n, seed, scale_exp=8):
    """Finite values of ``dtype`` spread over a band of exponents, as stored elements."""
    rng = np.random.default_rng(seed)
    v = rng.standard_normal(n) * np.exp2(rng.integers(-scale_exp, scale_exp, n))
    if dtype == "bfloat16":
        return arith.f32_to_bf16_bits(v.astype(np.float32))
    return v.astype(arith.STORAGE[dtype])


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32", "float64"])
def test_add_rounds_the_exact_sum_once(dtype):
    a = random_values(dtype, 1500, 1)
    b = random_values(dtype, 1500, 2)
    got = arith.as_values(arith.add_rounded(a, b, dtype), dtype)
    va, vb = arith.as_values(a, dtype), arith.as_values(b, dtype)
    for g, x, y in zip(got, va, vb):
        assert g == round_to_format(Fraction(x) + Fraction(y), dtype)


def test_float16_add_edges_and_torch():
    # 2048 + 1: halfway between 2048 and 2050 -> even 2048; 2048 + 3 -> 2052;
    # 65504 + 16: halfway between the largest half and 2^16 -> rounds to inf
    a = np.array([2048, 2048, 65504, -65504, 1e-7, 0.0], np.float16)
    b = np.array([1, 3, 16, -16, 1e-7, -0.0], np.float16)
    got = arith.add_rounded(a, b, "float16")
    assert got[0] == 2048 and got[1] == 2052 and got[2] == np.inf and got[3] == -np.inf
    t = (torch.from_numpy(a) + torch.from_numpy(b)).numpy()
    assert np.array_equal(got.view(np.uint16), t.view(np.uint16))
    x = random_values("float16", 20000, 3)
    y = random_values("float16", 20000, 4)
    t = (torch.from_numpy(x) + torch.from_numpy(y)).numpy()
    assert np.array_equal(arith.add_rounded(x, y, "float16").view(np.uint16), t.view(np.uint16))


def test_int64_wraps_modulo_2_64():
    rng = np.random.default_rng(5)
    a = rng.integers(-2**63, 2**63, 2000, dtype=np.int64)
    b = rng.integers(-2**63, 2**63, 2000, dtype=np.int64)
    got = arith.add_rounded(a, b, "int64")
    for g, x, y in zip(got, a, b):
        w = (int(x) + int(y)) % 2**64
        assert int(g) == (w - 2**64 if w >= 2**63 else w)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32", "float64"])
@pytest.mark.parametrize("p", [2, 3, 7, 9, 64])
def test_pre_divide_rounds_the_exact_quotient(dtype, p):
    x = random_values(dtype, 600, p)
    got = arith.as_values(arith.pre_divide(x, dtype, p), dtype)
    for g, v in zip(got, arith.as_values(x, dtype)):
        assert g == round_to_format(Fraction(v) / p, dtype)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
def test_wide_terms_and_narrowing(dtype):
    wide = arith.WIDE[dtype]
    x = random_values(dtype, 600, 9)
    vals = arith.as_values(x, dtype)
    # widening is exact
    assert np.array_equal(arith.widen(x, dtype).astype(np.float64), vals)
    # an average's wide term: the exact quotient rounded once to the wide type
    for p in (3, 9):
        got = arith.wide_term(x, dtype, "avg", p).astype(np.float64)
        for g, v in zip(got, vals):
            assert g == round_to_format(Fraction(v) / p, wide)
    # narrowing a wide value rounds it once to the element type
    w = random_values(wide, 600, 10, scale_exp=4)
    got = arith.as_values(arith.narrow(w, dtype), dtype)
    for g, v in zip(got, np.asarray(w, np.float64)):
        assert g == round_to_format(Fraction(float(v)), dtype)


@pytest.mark.parametrize("dtype", ["int32", "int64", "float16", "bfloat16", "float32", "float64"])
def test_max_matches_numpy_maximum(dtype):
    if dtype in ("int32", "int64"):
        rng = np.random.default_rng(12)
        info = np.iinfo(arith.STORAGE[dtype])
        a = rng.integers(info.min, info.max, 5000, dtype=arith.STORAGE[dtype])
        b = rng.integers(info.min, info.max, 5000, dtype=arith.STORAGE[dtype])
        assert np.array_equal(arith.max_exact(a, b, dtype), np.maximum(a, b))
        return
    a = random_values(dtype, 5000, 13)
    b = random_values(dtype, 5000, 14)
    va, vb = arith.as_values(a, dtype), arith.as_values(b, dtype)
    keep = (va != 0) | (vb != 0)
    got = arith.as_values(arith.max_exact(a, b, dtype), dtype)
    assert np.array_equal(got[keep], np.maximum(va, vb)[keep])


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32", "float64"])
def test_max_signed_zero_and_nan(dtype):
    bits = arith.BITS[dtype]
    sign = int(bits(1) << bits(8 * arith.ITEMSIZE[dtype] - 1))
    if dtype == "bfloat16":
        pz, nz = np.array([0], np.uint16), np.array([sign], np.uint16)
        one = arith.f32_to_bf16_bits(np.array([1.0], np.float32))
        nan = np.array([0x7FC1], np.uint16)
    else:
        t = arith.STORAGE[dtype]
        pz, nz, one = np.array([0.0], t), np.array([-0.0], t), np.array([1.0], t)
        nan = np.array([np.nan], t)
    for a, b in ((pz, nz), (nz, pz)):
        assert int(arith.max_exact(a, b, dtype).view(bits)[0]) == 0       # +0 either way
    for a, b in ((nan, one), (one, nan)):
        assert int(arith.max_exact(a, b, dtype).view(bits)[0]) == arith.QNAN[dtype]


def test_float64_ring_order_matters():
    # chunk 0 of p = 3, N = 3 starts at rank 0: (1e16 + 1) + 1 -> 1e16 (each +1 is a
    # tie at ulp 2, kept at the even 1e16); chunk 1 starts at rank 1: (1 + 1) + 1e16
    # is exactly 1e16 + 2
    xs = [np.array([1e16, 1e16, 1e16]), np.array([1.0, 1.0, 1.0]), np.array([1.0, 1.0, 1.0])]
    got = oracle.ring_fold(xs, "float64")
    assert got[0] == 1e16 and got[1] == 1e16 + 2
    final, _, _ = oracle.ring_allreduce(xs, "float64")
    assert all(np.array_equal(f, got) for f in final)


def test_wide_accumulation_keeps_what_per_hop_rounding_drops():
    # p = 64, bf16, one element: 256 then 63 ones (rank 0 leads chunk 0).  Per hop,
    # 256 + 1 = 257 is a tie between 256 and 258 and stays at the even 256, so the
    # ring gives 256.  Accumulated in float32 the sum is 319 exactly; rounded once
    # to bf16 (spacing 2 from 256 to 512) 319 is a tie between 318 and 320 and
    # goes to the even significand, 320.
    p = 64
    xs = [arith.f32_to_bf16_bits(np.array([256.0 if r == 0 else 1.0], np.float32)) for r in range(p)]
    per_hop = arith.as_values(oracle.ring_fold(xs, "bfloat16"), "bfloat16")
    wide = arith.as_values(oracle.ring_fold(xs, "bfloat16", wide=True), "bfloat16")
    assert per_hop[0] == 256.0 and wide[0] == 320.0


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
def test_wide_max_is_the_exact_max(dtype):
    xs = inputs.make_inputs(5, 333, dtype, seed=3, sigma=3.0)
    a = oracle.ring_fold(xs, dtype, op="max", wide=True)
    b = oracle.ring_fold(xs, dtype, op="max")
    assert np.array_equal(a.view(arith.BITS[dtype]), b.view(arith.BITS[dtype]))
    v = np.max(np.stack([arith.as_values(x, dtype) for x in xs]), axis=0)
    assert np.array_equal(arith.as_values(a, dtype), v)


def test_pre_divide_prevents_float16_overflow():
    # p = 8 ranks of 8192: the sum 65536 overflows float16 (largest 65504), the
    # average of pre-divided terms (1024 each, summed exactly) is 8192
    xs = [np.full(8, 8192.0, np.float16) for _ in range(8)]
    assert np.all(np.isinf(oracle.ring_fold(xs, "float16")))
    assert np.all(oracle.ring_fold(xs, "float16", op="avg") == 8192.0)
    assert np.all(oracle.ring_fold(xs, "float16", wide=True) == np.inf)   # 65536 > 65504
    assert np.all(oracle.ring_fold(xs, "float16", op="avg", wide=True) == 8192.0)


# avg is defined for floating-point types only
DTYPE_OPS = [(d, o) for d in ("int32", "int64", "float16", "bfloat16", "float32", "float64")
             for o in ("sum", "max", "avg") if o != "avg" or d not in ("int32", "int64")]


@pytest.mark.parametrize("dtype,op", DTYPE_OPS)
@pytest.mark.parametrize("p,n", [(2, 9), (3, 10), (4, 33), (9, 1003), (16, 257)])
def test_simulator_matches_closed_form_all_ops(dtype, op, p, n):
    xs = inputs.make_inputs(p, n, dtype, seed=p * 7 + n, sigma=3.0)
    for d in (1, -1):
        final, after_rs, _ = oracle.ring_allreduce(xs, dtype, direction=d, op=op)
        fold = oracle.ring_fold(xs, dtype, direction=d, op=op)
        for r in range(p):
            assert np.array_equal(final[r].view(arith.BITS[dtype]), fold.view(arith.BITS[dtype]))
            part = oracle.rs_partial(xs, dtype, r, d, op=op)
            assert np.array_equal(after_rs[r].view(arith.BITS[dtype]), part.view(arith.BITS[dtype]))


@pytest.mark.parametrize("dtype", ["int32", "int64"])
@pytest.mark.parametrize("p,n", [(2, 5), (5, 17), (9, 100)])
def test_integer_sum_and_max_brute_force(dtype, p, n):
    t = arith.STORAGE[dtype]
    info = np.iinfo(t)
    rng = np.random.default_rng(p + n)
    xs = [rng.integers(info.min, info.max, n, dtype=t) for _ in range(p)]
    bits = 8 * arith.ITEMSIZE[dtype]
    want = []
    for i in range(n):
        w = sum(int(x[i]) for x in xs) % 2**bits
        want.append(w - 2**bits if w >= 2**(bits - 1) else w)
    assert oracle.ring_fold(xs, dtype).tolist() == want
    assert oracle.tree_allreduce(xs, dtype)[0][0].tolist() == want
    mx = [max(int(x[i]) for x in xs) for i in range(n)]
    assert oracle.ring_fold(xs, dtype, op="max").tolist() == mx
    assert oracle.tree_allreduce(xs, dtype, op="max")[0][0].tolist() == mx


def test_avg_small_integers_exact():
    # p = 4, values 4, 8, 12, 16: quarters 1, 2, 3, 4 are exact and sum to 10
    xs = [np.full(6, v, np.float32) for v in (4.0, 8.0, 12.0, 16.0)]
    for dtype in ("float16", "float32", "float64", "bfloat16"):
        ys = ([arith.f32_to_bf16_bits(x) for x in xs] if dtype == "bfloat16"
              else [x.astype(arith.STORAGE[dtype]) for x in xs])
        for f in (oracle.ring_fold(ys, dtype, op="avg"),
                  oracle.tree_allreduce(ys, dtype, op="avg")[0][0],
                  oracle.bidir_allreduce(ys, dtype, op="avg")[0][0]):
            assert np.all(arith.as_values(f, dtype) == 10.0)
