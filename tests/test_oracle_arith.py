"""Pins for the oracle's per-hop arithmetic (CPU only).

The rounding helpers are checked against torch's own CPU conversions (a library
routine with IEEE round-to-nearest-even semantics) and against exact integer or
float64 arithmetic, never against themselves.
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.arith import add_rounded, bf16_bits_to_f32, f32_to_bf16_bits


def _torch_bf16_bits(x_f32):
    t = torch.from_numpy(np.asarray(x_f32, np.float32).copy())
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_matches_torch_random():
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, 200_000, dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32)
    x = x[np.isfinite(x)]
    assert np.array_equal(f32_to_bf16_bits(x), _torch_bf16_bits(x))


def test_bf16_round_ties_to_even():
    # low 16 bits exactly 0x8000 -> a tie; kept part even stays, odd goes up
    hi = np.arange(0, 0x7F7F, 37, dtype=np.uint32)
    for sign in (0, 0x8000):
        u = ((hi | sign) << 16) | 0x8000
        x = u.view(np.float32)
        got = f32_to_bf16_bits(x)
        want = np.where(hi & 1, (hi | sign) + 1, hi | sign).astype(np.uint16)
        assert np.array_equal(got, want)
        assert np.array_equal(got, _torch_bf16_bits(x))


def test_bf16_round_edges():
    vals = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, -3.4028235e38,
                     1e-45, -1e-45, 1.1754942e-38, 65504.0, 1.0 + 2**-8,
                     1.0 + 3 * 2**-9], dtype=np.float32)
    assert np.array_equal(f32_to_bf16_bits(vals), _torch_bf16_bits(vals))
    # largest float32 rounds past the largest bf16 -> infinity
    assert f32_to_bf16_bits(np.array([3.4028235e38], np.float32))[0] == 0x7F80
    nan_bits = f32_to_bf16_bits(np.array([np.nan], np.float32))[0]
    assert (nan_bits & 0x7F80) == 0x7F80 and (nan_bits & 0x7F) != 0


def test_bf16_widen_is_exact():
    bits = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    got = bf16_bits_to_f32(bits)
    t = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).float().numpy()
    fin = np.isfinite(t)
    assert np.array_equal(got[fin].view(np.uint32), t[fin].view(np.uint32))


def test_int32_add_wraps():
    a = np.array([2**31 - 1, -2**31, 5, -7, 2**30], np.int32)
    b = np.array([1, -1, -5, 7, 2**30], np.int32)
    got = add_rounded(a, b, "int32")
    want = [((int(x) + int(y) + 2**31) % 2**32) - 2**31 for x, y in zip(a, b)]
    assert got.dtype == np.int32 and got.tolist() == want


def test_fp32_add_is_correctly_rounded():
    # the exact sum of two binary32 values rounded once to binary32 equals the
    # binary64 sum rounded to binary32 (double rounding is harmless because
    # 53 >= 2*24 + 2), so a float64 detour is an independent check
    rng = np.random.default_rng(5)
    a = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-20, 20, 100_000)).astype(np.float32)
    b = (rng.standard_normal(100_000) * 10.0 ** rng.integers(-20, 20, 100_000)).astype(np.float32)
    want = (a.astype(np.float64) + b.astype(np.float64)).astype(np.float32)
    got = add_rounded(a, b, "float32")
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


def test_bf16_add_is_correctly_rounded():
    # exact sum of two bf16 values, rounded to binary64 (harmless, 53 >= 2*8+2)
    # and then to bf16 by torch (via binary32: harmless again), must equal the
    # oracle's binary32-add-then-round path
    rng = np.random.default_rng(6)
    a = _torch_bf16_bits(rng.standard_normal(100_000).astype(np.float32)
                         * np.float32(2.0) ** rng.integers(-30, 30, 100_000).astype(np.float32))
    b = _torch_bf16_bits(rng.standard_normal(100_000).astype(np.float32)
                         * np.float32(2.0) ** rng.integers(-30, 30, 100_000).astype(np.float32))
    exact = bf16_bits_to_f32(a).astype(np.float64) + bf16_bits_to_f32(b).astype(np.float64)
    want = torch.from_numpy(exact).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = add_rounded(a, b, "bfloat16")
    assert np.array_equal(got, want)


def test_bf16_add_tie_case_by_hand():
    # 1 + 2**-8 sits exactly halfway between the bf16 neighbours 1 and 1 + 2**-7;
    # ties go to the even one, 1.0 (0x3F80)
    one = f32_to_bf16_bits(np.array([1.0], np.float32))
    half_ulp = f32_to_bf16_bits(np.array([2.0**-8], np.float32))
    assert add_rounded(one, half_ulp, "bfloat16")[0] == 0x3F80
    # 1 + 2**-7 + 2**-8 ties between 1 + 2**-7 (odd) and 1 + 2**-6 (even)
    a = f32_to_bf16_bits(np.array([1.0 + 2.0**-7], np.float32))
    assert add_rounded(a, half_ulp, "bfloat16")[0] == 0x3F82


def test_as_values():
    assert oracle.as_values(np.array([3], np.int32), "int32").dtype == np.int64
    bits = f32_to_bf16_bits(np.array([1.5, -2.0], np.float32))
    assert oracle.as_values(bits, "bfloat16").tolist() == [1.5, -2.0]


# ------------------------------------------------------------ subnormals

from fractions import Fraction

# (precision in bits including the leading one, smallest normal exponent)
_FORMATS = {"float32": (24, -126), "bfloat16": (8, -126), "float16": (11, -14),
            "float64": (53, -1022)}


def _round_exact(v, dtype):
    """The IEEE binary value nearest to the rational v, ties to even, with
    gradual underflow: the spacing below 2**emin stays that of the smallest
    binade.  Written from the format's definition, not from numpy."""
    prec, emin = _FORMATS[dtype]
    if v == 0:
        return Fraction(0)
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()   # within one of floor(log2 a)
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    e = max(e, emin)
    q = Fraction(2) ** (e - (prec - 1))          # spacing of representable values here
    m = a / q
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    r = lo * q
    return r if v > 0 else -r


def _values(bits, dtype):
    return [Fraction(float(x)) for x in oracle.as_values(bits, dtype)]


@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "float16", "float64"])
def test_add_rounded_with_subnormals_matches_exact_rounding(dtype):
    """Sums of subnormal and near-subnormal operands: the oracle's hop equals the
    exact sum rounded once, so no operand or result is flushed to zero."""
    prec, emin = _FORMATS[dtype]
    rng = np.random.default_rng(prec)
    tiny = 2.0 ** (emin - prec + 1)              # smallest subnormal
    k = rng.integers(-3 * 2 ** (prec - 1), 3 * 2 ** (prec - 1), (2, 1500))
    # multiples of the smallest subnormal (subnormal and just-normal values),
    # and products with odd numbers that need rounding when they are normal
    raw = np.concatenate([k * tiny, (2 * k + 1) * tiny * rng.integers(1, 9, (2, 1500))], axis=1)
    if dtype == "bfloat16":
        a = f32_to_bf16_bits(raw[0].astype(np.float32))
        b = f32_to_bf16_bits(raw[1].astype(np.float32))
    else:
        t = oracle.arith.STORAGE[dtype]
        a, b = raw[0].astype(t), raw[1].astype(t)
    got = add_rounded(a, b, dtype)
    va, vb, vg = _values(a, dtype), _values(b, dtype), _values(got, dtype)
    subnormal_results = 0
    for x, y, g in zip(va, vb, vg):
        want = _round_exact(x + y, dtype)
        assert g == want, (dtype, x, y, g, want)
        subnormal_results += 0 < abs(want) < Fraction(2) ** emin
    assert subnormal_results > 500
