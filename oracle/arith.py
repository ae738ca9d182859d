"""Per-hop addition, rounded to the buffer's element type (oracle; test infrastructure only).

Which precision each hop uses: [InDepth] "An implementation" accumulates every
hop of the torch ring with an in-place add on the tensor itself, i.e. in the
tensor's own dtype, and [Derive] "What interviewers probe next" notes that the
library's default accumulation type is the buffers' own.  So every hop of the
ring rounds its sum back to the element type of the buffers:

* int32    -- two's-complement sum, wrapped modulo 2**32 (the pages are silent
              on overflow; wrapping is what an in-place int32 add does);
* float32  -- IEEE-754 binary32 addition, round to nearest even;
* bfloat16 -- both operands widened exactly to binary32, added there (round to
              nearest even), then narrowed to bfloat16 (round to nearest even).
              The detour through binary32 changes nothing: double rounding is
              harmless for the sum of two values of precision q when the
              intermediate precision is at least 2q + 2 (Figueroa, "When is
              double rounding innocuous?", SIGNUM Newsletter 30(3), 1995);
              here q = 8 and the intermediate has 24 bits.

* float16  -- IEEE-754 binary16; the exact sum rounded once to nearest even
              (numpy adds two halves in binary32 and rounds back, which is the
              same by the rule above: q = 11, 24 >= 24);
* float64  -- IEEE-754 binary64 addition, round to nearest even;
* int64    -- two's-complement sum wrapped modulo 2**64.

bfloat16 values are carried as uint16 bit patterns.

Other reductions ([Deepinsea] "AllReduce 语义": sum, average, maximum):

* max      -- the larger operand, exactly (no rounding is involved).  Floats:
              a NaN operand gives the type's canonical quiet NaN, and +0 counts
              as larger than -0 (IEEE 754-2019 maximum), so the result does not
              depend on the order of the operands.
* avg      -- [InDepth] "Failure modes": fp16 sums over many ranks can
              overflow, so divide before summing.  Every rank's contribution
              enters the sum as x / p rounded to the element type (floats only);
              the divided values are then summed exactly as for "sum".
              The quotient here is formed in binary64 and narrowed once more;
              both roundings are harmless by the rule above (53 >= 2*24 + 2).
* wide     -- [InDepth] "Failure modes": accumulate in a wider type.
              bfloat16 and float16 accumulate in binary32, float32 in binary64:
              every term is widened exactly, every hop rounds to the wide type,
              and the final sum is rounded once to the element type.

"""

import numpy as np

DTYPES = ("int32", "float32", "bfloat16", "float16", "float64", "int64")
FLOATS = ("float32", "bfloat16", "float16", "float64")
OPS = ("sum", "max", "avg")

# numpy storage type of each element type
STORAGE = {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16,
           "float16": np.float16, "float64": np.float64, "int64": np.int64}

# bytes per element
ITEMSIZE = {"int32": 4, "float32": 4, "bfloat16": 2, "float16": 2, "float64": 8, "int64": 8}

# unsigned view of each element type, for bitwise comparison
BITS = {"int32": np.uint32, "float32": np.uint32, "bfloat16": np.uint16,
        "float16": np.uint16, "float64": np.uint64, "int64": np.uint64}

# wider accumulation type of the "wide" mode
WIDE = {"bfloat16": "float32", "float16": "float32", "float32": "float64"}

# canonical quiet NaN of each float type, as bits
QNAN = {"float32": 0x7FC00000, "bfloat16": 0x7FC0, "float16": 0x7E00,
        "float64": 0x7FF8000000000000}


def bf16_bits_to_f32(bits):
    """Exact widening of bfloat16 bit patterns to float32 values.

    A bfloat16 is the upper half of a binary32 with the same sign, exponent and
    leading 7 fraction bits, so widening appends 16 zero bits.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x):
    """Round float32 values to bfloat16 bit patterns, to nearest, ties to even.

    The 16 low bits are dropped after adding just under half an ulp of the kept
    part, plus one when the kept part is odd: a remainder above half rounds up,
    below half rounds down, exactly half rounds to the even neighbour.  Overflow
    rounds to infinity as IEEE requires.  NaNs stay NaN (quiet bit forced on).
    """
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    is_nan = (u & 0x7FFFFFFF) > 0x7F800000
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    quiet_nan = (u >> 16) | 0x0040
    return np.where(is_nan, quiet_nan, rounded).astype(np.uint16)


def as_values(a, dtype):
    """Numerical values of stored elements (float64 for floats, int64 for ints)."""
    if dtype == "int32":
        return np.asarray(a, dtype=np.int32).astype(np.int64)
    if dtype == "int64":
        return np.asarray(a, dtype=np.int64).copy()
    if dtype == "float32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bfloat16":
        return bf16_bits_to_f32(a).astype(np.float64)
    if dtype == "float16":
        return np.asarray(a, dtype=np.float16).astype(np.float64)
    if dtype == "float64":
        return np.asarray(a, dtype=np.float64).copy()
    raise ValueError(dtype)


def from_f64(v, dtype):
    """Round float64 values to ``dtype`` (nearest even), in STORAGE[dtype]."""
    v = np.asarray(v, dtype=np.float64)
    if dtype == "float64":
        return v.copy()
    if dtype == "float32":
        return v.astype(np.float32)
    if dtype == "float16":
        return v.astype(np.float16)
    if dtype == "bfloat16":
        # float64 -> float32 -> bfloat16: both roundings to nearest even; the
        # pair equals one rounding of a quotient or sum of bfloat16 values
        return f32_to_bf16_bits(v.astype(np.float32))
    raise ValueError(dtype)


def add_rounded(a, b, dtype):
    """One hop: a + b rounded to ``dtype``; operands and result in STORAGE[dtype]."""
    if dtype == "int32":
        s = np.asarray(a, np.int32).astype(np.int64) + np.asarray(b, np.int32).astype(np.int64)
        return (s & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    if dtype == "int64":
        s = (np.asarray(a, np.int64).view(np.uint64).astype(np.uint64)
             + np.asarray(b, np.int64).view(np.uint64))       # unsigned: wraps mod 2**64
        return s.view(np.int64)
    if dtype == "float16":
        a = np.asarray(a, np.float16).astype(np.float32)
        b = np.asarray(b, np.float16).astype(np.float32)
        return np.add(a, b, dtype=np.float32).astype(np.float16)
    if dtype == "float64":
        return np.add(np.asarray(a, np.float64), np.asarray(b, np.float64), dtype=np.float64)
    if dtype == "float32":
        a = np.asarray(a, np.float32)
        b = np.asarray(b, np.float32)
        return np.add(a, b, dtype=np.float32)
    if dtype == "bfloat16":
        s = np.add(bf16_bits_to_f32(a), bf16_bits_to_f32(b), dtype=np.float32)
        return f32_to_bf16_bits(s)
    raise ValueError(dtype)


def max_exact(a, b, dtype):
    """The larger of a and b (see the module notes for NaN and signed zero)."""
    if dtype in ("int32", "int64"):
        return np.maximum(np.asarray(a, STORAGE[dtype]), np.asarray(b, STORAGE[dtype]))
    a = np.asarray(a, STORAGE[dtype])
    b = np.asarray(b, STORAGE[dtype])
    va, vb = as_values(a, dtype), as_values(b, dtype)
    bits_a, bits_b = a.view(BITS[dtype]), b.view(BITS[dtype])
    # equal values with different bits are +0 and -0: take the one without the sign bit
    sign = BITS[dtype](1) << BITS[dtype](8 * ITEMSIZE[dtype] - 1)
    pick_b = (vb > va) | ((vb == va) & ((bits_a & sign) != 0))
    out = np.where(pick_b, bits_b, bits_a)
    nan = np.isnan(va) | np.isnan(vb)
    out = np.where(nan, BITS[dtype](QNAN[dtype]), out).astype(BITS[dtype])
    return out.view(STORAGE[dtype])


def combine(a, b, dtype, op):
    """One hop of reduction ``op``: "sum" and "avg" add (avg's terms are divided
    before they enter), "max" takes the larger."""
    if op in ("sum", "avg"):
        return add_rounded(a, b, dtype)
    if op == "max":
        return max_exact(a, b, dtype)
    raise ValueError(op)


def pre_divide(a, dtype, p):
    """x / p rounded to ``dtype`` (floats only): a contribution to an average."""
    if dtype not in FLOATS:
        raise ValueError(f"avg needs a floating-point type, not {dtype}")
    return from_f64(as_values(a, dtype) / float(p), dtype)


def widen(a, dtype):
    """Exact values of ``a`` in the wide accumulation type WIDE[dtype]."""
    w = WIDE[dtype]
    return as_values(a, dtype).astype(STORAGE[w])


def narrow(w, dtype):
    """Round wide accumulator values to ``dtype`` once (nearest even)."""
    wide = WIDE[dtype]
    if wide == "float64":
        return np.asarray(w, np.float64).astype(STORAGE[dtype])
    w = np.asarray(w, np.float32)
    if dtype == "bfloat16":
        return f32_to_bf16_bits(w)
    return w.astype(np.float16)


def wide_term(a, dtype, op, p):
    """A term of the wide fold: widened, and for "avg" divided by p in the wide type."""
    w = widen(a, dtype)
    if op == "avg":
        # float64 quotient rounded to the wide type: one correct rounding
        return (w.astype(np.float64) / float(p)).astype(STORAGE[WIDE[dtype]])
    return w


def wide_add(a, b, dtype):
    """a + b rounded to the wide type of ``dtype``."""
    t = STORAGE[WIDE[dtype]]
    return np.add(np.asarray(a, t), np.asarray(b, t), dtype=t)
