"""Per-hop addition, rounded to the buffer's element type (oracle; test infrastructure only).

Which precision each hop uses: [InDepth] "An implementation" accumulates every
hop of the torch ring with an in-place add on the tensor itself, i.e. in the
tensor's own dtype, and [Derive] "What interviewers probe next" states that the
library reduces in the buffer's dtype unless told otherwise.  So every hop of the
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

bfloat16 values are carried as uint16 bit patterns.
"""

import numpy as np

DTYPES = ("int32", "float32", "bfloat16")

# numpy storage type of each element type
STORAGE = {"int32": np.int32, "float32": np.float32, "bfloat16": np.uint16}

# bytes per element
ITEMSIZE = {"int32": 4, "float32": 4, "bfloat16": 2}


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
    if dtype == "float32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    if dtype == "bfloat16":
        return bf16_bits_to_f32(a).astype(np.float64)
    raise ValueError(dtype)


def add_rounded(a, b, dtype):
    """One hop: a + b rounded to ``dtype``; operands and result in STORAGE[dtype]."""
    if dtype == "int32":
        s = np.asarray(a, np.int32).astype(np.int64) + np.asarray(b, np.int32).astype(np.int64)
        return (s & 0xFFFFFFFF).astype(np.uint32).view(np.int32)
    if dtype == "float32":
        a = np.asarray(a, np.float32)
        b = np.asarray(b, np.float32)
        return np.add(a, b, dtype=np.float32)
    if dtype == "bfloat16":
        s = np.add(bf16_bits_to_f32(a), bf16_bits_to_f32(b), dtype=np.float32)
        return f32_to_bf16_bits(s)
    raise ValueError(dtype)
