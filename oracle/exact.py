"""Float64 reference sum and the error measure for re-ordered sums (oracle; test infrastructure only).

[InDepth] "An implementation" runs its simulator on buffers widened to float64;
that wide sum is the yardstick for algorithms whose summation order differs from
the ring's (the tree), which [InDepth] says to compare with a tolerance rather
than bit for bit because the order differs.

Tolerance reading: an element-wise relative error is unbounded wherever the exact
sum is close to zero, so errors are measured normwise over the whole result:

    err = max_i |got_i - exact_i| / max_i |exact_i|.
"""

import numpy as np

from .arith import as_values


def exact_sum(xs, dtype):
    """Element-wise sum of the p ranks' stored values, in float64 (int64 for ints).

    The p <= 64 operands are summed in rank order in float64; for bfloat16 and
    float32 inputs that is exact or within a few float64 ulps, far below any
    tolerance it is used for.
    """
    acc = as_values(xs[0], dtype).copy()
    for x in xs[1:]:
        acc = acc + as_values(x, dtype)
    return acc


def normwise_error(got, exact):
    """max |got - exact| / max |exact|; 0 when both are all zero."""
    got = np.asarray(got, dtype=np.float64)
    exact = np.asarray(exact, dtype=np.float64)
    if got.size == 0:
        return 0.0
    scale = np.max(np.abs(exact))
    diff = np.max(np.abs(got - exact))
    if scale == 0.0:
        return 0.0 if diff == 0.0 else float("inf")
    return float(diff / scale)
