"""Binomial-tree all-reduce (oracle; test infrastructure only).

[Derive] "Where it stops scaling": a tree all-reduce reduces up a binary tree and
broadcasts back down, in about 2 log2(n) steps instead of the ring's 2(n - 1);
[InDepth] "Trade-offs" and "Failure modes" name it as the choice for small
messages.  The pages do not fix the tree's shape, so this takes the plainest one:
a binomial tree rooted at rank 0 with L = ceil(log2 p) levels.

  reduce,    k = 0 .. L-1:   for every r that is a multiple of 2**(k+1) and has
                             a partner r + 2**k < p:  B[r] <- B[r] + B[r + 2**k]
                             (rounded to the element type, whole buffer)
  broadcast, k = L-1 .. 0:   for the same pairs:      B[r + 2**k] <- B[r]

Each step moves the whole buffer, not a chunk.  Rank 0 ends the reduction with
the sum; after the broadcast every rank holds that same value.
"""

import numpy as np

from .arith import combine, pre_divide


def tree_levels(p):
    """L = ceil(log2 p), the number of reduce (and of broadcast) steps."""
    levels = 0
    while (1 << levels) < p:
        levels += 1
    return levels


def tree_pairs(p, k):
    """(parent, child) pairs active at level k."""
    stride = 1 << k
    return [(r, r + stride) for r in range(0, p, 2 * stride) if r + stride < p]


def tree_allreduce(bufs, dtype, op="sum"):
    """Returns (final buffers, rank 0's buffer after the reduction, step count).

    "max" combines with the exact maximum; "avg" divides every buffer by p first.
    """
    bufs = [np.array(b, copy=True) for b in bufs]
    p = len(bufs)
    if op == "avg":
        bufs = [pre_divide(b, dtype, p) for b in bufs]
    levels = tree_levels(p)
    steps = 0
    for k in range(levels):
        for parent, child in tree_pairs(p, k):
            bufs[parent] = combine(bufs[parent], bufs[child], dtype, op)
        steps += 1
    reduced = bufs[0].copy()
    for k in reversed(range(levels)):
        for parent, child in tree_pairs(p, k):
            bufs[child] = bufs[parent].copy()
        steps += 1
    return bufs, reduced, steps
