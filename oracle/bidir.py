"""Bidirectional ring all-reduce (oracle; test infrastructure only).

[InDepth] "What real libraries add", bidirectional rings: links are full duplex,
so a second ring runs the opposite way on half of the data.  The page does not
say which half, nor what happens with an odd N; the reading taken here splits the
buffer with the same rule as the chunk partition, chunk_bounds(N, 2), so the
first ceil(N/2) elements go round the forward ring and the remaining floor(N/2)
round the mirrored ring (rank r sends to r - 1; see ``schedule``).  Each half is
an ordinary ring all-reduce with its own p chunks.
"""

import numpy as np

from .fold import ring_fold_window
from .ring import ring_allreduce
from .schedule import chunk_bounds


def bidir_halves(n):
    """[(lo, hi) of the forward half, (lo, hi) of the mirrored half]."""
    return chunk_bounds(n, 2)


def bidir_allreduce(bufs, dtype, op="sum"):
    """Returns (final buffers, buffers after both reduce-scatters)."""
    p = len(bufs)
    n = len(bufs[0])
    (a0, a1), (b0, b1) = bidir_halves(n)
    fwd, fwd_rs, _ = ring_allreduce([np.asarray(b)[a0:a1] for b in bufs], dtype, 1, op=op)
    rev, rev_rs, _ = ring_allreduce([np.asarray(b)[b0:b1] for b in bufs], dtype, -1, op=op)
    final = [np.concatenate([fwd[r], rev[r]]) for r in range(p)]
    after_rs = [np.concatenate([fwd_rs[r], rev_rs[r]]) for r in range(p)]
    return final, after_rs


def bidir_fold_window(windows, lo, n, dtype, op="sum"):
    """The bidirectional result for elements [lo, lo + len(window)) of n-element
    buffers: the part of the window in the forward half folds in the forward
    ring's order over that half's chunks, the part in the mirrored half in the
    mirrored ring's order over its chunks.  ``windows[r]`` holds rank r's
    elements of the window, which may straddle the two halves."""
    w = len(windows[0])
    hi = lo + w
    if not 0 <= lo <= hi <= n:
        raise ValueError("window outside the buffer")
    (a0, a1), (b0, b1) = bidir_halves(n)
    parts = []
    if lo < a1:
        s, e = lo, min(hi, a1)
        parts.append(ring_fold_window([np.asarray(x)[s - lo:e - lo] for x in windows], s - a0,
                                      a1 - a0, dtype, 1, op=op))
    if hi > b0:
        s, e = max(lo, b0), hi
        parts.append(ring_fold_window([np.asarray(x)[s - lo:e - lo] for x in windows], s - b0,
                                      b1 - b0, dtype, -1, op=op))
    if not parts:
        return np.empty_like(np.asarray(windows[0]))
    return np.concatenate(parts)
