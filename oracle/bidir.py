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
