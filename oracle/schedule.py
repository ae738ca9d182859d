"""Chunk partition and the ring's index rules (oracle; test infrastructure only).

[InDepth] "The schedule": the p ranks form a logical ring in which every rank
talks to two neighbours, sending to the next and receiving from the previous.
Every rank's N-element buffer is cut into p chunks.  Reduce-scatter step s:
rank r sends chunk (r - s) mod p to rank r + 1, whose copy of that chunk then
becomes the sum of the two.  All-gather step s:
rank r sends chunk (r + 1 - s) mod p and the receiver overwrites.  After the
reduce-scatter rank r holds the finished sum of chunk (r + 1) mod p.

[InDepth] "An implementation": when p does not divide N, the first N mod p chunks
carry one element more than the rest (the same rule as torch.tensor_split, whose
first pieces are the largest).

The second ring of the bidirectional variant ([InDepth] "What real libraries
add", bidirectional rings) runs the other way round.  It is the forward ring seen
through the mirror r -> -r (mod p): rank r sends to r - 1, reduce-scatter step s
sends chunk (r + s) mod p, all-gather step s sends chunk (r - 1 + s) mod p, and
rank r ends the reduce-scatter owning chunk (r - 1) mod p.  ``direction`` selects
the ring: +1 forward, -1 mirrored.
"""


def chunk_bounds(n, p):
    """Half-open element ranges [start, end) of the p chunks of an n-element buffer.

    [InDepth] "An implementation": every chunk gets floor(n/p) elements and the
    first n mod p chunks one more, laid end to end from element 0.  Python ints
    throughout, so buffers beyond 2**32 elements are exact.
    """
    if p < 1:
        raise ValueError("p must be >= 1")
    if n < 0:
        raise ValueError("n must be >= 0")
    short = n // p
    longer = n - short * p          # chunks that take one extra element
    bounds = []
    lo = 0
    for c in range(p):
        size = short + 1 if c < longer else short
        bounds.append((lo, lo + size))
        lo += size
    assert lo == n
    return bounds


def chunk_of(i, n, p):
    """Index of the chunk that element i of an n-element buffer belongs to.

    Found by scanning the bounds, so it holds by construction for every i.
    """
    if not 0 <= i < n:
        raise IndexError(i)
    for c, (lo, hi) in enumerate(chunk_bounds(n, p)):
        if lo <= i < hi:
            return c
    raise AssertionError("unreachable")


def right_of(r, p, direction=1):
    """Rank that r sends to: r + 1 on the forward ring, r - 1 on the mirrored ring."""
    return (r + direction) % p


def left_of(r, p, direction=1):
    """Rank that r receives from."""
    return (r - direction) % p


def rs_send_chunk(r, s, p, direction=1):
    """Chunk rank r sends at reduce-scatter step s ([InDepth] "The schedule")."""
    return (r - direction * s) % p


def ag_send_chunk(r, s, p, direction=1):
    """Chunk rank r sends at all-gather step s ([InDepth] "The schedule")."""
    return (r + direction * (1 - s)) % p


def owned_chunk(r, p, direction=1):
    """Chunk whose full sum rank r holds once the reduce-scatter is over."""
    return (r + direction) % p
