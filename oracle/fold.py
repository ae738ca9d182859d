"""Closed form of the ring's accumulation order (oracle; test infrastructure only).

A second, independent statement of what the ring computes, read off the rules of
[InDepth] "The schedule" rather than simulated: chunk c is first sent by rank c
(at reduce-scatter step 0 the sender of chunk c is the rank r with r - s = c),
and every hop moves it one rank further and adds that rank's contribution.  So an
element i of chunk c is summed in the order

    x_c[i], x_{c+d}[i], x_{c+2d}[i], ..., x_{c+(p-1)d}[i]      (indices mod p)

with a rounding to the element type after every addition, d = +1 on the forward
ring and d = -1 on the mirrored one.  The last rank of that sequence, c - d, is
the owner; the all-gather copies its value to everyone without arithmetic
([Fable] "What it is"; [InDepth] "The schedule").  Partway through the
reduce-scatter, rank r holds in chunk c the fold of the first ((r - c) * d mod p)
+ 1 terms of that sequence.

``ring_fold_window`` evaluates the same order for a window of a buffer too large
to hold on the host; it only needs the window's elements and their global
positions.
"""

import numpy as np

from .arith import add_rounded
from .schedule import chunk_bounds


def _fold_terms(terms, dtype):
    acc = np.array(terms[0], copy=True)
    for t in terms[1:]:
        acc = add_rounded(acc, t, dtype)
    return acc


def ring_fold(xs, dtype, direction=1):
    """All-reduce result (identical on every rank) by folding in ring order."""
    p = len(xs)
    n = len(xs[0])
    out = np.empty_like(np.asarray(xs[0]))
    for c, (lo, hi) in enumerate(chunk_bounds(n, p)):
        if hi == lo:
            continue
        order = [(c + direction * k) % p for k in range(p)]
        out[lo:hi] = _fold_terms([np.asarray(xs[q])[lo:hi] for q in order], dtype)
    return out


def rs_partial(xs, dtype, r, direction=1):
    """Rank r's whole buffer right after the reduce-scatter, from the closed form."""
    p = len(xs)
    n = len(xs[0])
    out = np.array(xs[r], copy=True)
    for c, (lo, hi) in enumerate(chunk_bounds(n, p)):
        if hi == lo:
            continue
        m = ((r - c) * direction) % p + 1          # terms folded so far
        order = [(c + direction * k) % p for k in range(m)]
        out[lo:hi] = _fold_terms([np.asarray(xs[q])[lo:hi] for q in order], dtype)
    return out


def rs_owned(xs, dtype, r, direction=1):
    """Rank r's buffer after a reduce-scatter that writes only the owned chunk.

    The owned chunk, (r + direction) mod p ([InDepth] "The schedule": rank r ends
    the reduce-scatter holding chunk r + 1), carries the full ring-order fold;
    every other chunk keeps rank r's input.  This is what a reduce-scatter used on
    its own must deliver ([InDepth] "Trade-offs"); the partial sums the
    step-by-step ring leaves in the other chunks are a by-product of its schedule.
    """
    p = len(xs)
    n = len(xs[0])
    out = np.array(xs[r], copy=True)
    c = (r + direction) % p
    lo, hi = chunk_bounds(n, p)[c]
    if hi > lo:
        order = [(c + direction * k) % p for k in range(p)]
        out[lo:hi] = _fold_terms([np.asarray(xs[q])[lo:hi] for q in order], dtype)
    return out


def ring_fold_window(windows, lo, n, dtype, direction=1):
    """Ring-order result for elements [lo, lo + len(window)) of n-element buffers.

    ``windows[r]`` holds rank r's elements of that window.  Each element's chunk
    follows from the global chunk bounds, so windows may straddle chunk edges.
    """
    p = len(windows)
    w = len(windows[0])
    hi = lo + w
    if not 0 <= lo <= hi <= n:
        raise ValueError("window outside the buffer")
    out = np.empty_like(np.asarray(windows[0]))
    for c, (clo, chi) in enumerate(chunk_bounds(n, p)):
        a, b = max(lo, clo), min(hi, chi)
        if a >= b:
            continue
        order = [(c + direction * k) % p for k in range(p)]
        out[a - lo:b - lo] = _fold_terms(
            [np.asarray(windows[q])[a - lo:b - lo] for q in order], dtype)
    return out
