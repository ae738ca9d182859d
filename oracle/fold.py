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

Other reductions (``arith``): "max" folds with the exact maximum; "avg" folds
the terms x_q / p (each rounded to the element type) with the rounded sum;
``wide=True`` folds widened terms in the wide type and rounds once at the end.
"""

import numpy as np

from .arith import combine, pre_divide, wide_term, wide_add, narrow
from .schedule import chunk_bounds


def _fold_terms(terms, dtype, op="sum", wide=False):
    p = len(terms)
    if wide and op != "max":              # a maximum is exact: nothing to widen
        acc = wide_term(terms[0], dtype, op, p)
        for t in terms[1:]:
            acc = wide_add(acc, wide_term(t, dtype, op, p), dtype)
        return narrow(acc, dtype)
    if op == "avg":
        terms = [pre_divide(t, dtype, p) for t in terms]
    acc = np.array(terms[0], copy=True)
    for t in terms[1:]:
        acc = combine(acc, t, dtype, op)
    return acc


def ring_fold(xs, dtype, direction=1, op="sum", wide=False):
    """All-reduce result (identical on every rank) by folding in ring order."""
    p = len(xs)
    n = len(xs[0])
    out = np.empty_like(np.asarray(xs[0]))
    for c, (lo, hi) in enumerate(chunk_bounds(n, p)):
        if hi == lo:
            continue
        order = [(c + direction * k) % p for k in range(p)]
        out[lo:hi] = _fold_terms([np.asarray(xs[q])[lo:hi] for q in order], dtype, op, wide)
    return out


def rs_partial(xs, dtype, r, direction=1, op="sum"):
    """Rank r's whole buffer right after the reduce-scatter, from the closed form.

    With "avg" every term is x_q / p, chunk r of rank r included (one term).
    """
    p = len(xs)
    n = len(xs[0])
    out = np.array(xs[r], copy=True)
    for c, (lo, hi) in enumerate(chunk_bounds(n, p)):
        if hi == lo:
            continue
        m = ((r - c) * direction) % p + 1          # terms folded so far
        order = [(c + direction * k) % p for k in range(m)]
        terms = [np.asarray(xs[q])[lo:hi] for q in order]
        if op == "avg":
            out[lo:hi] = _fold_terms([pre_divide(t, dtype, p) for t in terms], dtype, "sum")
        else:
            out[lo:hi] = _fold_terms(terms, dtype, op)
    return out


def rs_owned(xs, dtype, r, direction=1, op="sum", wide=False):
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
        out[lo:hi] = _fold_terms([np.asarray(xs[q])[lo:hi] for q in order], dtype, op, wide)
    return out


def ring_fold_window(windows, lo, n, dtype, direction=1, op="sum", wide=False):
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
            [np.asarray(windows[q])[a - lo:b - lo] for q in order], dtype, op, wide)
    return out
