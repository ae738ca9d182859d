"""Hierarchical (two-level) ring all-reduce (oracle; test infrastructure only).

[InDepth] "What real libraries add", hierarchy: the two-level scheme first
reduce-scatters within every node; each rank then all-reduces the 1/g of the
buffer it now owns with its counterparts (same position within their nodes) in
the other nodes; a final in-node all-gather spreads the result.  Only the middle
phase crosses nodes, and it moves 1/g of what a flat ring would send across
them.  [Deepinsea] "Ring vs Hierarchical" describes the same two-level ring.

Reading of the layout (the pages give none): p = g * m ranks; node q holds ranks
q*g .. q*g + g - 1 and rank r has local index l = r mod g.  Every ring below is
the plain ring of ``ring``:

1. intra-node reduce-scatter: in every node, a ring over local indices
   0 .. g-1 on the whole buffer cut into g chunks; local rank l ends owning
   chunk (l + 1) mod g, summed over the node;
2. inter-node all-reduce: for every local index l, a ring over nodes 0 .. m-1
   among the ranks q*g + l, on the shard = chunk (l + 1) mod g of the intra
   partition, cut into m sub-chunks;
3. intra-node all-gather: the node's rings copy every owned chunk round.

Averages divide every rank's buffer by the total p first, then sum.
``hier_fold`` states the same order per element without simulating: element i
in intra chunk c and, inside that shard, in sub-chunk d is

    A_q  = fold over local ranks c, c+1, ..., c+g-1 (mod g) of node q
    out  = fold over nodes d, d+1, ..., d+m-1 (mod m) of A_q

with every hop rounded to the element type.
"""

import numpy as np

from .arith import combine, pre_divide
from .ring import reduce_scatter, all_gather, ring_allreduce
from .schedule import chunk_bounds


def hier_layout(p, g):
    """(m, node ranks, local-index ranks) for p = g * m."""
    if g < 1 or p % g:
        raise ValueError(f"group size {g} must divide p = {p}")
    m = p // g
    nodes = [[q * g + l for l in range(g)] for q in range(m)]
    locals_ = [[q * g + l for q in range(m)] for l in range(g)]
    return m, nodes, locals_


def hier_allreduce(bufs, dtype, g, op="sum"):
    """Returns (final buffers, elements each rank sent across nodes, within nodes)."""
    p = len(bufs)
    n = len(bufs[0])
    m, nodes, locals_ = hier_layout(p, g)
    bufs = [np.array(b, copy=True) for b in bufs]
    if op == "avg":
        bufs = [pre_divide(b, dtype, p) for b in bufs]
        op = "sum"
    cross = [0] * p
    inner = [0] * p
    # 1. reduce-scatter inside every node
    for ranks in nodes:
        out, tr = reduce_scatter([bufs[r] for r in ranks], dtype, op=op)
        for r, b, s in zip(ranks, out, tr.sent):
            bufs[r] = b
            inner[r] += s
    # 2. cross-node ring all-reduce of the shard each local index owns
    intra = chunk_bounds(n, g)
    for l, ranks in enumerate(locals_):
        lo, hi = intra[(l + 1) % g]
        final, _, tr = ring_allreduce([bufs[r][lo:hi] for r in ranks], dtype, op=op)
        for r, b, s in zip(ranks, final, tr.sent):
            bufs[r][lo:hi] = b
            cross[r] += s
    # 3. all-gather inside every node
    for ranks in nodes:
        out, tr = all_gather([bufs[r] for r in ranks], dtype)
        for r, b, s in zip(ranks, out, tr.sent):
            bufs[r] = b
            inner[r] += s
    return bufs, cross, inner


def hier_fold(xs, dtype, g, op="sum"):
    """The hierarchical order per element (identical on every rank)."""
    p = len(xs)
    n = len(xs[0])
    m = p // g
    if g < 1 or p % g:
        raise ValueError(f"group size {g} must divide p = {p}")
    terms = [np.asarray(x) for x in xs]
    if op == "avg":
        terms = [pre_divide(x, dtype, p) for x in terms]
        op = "sum"
    out = np.empty_like(terms[0])
    for c, (lo, hi) in enumerate(chunk_bounds(n, g)):
        for d, (a, b) in enumerate(chunk_bounds(hi - lo, m)):
            if a == b:
                continue
            s0, s1 = lo + a, lo + b
            total = None
            for k2 in range(m):
                q = (d + k2) % m
                acc = None
                for k1 in range(g):
                    x = terms[q * g + (c + k1) % g][s0:s1]
                    acc = x.copy() if acc is None else combine(acc, x, dtype, op)
                total = acc if total is None else combine(total, acc, dtype, op)
            out[s0:s1] = total
    return out


def hier_fold_window(windows, lo, n, dtype, g, op="sum"):
    """The hierarchical order for elements [lo, lo + len(window)) of n-element buffers.

    ``windows[r]`` holds rank r's elements of that window; every element's intra
    chunk and inter piece follow from the global partition, so windows may
    straddle either kind of edge.
    """
    p = len(windows)
    m = p // g
    if g < 1 or p % g:
        raise ValueError(f"group size {g} must divide p = {p}")
    w = len(windows[0])
    hi = lo + w
    if not 0 <= lo <= hi <= n:
        raise ValueError("window outside the buffer")
    terms = [np.asarray(x) for x in windows]
    if op == "avg":
        terms = [pre_divide(x, dtype, p) for x in terms]
        op = "sum"
    out = np.empty_like(terms[0])
    for c, (clo, chi) in enumerate(chunk_bounds(n, g)):
        for d, (a, b) in enumerate(chunk_bounds(chi - clo, m)):
            s0, s1 = max(lo, clo + a), min(hi, clo + b)
            if s0 >= s1:
                continue
            total = None
            for k2 in range(m):
                q = (d + k2) % m
                acc = None
                for k1 in range(g):
                    x = terms[q * g + (c + k1) % g][s0 - lo:s1 - lo]
                    acc = x.copy() if acc is None else combine(acc, x, dtype, op)
                total = acc if total is None else combine(total, acc, dtype, op)
            out[s0 - lo:s1 - lo] = total
    return out
