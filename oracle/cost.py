"""Step counts, traffic and the latency-bandwidth cost model (oracle; test infrastructure only).

[InDepth] "The schedule" and [Derive] "A strong answer": each phase has p - 1
steps; at every step each rank sends one chunk of about N/p elements; so a rank
sends 2(p - 1)/p * N elements over the whole all-reduce, which stays below 2N
for any p.  [Derive] "Where it stops scaling" adds a fixed latency alpha per
step: T_ring = 2(p - 1) * alpha + 2(p - 1)/p * S / B for an S-byte buffer and a
per-direction link bandwidth B.  A binomial tree takes 2 ceil(log2 p) steps, each
moving the whole buffer ([Derive] "Where it stops scaling": fewer latencies, a
bandwidth term worse by a constant).

The per-rank formula 2(p - 1)/p * N is exact only when p divides N.  With the
uneven chunks of [InDepth] "An implementation", rank r sends every chunk except
(r + 1) mod p during the reduce-scatter and every chunk except (r + 2) mod p
during the all-gather, i.e. 2N - |chunk r+1| - |chunk r+2| elements; summed
over ranks that is exactly 2(p - 1)N.

One-memory traffic: when all p buffers live in the same memory, a receive-add
reads two chunks and writes one and a receive-copy reads one and writes one, so
the ring as scheduled touches 3(p-1)N + 2(p-1)N = 5(p-1)N elements; the smallest
possible traffic is 2pN (each buffer read once and written once, since each
output element depends on all p inputs and every buffer is overwritten).
"""

import math

from .schedule import chunk_bounds


def ring_steps(p):
    """Sequential steps of the ring all-reduce: 2(p - 1)."""
    return 2 * (p - 1)


def tree_steps(p):
    """Sequential steps of the binomial tree: 2 ceil(log2 p)."""
    return 2 * math.ceil(math.log2(p)) if p > 1 else 0


def traffic_factor(p):
    """2(p - 1)/p: buffers' worth of data each rank sends."""
    return 2.0 * (p - 1) / p


def ring_bytes_per_rank(size_bytes, p):
    """Bytes a rank sends over the whole all-reduce, 2(p - 1)/p * S."""
    return traffic_factor(p) * size_bytes


def ring_sends_per_rank(n, p):
    """Exact elements sent by each rank for an n-element buffer, uneven chunks included."""
    lens = [hi - lo for lo, hi in chunk_bounds(n, p)]
    if p == 1:
        return [0]
    return [2 * n - lens[(r + 1) % p] - lens[(r + 2) % p] for r in range(p)]


def t_ring(p, size_bytes, bandwidth, alpha):
    """T_ring = 2(p-1) alpha + 2(p-1)/p * S / B  ([Derive] "Where it stops scaling")."""
    return ring_steps(p) * alpha + ring_bytes_per_rank(size_bytes, p) / bandwidth


def t_ring_terms(p, size_bytes, bandwidth, alpha):
    """(latency term, bandwidth term) of T_ring."""
    return ring_steps(p) * alpha, ring_bytes_per_rank(size_bytes, p) / bandwidth


def t_tree(p, size_bytes, bandwidth, alpha):
    """Tree time under the same model: every one of its steps moves the whole buffer.

    Reading: the page gives only the step count and "worse by a constant" for
    the bandwidth term; pricing each of the 2 ceil(log2 p) steps at alpha + S/B
    is the plainest model consistent with both.
    """
    return tree_steps(p) * (alpha + size_bytes / bandwidth)


def choose_ring_or_tree(p, size_bytes, bandwidth, alpha):
    """The algorithm the cost model favours: "tree" if T_tree < T_ring, else "ring".

    [InDepth] "Trade-offs" and [Derive] "Where it stops scaling": libraries price
    both algorithms for every call; big messages go to the ring, small ones to
    the tree.  Ties go to the ring.
    """
    return "tree" if t_tree(p, size_bytes, bandwidth, alpha) < t_ring(p, size_bytes, bandwidth, alpha) else "ring"


def ring_tree_crossover(p, bandwidth, alpha):
    """Buffer size S* at which T_ring = T_tree (None if the tree never wins).

    Setting 2(p-1)a + 2(p-1)/p S/B = 2L(a + S/B) with L = ceil(log2 p):
    S* = B a (2(p-1) - 2L) / (2L - 2(p-1)/p).  The tree wins below S*.
    """
    L = math.ceil(math.log2(p)) if p > 1 else 0
    lat = ring_steps(p) - 2 * L
    bw = 2 * L - traffic_factor(p)
    if lat <= 0 or bw <= 0:
        return None
    return bandwidth * alpha * lat / bw


def t_hier(p, g, size_bytes, b_intra, b_inter, alpha=0.0):
    """Two-level ring ([InDepth] "What real libraries add", hierarchy, and the
    worked example "flat versus hierarchical"): reduce-scatter over the g ranks of
    a node, ring all-reduce of the S/g shard over the m = p/g nodes, all-gather
    over the node; each phase priced like the flat ring's."""
    m = p // g
    intra = (g - 1) * alpha + phase_time(g, size_bytes, b_intra)
    inter = t_ring(m, size_bytes / g, b_inter, alpha)
    return 2 * intra + inter


def one_memory_min_elements(n, p):
    """2pN: each of the p buffers read once and written once."""
    return 2 * p * n


def one_memory_ring_elements(n, p):
    """5(p-1)N: reads and writes of the ring as scheduled, buffers in one memory."""
    return 5 * (p - 1) * n


def phase_time(p, size_bytes, bandwidth):
    """Bandwidth time of one phase (reduce-scatter or all-gather): (p-1)/p * S / B.

    [Derive] "What interviewers probe next": a reduce-scatter is exactly the
    first phase, half of an all-reduce.
    """
    return (p - 1) / p * size_bytes / bandwidth
