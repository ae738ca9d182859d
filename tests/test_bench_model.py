"""The byte counts bench.py rates each algorithm on, against the oracle (CPU).

bench.py divides every measured time into the HBM bytes the algorithm moves.
Those counts are checked here against the element reads and writes that the
oracle's simulators perform when every buffer lives in one memory (one byte per
element, so elements and bytes coincide):

* ring all-reduce and its phases: the lock-step simulator's own read/write
  tally ([InDepth] "The schedule");
* the slice-carrying pipelined ring: an executable trace of its accesses,
  checked against the oracle's result and counted;
* binomial tree: one read-read-write per reduce pair and one read-write per
  broadcast pair of the oracle's tree ([Derive] "Where it stops scaling");
* two-level ring: the tallies of the in-node reduce-scatter, the cross-node ring
  all-reduces of the shards and the in-node all-gather, run on the oracle's
  layout ([InDepth] "What real libraries add", hierarchy);
* fused passes: every buffer read once and written once.
"""

import numpy as np
import pytest

import bench
import oracle
from oracle import cost
from oracle.ring import reduce_scatter, all_gather
from oracle.tree import tree_levels, tree_pairs

CASES = [(2, 10), (3, 7), (4, 4), (8, 64), (8, 1001), (9, 1000), (12, 60), (16, 5)]


def _zeros(p, n):
    return [np.zeros(n, np.int32) for _ in range(p)]


@pytest.mark.parametrize("p,n", CASES)
def test_ring_family_moves_what_the_simulator_moves(p, n):
    _, _, tr = oracle.ring_allreduce(_zeros(p, n), "int32")
    for algo in ("ring_step", "ring_pipelined_flags", "ring_channels", "ring_bidir"):
        assert bench.own_bytes(algo, p, n) == tr.reads + tr.writes, algo


@pytest.mark.parametrize("p,n", CASES)
def test_phase_bytes(p, n):
    _, rs = reduce_scatter(_zeros(p, n), "int32")
    _, ag = all_gather(_zeros(p, n), "int32")
    assert bench.phase_bytes("reduce_scatter", "ring_step", p, n)[1] == rs.reads + rs.writes
    assert bench.phase_bytes("all_gather", "ring_step", p, n)[1] == ag.reads + ag.writes
    # the fused passes: every rank read, one owned chunk per rank written; every
    # owned chunk read once and written to the p - 1 other ranks
    bounds = oracle.chunk_bounds(n, p)
    owned = sum(hi - lo for lo, hi in bounds)
    assert bench.phase_bytes("reduce_scatter", "fused", p, n) == (p * n + owned,) * 2
    assert bench.phase_bytes("all_gather", "fused", p, n) == (owned + (p - 1) * owned,) * 2


@pytest.mark.parametrize("p,n", CASES + [(5, 3), (7, 11), (64, 2)])
def test_tree_moves_five_p_minus_one_buffers(p, n):
    reads = writes = 0
    for k in range(tree_levels(p)):
        pairs = len(tree_pairs(p, k))
        reads += 2 * pairs * n      # B[r] <- B[r] + B[r + 2^k]
        writes += pairs * n
        reads += pairs * n          # B[r + 2^k] <- B[r], on the way down
        writes += pairs * n
    assert bench.own_bytes("tree", p, n) == reads + writes


@pytest.mark.parametrize("p,g,n", [(4, 2, 10), (8, 4, 64), (8, 2, 1001), (9, 3, 1000),
                                   (12, 3, 60), (12, 4, 61), (16, 8, 5), (6, 1, 7), (6, 6, 7)])
def test_hier_moves_five_p_minus_one_buffers(p, g, n):
    m, nodes, locals_ = oracle.hier.hier_layout(p, g)
    total = 0
    for ranks in nodes:
        _, tr = reduce_scatter(_zeros(g, n), "int32")
        total += tr.reads + tr.writes
    intra = oracle.chunk_bounds(n, g)
    for l, ranks in enumerate(locals_):
        lo, hi = intra[(l + 1) % g]
        _, _, tr = oracle.ring_allreduce(_zeros(m, hi - lo), "int32")
        total += tr.reads + tr.writes
    for ranks in nodes:
        _, tr = all_gather(_zeros(g, n), "int32")
        total += tr.reads + tr.writes
    assert bench.own_bytes("hier", p, n) == total


@pytest.mark.parametrize("p,n", CASES)
def test_fused_moves_each_buffer_twice(p, n):
    assert bench.own_bytes("fused", p, n) == cost.one_memory_min_elements(n, p) == 2 * p * n
    assert bench.own_bytes("hier_fused", p, n) == 2 * p * n


def _rider_trace(xs):
    """The slice-carrying pipelined ring as a list of memory accesses, executed on
    copies of the inputs ([InDepth] "What real libraries add", pipelining): for
    each chunk c, the value starts from rank c's copy and visits ranks c+1, ...,
    c+p-1, each visit reading the receiver's copy and writing the receiver's
    new partial; then the finished value is written to ranks c, ..., c+p-2.
    Returns (final buffers, reads, writes) in elements."""
    p = len(xs)
    bufs = [x.copy() for x in xs]
    reads = writes = 0
    for c, (lo, hi) in enumerate(oracle.chunk_bounds(len(xs[0]), p)):
        for i in range(lo, hi):
            acc = bufs[c][i]
            reads += 1
            for k in range(1, p):
                r = (c + k) % p
                acc = np.int32(np.int64(acc) + np.int64(bufs[r][i]))   # wraps like int32
                reads += 1
                bufs[r][i] = acc
                writes += 1
            for k in range(p - 1):
                bufs[(c + k) % p][i] = acc
                writes += 1
    return bufs, reads, writes


@pytest.mark.parametrize("p,n", CASES)
def test_pipelined_ring_moves_3p_minus_2_buffers(p, n):
    rng = np.random.default_rng(p * 1000 + n)
    xs = [rng.integers(-1000, 1000, n, dtype=np.int32) for _ in range(p)]
    bufs, reads, writes = _rider_trace(xs)
    want = oracle.ring_fold(xs, "int32")
    assert all(np.array_equal(b, want) for b in bufs)
    assert bench.own_bytes("ring_pipelined", p, n) == reads + writes == (3 * p - 2) * n
    # the flag-driven form moves what the step-by-step simulator moves
    _, _, tr = oracle.ring_allreduce(_zeros(p, n), "int32")
    assert bench.own_bytes("ring_pipelined_flags", p, n) == tr.reads + tr.writes


@pytest.mark.parametrize("p,n", CASES)
def test_pipelined_phase_bytes(p, n):
    # reduce-scatter alone: the trace without its all-gather writes; it leaves
    # the simulator's partial states
    rng = np.random.default_rng(p + n)
    xs = [rng.integers(-1000, 1000, n, dtype=np.int32) for _ in range(p)]
    _, reads, writes = _rider_trace(xs)
    rs_moved = reads + writes - (p - 1) * n
    assert bench.phase_bytes("reduce_scatter", "ring_pipelined", p, n)[1] == rs_moved
    # all-gather alone: one read of each owned chunk, p - 1 writes
    assert bench.phase_bytes("all_gather", "ring_pipelined", p, n)[1] == p * n
