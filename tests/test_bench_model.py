"""The byte counts bench.py rates each algorithm on, against the oracle (CPU).

bench.py divides every measured time into the HBM bytes the algorithm moves.
Those counts are checked here against the element reads and writes that the
oracle's simulators perform when every buffer lives in one memory (one byte per
element, so elements and bytes coincide):

* ring all-reduce and its phases: the lock-step simulator's own read/write
  tally ([InDepth] "The schedule");
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
    for algo in ("ring_step", "ring_pipelined", "ring_channels", "ring_bidir"):
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
