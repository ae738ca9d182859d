"""Pins for the oracle's chunk partition and index rules (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import schedule


CASES = [(n, p) for p in (1, 2, 3, 4, 7, 8, 9, 16, 64)
         for n in (0, 1, 2, 3, 5, 7, 8, 9, 63, 64, 65, 100, 1000, 1_000_003)]


@pytest.mark.parametrize("n,p", CASES)
def test_chunk_sizes_match_library_split(n, p):
    # numpy.array_split and torch.tensor_split both give the first n mod p
    # pieces one extra element -- the rule the in-depth page states for its
    # chunk partition and uses via tensor_split
    bounds = oracle.chunk_bounds(n, p)
    sizes = [hi - lo for lo, hi in bounds]
    assert sizes == [len(a) for a in np.array_split(np.arange(n), p)]
    assert sizes == [t.numel() for t in torch.tensor_split(torch.arange(n), p)]
    assert bounds[0][0] == 0 and bounds[-1][1] == n
    for (a, b), (c, d) in zip(bounds, bounds[1:]):
        assert b == c
    assert max(sizes) - min(sizes) <= 1
    extra = n % p
    assert all(s == n // p + 1 for s in sizes[:extra])
    assert all(s == n // p for s in sizes[extra:])


def test_chunk_bounds_beyond_32_bits():
    bounds = oracle.chunk_bounds(8_000_000_000, 8)
    assert [hi - lo for lo, hi in bounds] == [1_000_000_000] * 8
    bounds = oracle.chunk_bounds(2**33 + 5, 3)
    assert bounds[-1][1] == 2**33 + 5
    assert [hi - lo for lo, hi in bounds] == [(2**33 + 5) // 3 + (i < (2**33 + 5) % 3)
                                             for i in range(3)]


def test_chunk_bounds_rejects_bad_args():
    with pytest.raises(ValueError):
        oracle.chunk_bounds(4, 0)
    with pytest.raises(ValueError):
        oracle.chunk_bounds(-1, 4)


@pytest.mark.parametrize("n,p", [(10, 3), (1, 4), (17, 5), (64, 8)])
def test_chunk_of_is_consistent(n, p):
    owners = [oracle.chunk_of(i, n, p) for i in range(n)]
    for c, (lo, hi) in enumerate(oracle.chunk_bounds(n, p)):
        assert owners[lo:hi] == [c] * (hi - lo)


def test_deepinsea_step_table(golden):
    # printed table: step 1 ranks 0..3 send chunks 0,1,2,3; step 2 send 3,0,1,2
    g = golden("deepinsea_examples.json")["reduce_scatter_step_table"]
    p = g["p"]
    for label, expected in g["steps"].items():
        s = int(label) - 1
        assert [oracle.rs_send_chunk(r, s, p) for r in range(p)] == expected
        # and the simulator actually sends those chunks
    xs = [np.zeros(8, np.float32) for _ in range(p)]
    _, _, tr = oracle.ring_allreduce(xs, "float32")
    assert tr.rs_table[0] == g["steps"]["1"] and tr.rs_table[1] == g["steps"]["2"]


@pytest.mark.parametrize("p", [2, 3, 4, 5, 8, 9, 64])
def test_each_step_is_a_permutation(p):
    # every chunk is in flight exactly once per step, in both phases and rings
    for d in (1, -1):
        for s in range(p - 1):
            assert sorted(oracle.rs_send_chunk(r, s, p, d) for r in range(p)) == list(range(p))
            assert sorted(oracle.ag_send_chunk(r, s, p, d) for r in range(p)) == list(range(p))


@pytest.mark.parametrize("p", [2, 3, 4, 9, 16])
def test_all_gather_starts_at_owner(p):
    # all-gather step 0: every rank sends the chunk it owns after reduce-scatter
    for d in (1, -1):
        for r in range(p):
            assert oracle.ag_send_chunk(r, 0, p, d) == oracle.owned_chunk(r, p, d)


@pytest.mark.parametrize("p", [2, 3, 4, 9])
def test_rs_chunk_reaches_owner(p):
    # following the reduce-scatter rule, chunk c leaves rank c at step 0 and after
    # p-1 hops sits on the rank that owns it
    for d in (1, -1):
        for c in range(p):
            r = c
            for s in range(p - 1):
                assert oracle.rs_send_chunk(r, s, p, d) == c
                r = oracle.right_of(r, p, d)
            assert oracle.owned_chunk(r, p, d) == c
