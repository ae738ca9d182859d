"""Pins for the oracle's ring schedule: printed examples, invariants, brute force.

Hand-derived floating-point cases pin the accumulation order: each uses values
whose sum depends on the order of the additions, with the expected value worked
out from IEEE round-to-nearest-even by hand (derivation in the comments).
"""

import math

import numpy as np
import pytest

import oracle
from oracle import cost
from ring_all_reduce_schedule_amd import inputs


# ---------------------------------------------------------------- printed examples

def test_worked_trace(golden):
    g = golden("trace_p4_n4.json")
    p, n = g["p"], g["n"]
    base = np.array(g["inputs_rule"]["base"], np.float32)
    xs = [np.float32(r + 1) * base for r in range(p)]
    assert all(np.array_equal(a, b) for a, b in zip(xs, inputs.trace_inputs()))
    final, after_rs, tr = oracle.ring_allreduce(xs, "float32", keep_states=True)
    for r in range(p):
        assert final[r].tolist() == g["expected_final_every_rank"]
    # chunk 0 on its way round the ring, one step at a time
    for hop in g["chunk0_reduce_scatter_path"]["after_rs_step"]:
        assert tr.states[hop["step"]][hop["rank"]][0] == hop["value"]
    # all-gather: the finished 10 leaves rank 3 and is copied to 0, then 1, then 2
    have = [tr.states[p - 2][r][0] == 10 for r in range(p)]
    assert have == [False, False, False, True]
    for k, (src, dst) in enumerate(g["chunk0_all_gather_path"]["hops"]):
        st = tr.states[p - 1 + k]
        assert tr.ag_table[k][src] == 0
        assert st[dst][0] == 10 and st[src][0] == 10
    assert tr.sent == [g["elements_sent_per_rank"]] * p


def test_deepinsea_semantics(golden):
    g = golden("deepinsea_examples.json")["semantics"]
    xs = [np.array(v, np.int32) for v in g["inputs"]]
    final, _, _ = oracle.ring_allreduce(xs, "int32")
    assert all(f.tolist() == g["expected_every_rank"] for f in final)
    xs = [np.array(v, np.float32) for v in g["inputs"]]
    final, _, _ = oracle.ring_allreduce(xs, "float32")
    assert all(f.tolist() == g["expected_every_rank"] for f in final)


# ---------------------------------------------------------------- brute force

SIZES = [(p, n) for p in (1, 2, 3, 4, 5, 8, 9) for n in (0, 1, 2, 3, 4, 7, 8, 9, 10, 17, 33)]


@pytest.mark.parametrize("p,n", SIZES)
def test_int32_equals_brute_force_sum(p, n):
    rng = np.random.default_rng(p * 100 + n)
    xs = [rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32) for _ in range(p)]
    want = [((sum(int(x[i]) for x in xs) + 2**31) % 2**32) - 2**31 for i in range(n)]
    for d in (1, -1):
        final, _, tr = oracle.ring_allreduce(xs, "int32", direction=d)
        for f in final:
            assert f.tolist() == want
        assert tr.steps == cost.ring_steps(p)


@pytest.mark.parametrize("p,n", SIZES)
def test_int32_rs_owner_holds_full_sum(p, n):
    rng = np.random.default_rng(7 + p * n)
    xs = [rng.integers(-1000, 1001, n).astype(np.int32) for _ in range(p)]
    want = np.sum(np.stack(xs).astype(np.int64), axis=0) if n else np.zeros(0)
    bounds = oracle.chunk_bounds(n, p)
    for d in (1, -1):
        after_rs = oracle.reduce_scatter(xs, "int32", direction=d)[0]
        for r in range(p):
            lo, hi = bounds[oracle.owned_chunk(r, p, d)]
            assert after_rs[r][lo:hi].tolist() == want[lo:hi].tolist()
        # forward ring: rank r owns chunk (r + 1) mod p
        if d == 1:
            assert all(oracle.owned_chunk(r, p) == (r + 1) % p for r in range(p))


def test_small_integer_floats_sum_exactly():
    # integer values whose partial sums stay below 2**8 are exact in bf16 and
    # in float32, so any order gives the integer sum
    p, n = 16, 1001
    for dtype in ("float32", "bfloat16"):
        xs = inputs.small_int_valued(p, n, dtype, -8, 8, seed=3)
        want = np.sum(np.stack([oracle.as_values(x, dtype) for x in xs]), axis=0)
        final, _, _ = oracle.ring_allreduce(xs, dtype)
        for f in final:
            assert np.array_equal(oracle.as_values(f, dtype), want)


# ---------------------------------------------------------------- order pins

E = 2.0 ** -24


def _three_rank_case():
    # chunk c is summed x_c, x_{c+1}, x_{c+2} on the forward ring.  Element c
    # (one element per chunk) gets:
    #   c = 0: (x0, x1, x2) = (1, 2**-24, -2**-24)
    #          forward:  1 + 2**-24 is a tie between 1 and 1 + 2**-23 -> 1 (even);
    #                    then 1 - 2**-24 is representable -> 1 - 2**-24
    #          any order that adds x1 and x2 first, or x0 and x2 first, gives 1
    #   c = 1: (x1, x2, x0) = (2**-24, 2**-24, 1)
    #          forward:  2**-24 + 2**-24 = 2**-23 exactly; + 1 = 1 + 2**-23 exactly
    #          any order that adds the 1 earlier rounds the small terms away -> 1
    #   c = 2: (x2, x0, x1) = (2**-24, 1, 2**-24)
    #          forward:  2**-24 + 1 -> 1 (tie, even); + 2**-24 -> 1
    #          mirrored order x2, x1, x0: 2**-23, then 1 + 2**-23
    # assemble per rank: rank q holds at element c the value that chunk c's
    # order assigns to it
    seq = {0: (1.0, E, -E), 1: (E, E, 1.0), 2: (E, 1.0, E)}
    xs = [np.zeros(3, np.float32) for _ in range(3)]
    for c, vals in seq.items():
        for k, v in enumerate(vals):
            xs[(c + k) % 3][c] = v
    return xs


def test_forward_order_by_hand():
    xs = _three_rank_case()
    final, _, _ = oracle.ring_allreduce(xs, "float32")
    want = np.array([1.0 - E, 1.0 + 2 * E, 1.0], np.float32)
    for f in final:
        assert np.array_equal(f, want)
    assert np.array_equal(oracle.ring_fold(xs, "float32"), want)


def test_mirrored_order_by_hand():
    # mirrored ring sums chunk c as x_c, x_{c-1}, x_{c-2}
    #   c = 0: x0, x2, x1 = 1, -2**-24, 2**-24: 1 - 2**-24 exact, + 2**-24 -> 1
    #   c = 1: x1, x0, x2 = 2**-24, 1, 2**-24: -> 1 (tie, even), -> 1
    #   c = 2: x2, x1, x0 = 2**-24, 2**-24, 1: 2**-23, then 1 + 2**-23
    xs = _three_rank_case()
    final, _, _ = oracle.ring_allreduce(xs, "float32", direction=-1)
    want = np.array([1.0, 1.0, 1.0 + 2 * E], np.float32)
    for f in final:
        assert np.array_equal(f, want)
    assert np.array_equal(oracle.ring_fold(xs, "float32", direction=-1), want)


def test_bf16_rounds_every_hop():
    # p = 3, one element: chunk 0 is summed 1, 2**-8, 2**-8.  Rounding each hop
    # to bf16: 1 + 2**-8 ties to 1 (even), and again -> 1.0.  Accumulating in a
    # wider type and rounding once would give 1 + 2**-7 (= 0x3F81) instead.
    b = inputs.f32_to_bf16_bits_torch
    xs = [b(np.array([1.0], np.float32)), b(np.array([2.0**-8], np.float32)),
          b(np.array([2.0**-8], np.float32))]
    final, _, _ = oracle.ring_allreduce(xs, "bfloat16")
    assert all(f[0] == 0x3F80 for f in final)


# ---------------------------------------------------------------- invariants

@pytest.mark.parametrize("p,n", [(4, 4), (4, 1), (9, 1000), (9, 1_003), (8, 64),
                                 (3, 2), (64, 640), (5, 0)])
def test_send_counts(p, n):
    xs = [np.zeros(n, np.int32) for _ in range(p)]
    _, _, tr = oracle.ring_allreduce(xs, "int32")
    assert sum(tr.sent) == 2 * (p - 1) * n
    assert tr.sent == cost.ring_sends_per_rank(n, p)
    if n % p == 0:
        assert all(s == 2 * (p - 1) * n // p for s in tr.sent)
    for s in tr.sent:
        assert abs(s - cost.traffic_factor(p) * n) <= 2 and s <= 2 * n
    assert tr.reads + tr.writes == cost.one_memory_ring_elements(n, p)


def test_p1_is_noop():
    x = [np.arange(5, dtype=np.float32)]
    final, _, tr = oracle.ring_allreduce(x, "float32")
    assert np.array_equal(final[0], x[0]) and tr.steps == 0 and tr.sent == [0]


@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
@pytest.mark.parametrize("p,n", [(2, 9), (3, 10), (4, 33), (8, 1000), (9, 1003), (16, 257)])
def test_simulator_matches_closed_form(dtype, p, n):
    xs = inputs.make_inputs(p, n, dtype, seed=p + n, sigma=3.0)
    for d in (1, -1):
        final, after_rs, _ = oracle.ring_allreduce(xs, dtype, direction=d)
        fold = oracle.ring_fold(xs, dtype, direction=d)
        for r in range(p):
            assert np.array_equal(final[r], fold)
            assert np.array_equal(after_rs[r], oracle.rs_partial(xs, dtype, r, d))


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("p,n", [(2, 9), (3, 10), (4, 4), (5, 3), (8, 1000), (9, 1003)])
def test_rs_owned_is_simulator_owned_chunk_and_input_elsewhere(dtype, p, n):
    # a reduce-scatter that writes only the owned chunk: that chunk equals what the
    # lock-step simulator leaves there, every other chunk is the rank's input
    xs = inputs.make_inputs(p, n, dtype, seed=7 * p + n, sigma=3.0)
    bounds = oracle.chunk_bounds(n, p)
    for d in (1, -1):
        after_rs, _ = oracle.reduce_scatter(xs, dtype, direction=d)
        for r in range(p):
            got = oracle.rs_owned(xs, dtype, r, d)
            own = oracle.owned_chunk(r, p, d)
            for c, (lo, hi) in enumerate(bounds):
                want = after_rs[r][lo:hi] if c == own else xs[r][lo:hi]
                assert np.array_equal(got[lo:hi], want)


def test_rs_owned_int32_brute_force():
    p, n = 5, 23
    rng = np.random.default_rng(5)
    xs = [rng.integers(-2**31, 2**31, n, dtype=np.int64).astype(np.int32) for _ in range(p)]
    total = np.sum(np.stack(xs).astype(np.int64), axis=0).astype(np.int32)
    for r in range(p):
        lo, hi = oracle.chunk_bounds(n, p)[(r + 1) % p]
        assert np.array_equal(oracle.rs_owned(xs, "int32", r)[lo:hi], total[lo:hi])


@pytest.mark.parametrize("direction", [1, -1])
def test_fold_window_matches_whole(direction):
    p, n = 9, 1003
    xs = inputs.make_inputs(p, n, "bfloat16", seed=9)
    whole = oracle.ring_fold(xs, "bfloat16", direction=direction)
    for lo, hi in [(0, 5), (100, 300), (110, 115), (998, 1003), (0, 1003)]:
        got = oracle.ring_fold_window([x[lo:hi] for x in xs], lo, n, "bfloat16", direction)
        assert np.array_equal(got, whole[lo:hi])


def test_dead_rank_times_out():
    xs = [np.ones(8, np.float32) for _ in range(4)]
    with pytest.raises(oracle.RingTimeout) as e:
        oracle.ring_allreduce(xs, "float32", dead_rank=2)
    assert e.value.rank == 3 and e.value.phase == "reduce-scatter" and e.value.step == 0
    with pytest.raises(oracle.RingTimeout) as e:
        oracle.ring_allreduce(xs, "float32", direction=-1, dead_rank=2)
    assert e.value.rank == 1
