"""Pins for the float64 reference, the error measure and the cost model (CPU only)."""

import math

import numpy as np
import pytest

import oracle
from oracle import cost
from ring_all_reduce_schedule_amd import inputs


def test_exact_sum_matches_fsum():
    # math.fsum is a correctly rounded sum; the float64 running sum of <= 64
    # bf16/fp32 values must agree to a few float64 ulps
    for dtype, p in (("float32", 8), ("bfloat16", 64)):
        xs = inputs.make_inputs(p, 2000, dtype, seed=1, sigma=1.0)
        got = oracle.exact_sum(xs, dtype)
        vals = [oracle.as_values(x, dtype) for x in xs]
        want = np.array([math.fsum(v[i] for v in vals) for i in range(2000)])
        assert np.all(np.abs(got - want) <= 8 * np.spacing(np.maximum(np.abs(want), 1e-300)))


def test_exact_sum_int():
    xs = [np.array([2**31 - 1, -5], np.int32)] * 3
    assert oracle.exact_sum(xs, "int32").tolist() == [3 * (2**31 - 1), -15]


def test_normwise_error():
    assert oracle.normwise_error([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert oracle.normwise_error([1.0, 2.5], [1.0, 2.0]) == 0.25
    assert oracle.normwise_error([0.0], [0.0]) == 0.0
    assert oracle.normwise_error([], []) == 0.0


def test_traffic_factor_printed(golden):
    g = golden("cost_figures.json")["traffic_factor"]
    for v in g["values"]:
        assert round(cost.traffic_factor(v["n"]), g["decimals"]) == v["factor"]


def test_bytes_per_rank_printed(golden):
    for v in golden("cost_figures.json")["bytes_per_rank"]["values"]:
        assert cost.ring_bytes_per_rank(v["S_GB"] * 1e9, v["n"]) / 1e9 == pytest.approx(v["GB"])


def test_bandwidth_time_printed(golden):
    for v in golden("cost_figures.json")["bandwidth_time"]["values"]:
        t = cost.t_ring(v["n"], v["S_GB"] * 1e9, v["B_GBps"] * 1e9, 0.0)
        assert t == pytest.approx(v["seconds"], rel=v["rel_tol"])


def test_latency_vs_bandwidth_printed(golden):
    g = golden("cost_figures.json")["latency_vs_bandwidth"]
    for v in g["values"]:
        lat, bw = cost.t_ring_terms(v["n"], v["S_bytes"], 50e9, 10e-6)
        assert lat * 1e3 == pytest.approx(v["latency_ms"], rel=g["rel_tol"])
        assert bw * 1e3 == pytest.approx(v["bandwidth_ms"], rel=g["rel_tol"])
    lat, bw = cost.t_ring_terms(1024, 1e6, 50e9, 10e-6)
    assert lat / bw == pytest.approx(g["latency_over_bandwidth_small_buffer"], rel=0.05)


def test_tree_vs_ring_latency_count(golden):
    g = golden("cost_figures.json")["tree_vs_ring_latencies"]
    assert cost.tree_steps(g["n"]) == g["tree"]
    assert cost.ring_steps(g["n"]) == g["ring"]


def test_fable_station_counts(golden):
    for v in golden("cost_figures.json")["stations"]["values"]:
        assert cost.ring_steps(v["p"]) == v["steps"]


def test_hierarchical_phase_figures(golden):
    g = golden("cost_figures.json")["hierarchical_phase"]
    a = g["intra_rs"]
    assert cost.phase_time(a["p"], a["S_GB"] * 1e9, a["B_GBps"] * 1e9) == pytest.approx(a["seconds"])
    b = g["cross_ar"]
    assert cost.t_ring(b["p"], b["S_GB"] * 1e9, b["B_GBps"] * 1e9, 0.0) == pytest.approx(b["seconds"])


def test_trace_sends(golden):
    g = golden("trace_p4_n4.json")
    assert cost.traffic_factor(4) * 4 == g["elements_sent_per_rank"]
    assert cost.ring_sends_per_rank(4, 4) == [6, 6, 6, 6]


def test_deepinsea_single_element_sends():
    # p = 4, N = 1: chunk 0 holds the element and chunks 1..3 are empty.  Rank r
    # sends chunk 0 once in each phase unless chunk 0 is r+1 (skipped in the
    # reduce-scatter) or r+2 (skipped in the all-gather): ranks 2 and 3 send once.
    assert cost.ring_sends_per_rank(1, 4) == [2, 2, 1, 1]
    xs = [np.array([v], np.int32) for v in (1, 2, 3, 4)]
    _, _, tr = oracle.ring_allreduce(xs, "int32")
    assert tr.sent == [2, 2, 1, 1]


def test_model_is_monotone_and_bounded():
    for p in (2, 8, 64, 1024):
        assert cost.traffic_factor(p) < 2.0
        assert cost.ring_bytes_per_rank(1.0, p) < cost.ring_bytes_per_rank(1.0, 2 * p)


def test_ring_tree_choice_printed(golden):
    g = golden("cost_figures.json")["reversal"]
    for c in g["cases"]:
        assert cost.choose_ring_or_tree(c["n"], c["S_bytes"], g["B_Bps"], g["alpha_s"]) == c["winner"]


def test_crossover_is_a_few_hundred_kilobytes_per_rank(golden):
    g = golden("cost_figures.json")["reversal"]
    lo, hi = g["crossover_S_per_rank_bytes_range"]
    for p in (64, 1024):
        for b in (g["B_Bps"], g["also_B_Bps"]):
            s = cost.ring_tree_crossover(p, b, g["alpha_s"])
            assert lo <= s / p <= hi


@pytest.mark.parametrize("p", [4, 5, 8, 9, 16, 64, 1024])
def test_crossover_closed_form_matches_bisection(p):
    # the closed form against a root of T_ring - T_tree found by bisection
    b, a = 50e9, 1e-5
    f = lambda s: cost.t_ring(p, s, b, a) - cost.t_tree(p, s, b, a)
    lo, hi = 0.0, 1e12
    assert f(lo) > 0 > f(hi)
    for _ in range(200):
        mid = (lo + hi) / 2
        lo, hi = (mid, hi) if f(mid) > 0 else (lo, mid)
    s = cost.ring_tree_crossover(p, b, a)
    assert s == pytest.approx(lo, rel=1e-9)
    assert cost.choose_ring_or_tree(p, s * 0.999, b, a) == "tree"
    assert cost.choose_ring_or_tree(p, s * 1.001, b, a) == "ring"


@pytest.mark.parametrize("p", [2, 3])
def test_two_or_three_ranks_never_choose_the_tree(p):
    # p = 2: one tree level costs 2(a + S/B) against the ring's 2a + S/B; p = 3:
    # both take 4 steps and the tree moves more bytes per step
    assert cost.ring_tree_crossover(p, 50e9, 1e-5) is None
    for s in (1.0, 1e3, 1e9):
        assert cost.choose_ring_or_tree(p, s, 50e9, 1e-5) == "ring"
