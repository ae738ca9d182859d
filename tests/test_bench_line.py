"""bench.py's last stdout line: short enough for a reader that keeps only the
tail of stdout, and carrying the headline, its roofline and its CPU baseline.

The full record is built here with the shapes a real run produces (seven rank
counts x nine sizes in the alpha sweep, three per-workload records of eight
algorithms, ten variants), filled with placeholder numbers.
"""

import json

import bench

ALGOS = ("fused", "ring_step", "ring_pipelined", "ring_bidir", "ring_channels", "tree",
         "hier", "hier_fused")


def _full_result():
    sizes = [1 << 10, 4 << 10, 16 << 10, 64 << 10, 256 << 10, 1 << 20, 4 << 20, 16 << 20,
             64 << 20]
    fit = {}
    for p in (2, 4, 8, 9, 16, 32, 64):
        rows = [{"S_per_rank": s, **{f"{a}_ms": 0.123456 for a in ALGOS[:6]}} for s in sizes]
        fit[f"p{p}"] = {"sizes": rows,
                        **{a: {"alpha_us": 3.21, "B_GBps_per_rank": 812.34} for a in ALGOS[:6]},
                        "largest_S_per_rank_where_tree_beats_ring": 1 << 20,
                        "model_crossover_S_per_rank": 123456,
                        "not_fused_fastest": [[p, 1024, "tree", 0.0062, 0.0078]]}
    keys = ("ms_cold", "GBps_cold", "pct_peak_cold", "pct_of_copy_cold", "ms_warm", "GBps_warm",
            "pct_of_copy_warm", "hbm_bytes")
    per_workload = {name: {algo: {k: 1.2345 for k in keys} for algo in ALGOS}
                    for name in ("p9_int32_n1000003", "p64_bf16_1MiB", "p8_fp32_256MiB")}
    variants = {name: {"ms": 87.123, "GBps_on_2pS": 2938.1, "hbm_bytes": 560000000000,
                       "GBps_on_hbm_bytes": 6427.7, "pct_peak_on_hbm_bytes": 80.35}
                for name in ("ring_step", "ring_pipelined", "ring_bidir", "ring_channels", "tree",
                             "hier", "hier_fused", "fused_wide_fp32_accumulate", "fused_avg",
                             "fused_max")}
    return {
        "metric": bench.METRIC, "value": 6318.6, "unit": "GB/s", "n_gpus": 1, "steps": 20,
        "warmup": 5, "ms_per_step": 40.5152, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded normal/uniform draws, generated in HBM or on the host)",
        "config": {"workload": "p8_bf16_16GB", "p": 8, "n_per_rank": 8000000000,
                   "bytes_per_rank": 16000000000, "algo": "fused",
                   "bytes_counted": "2*p*S (each rank buffer read once and written once)",
                   "bytes_per_step": 256000000000},
        "pct_of_hbm_peak": 78.98, "busbw_emulated_GBps": 691.1,
        "roofline": {"bound": "hbm", "achieved": 6319.4, "peak": 8000.0, "unit": "GB/s",
                     "frac": 0.7899, "traffic": 255952500000.0,
                     "kernel": "ra::k_fused<bfloat16>", "launch_ms_mean": 40.5105,
                     "launch_ms_min": 40.4889, "kernel_source_sha": "b7ed246b3f8532cc"},
        "wall_s_timed": 0.815,
        "ceiling": {"kernel": "ra::k_copy", "bytes_moved": 17179869184, "GBps": 6507.0},
        "pct_of_copy_ceiling": 97.1,
        "cpu_baseline": {"value": 0.5779, "unit": "GB/s", "cores": 1, "kind": "oracle",
                         "seconds": 22.298, "host_cores_available": 16,
                         "sample": "lock-step oracle (numpy, one thread) all-reducing the first "
                                   "402,653,184 elements of each of the 8 rank buffers of the "
                                   "workload (p=8, N=402,653,184 bfloat16); rate on 2*p*S of "
                                   "that sample"},
        "variants": variants,
        "phases": {f"{c}_{a}": {"ms": 1.0, "bytes_floor": 1, "GBps_on_floor": 1.0}
                   for c in ("reduce_scatter", "all_gather") for a in ("fused", "ring_step")},
        "per_workload": per_workload,
        "cpu_baseline_per_workload": {"x": {"seconds": 1.0}},
        "alpha": {"in_kernel_step_us_p64_1KiB": 2.64, "fit": fit},
        "alpha_us": 2.64,
        "detail_file": "gpurun_out/bench_detail.json",
    }


def test_full_record_is_far_longer_than_the_line():
    assert len(json.dumps(_full_result())) > 4 * bench.SUMMARY_MAX_CHARS


def test_summary_line_is_short_and_complete():
    line = json.dumps(bench.summary_line(_full_result()))
    assert len(line) < 4096
    assert "\n" not in line
    got = json.loads(line)
    for key in ("metric", "value", "unit", "n_gpus", "steps", "ms_per_step", "dtype", "config",
                "roofline", "cpu_baseline", "pct_of_copy_ceiling", "alpha_us",
                "crossover_S_per_rank", "algos_ms"):
        assert key in got, key
    assert got["config"]["workload"] == "p8_bf16_16GB"
    for key in ("bound", "achieved", "peak", "unit", "frac", "traffic"):
        assert key in got["roofline"], key
    for key in ("value", "unit", "cores", "kind", "sample"):
        assert key in got["cpu_baseline"], key
    assert set(got["crossover_S_per_rank"]) == {f"p{p}" for p in (2, 4, 8, 9, 16, 32, 64)}
    for key in ("per_workload", "variants", "phases", "alpha"):
        assert key not in got, key


def test_summary_line_without_extras():
    """--no-extras (profiling runs): the line still carries the headline."""
    r = _full_result()
    for k in ("variants", "phases", "per_workload", "alpha", "ceiling", "alpha_us",
              "pct_of_copy_ceiling", "cpu_baseline_per_workload"):
        r.pop(k)
    got = bench.summary_line(r)
    assert got["value"] == 6318.6 and "roofline" in got and "algos_ms" not in got


def test_summary_line_drops_optional_parts_before_growing_too_long():
    r = _full_result()
    r["alpha"]["fit"]["p2"]["not_fused_fastest"] = [[2, 1 << k, "tree", 0.1, 0.2]
                                                    for k in range(400)]
    line = json.dumps(bench.summary_line(r))
    assert len(line) <= bench.SUMMARY_MAX_CHARS
    assert json.loads(line)["roofline"]["frac"] == 0.7899


def test_counter_summary_matches_the_kernel_sources():
    """The committed counter summary of the headline kernel was taken on the
    current one-pass kernel sources: bench.py fills `roofline.traffic` (and the
    traced kernel's name) from it only while their hash matches, so a change to
    those sources must come with a new summary."""
    traffic, kernel = bench.read_traffic(bench.kernel_source_sha(), 2 * 8 * 16_000_000_000)
    assert traffic is not None, "profiles/fused_p8_bf16_16GB_hbm_traffic.md is stale"
    assert abs(traffic / (2 * 8 * 16e9) - 1) < 0.01
    assert kernel and kernel.startswith("ra::k_fused")
