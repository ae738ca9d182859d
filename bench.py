#!/usr/bin/env python3
"""Benchmark: effective all-reduce bandwidth of the ring schedule on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--algo ALGO]

One "step" is one all-reduce of the workload's p rank buffers (all resident in
HBM before timing starts) through the C ABI (ra_allreduce_ex).  The default
workload is p8_bf16_16GB: 8 virtual ranks x 8e9 bf16 elements (16 GB per rank,
128 GB in all), drawn on the device.  The figure of merit is the effective
bandwidth on the least traffic any one-GPU all-reduce needs, 2*p*S bytes (every
rank buffer read once and written once), against the 8 TB/s HBM3E peak.

Prints ONE short JSON line on stdout, last (at most 4 KB: a reader that keeps
only the tail of stdout still gets it whole).  Besides the driver's fields it
carries
  roofline      the all-reduce kernel's achieved bytes/s vs the HBM peak, its
                launch duration from HIP events on the launch stream, and the
                HBM traffic read from the committed rocprofv3 counter summary
                (null when that summary was taken on different kernel source)
  cpu_baseline  the CPU oracle timed on a bounded sample of the same workload
  algos_ms      every other algorithm's time on the same buffers
  alpha_us      per-step latency of the step-by-step ring (in-kernel timestamps)
  crossover_S_per_rank  per rank count: the largest per-rank size at which the
                tree beat the ring, and the pages' model crossover
  copy_ceiling_GBps  a plain copy of the same byte count (read + write)
The full record (per-workload rates, the alpha fits, the standalone phases)
goes to the --detail file (default gpurun_out/bench_detail.json).

Buffers are all-reduced in place, so values grow by about p per call; the
default step counts stay far from bf16 overflow and inputs are redrawn before
the variant timings.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("effective all-reduce GB/s & % of HBM peak per S,p on 1 MI355X; "
          "per-step α (µs)")
HBM_PEAK_GBPS = 8000.0
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "fused_p8_bf16_16GB_hbm_traffic.md")
# the sources k_fused is compiled from: the traffic figure is valid only for them
KERNEL_SOURCES = [os.path.join(ROOT, "ring_all_reduce_schedule_amd", "csrc", f)
                  for f in ("ra_fused.hip", "ra_elem.h")]


def kernel_source_sha():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def parse_args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="p8_bf16_16GB")
    ap.add_argument("--algo", default="fused")
    ap.add_argument("--grid", type=int, default=0,
                    help="ra_options.grid for the timed algorithm (0 = the library's choice)")
    ap.add_argument("--channels", type=int, default=0,
                    help="ra_options.channels for ring_channels (0 = automatic)")
    ap.add_argument("--group", type=int, default=0,
                    help="ra_options.group for hier / hier_fused (0 = the library's default)")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip variants, alpha, ceiling (profiling runs)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample", type=int, default=3 << 27,
                    help="elements per rank of the CPU-oracle sample")
    ap.add_argument("--mode", default="allreduce",
                    choices=["allreduce", "copy", "reduce_scatter", "all_gather"],
                    help="copy: only the plain copy kernel, for counter calibration; "
                         "reduce_scatter / all_gather: only that phase with --algo on the "
                         "workload's buffers (counter runs)")
    ap.add_argument("--detail", default=os.path.join(ROOT, "gpurun_out", "bench_detail.json"),
                    help="file for the full measurement record ('' = none)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def alloc_workload(name, torch, B, inputs):
    """The p rank buffers of a workload (one allocation per rank), filled."""
    w = inputs.WORKLOADS[name]
    p, n, dtype = w["p"], w["n"], w["dtype"]
    tdt = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16}[dtype]
    bufs = [torch.empty(n, dtype=tdt, device="cuda") for _ in range(p)]
    fill_workload(name, bufs, torch, inputs)
    return w, bufs


def fill_workload(name, bufs, torch, inputs):
    w = inputs.WORKLOADS[name]
    if w.get("on_device"):
        inputs.device_normal_bf16(bufs, w["sigma"], w["seed"])
    else:
        import numpy as np
        for b, x in zip(bufs, inputs.workload_inputs(name)):
            if w["dtype"] == "bfloat16":
                b.copy_(torch.from_numpy(x.view(np.int16)).view(torch.bfloat16))
            else:
                b.copy_(torch.from_numpy(x))
    torch.cuda.synchronize()


_SPIN = {}


def run_ahead(torch, k):
    """Hold the stream in a device-side spin while the host enqueues k calls.

    A start event that reaches the GPU before the host has enqueued its call
    times the host's enqueue rate instead of the kernel (a small all-reduce takes
    less GPU time than its Python call).  The spin, enqueued before the first
    start event, lets the host run ahead, so every event pair brackets work that
    is already queued.  0.1 ms of spin per call covers the host cost of a call
    and its flush many times over."""
    if not hasattr(torch.cuda, "_sleep"):
        return
    if "cycles_per_ms" not in _SPIN:
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        torch.cuda._sleep(4_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SPIN["cycles_per_ms"] = 4_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(_SPIN["cycles_per_ms"] * (1.0 + 0.1 * k)))


def time_calls(fn, k, torch, flush=None):
    """Per-call durations (ms) from HIP events on the current stream, plus the
    span from the first start to the last end.  `flush`, if given, runs before
    each call, outside its events (to evict the Infinity Cache).  The calls are
    queued behind a short device spin (run_ahead), so the events time the GPU."""
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(k)]
    torch.cuda.synchronize()
    run_ahead(torch, k)
    for i in range(k):
        if flush is not None:
            flush()
        starts[i].record()
        fn()
        ends[i].record()
    torch.cuda.synchronize()
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    span = starts[0].elapsed_time(ends[-1])
    return per, span


def read_traffic(sha, launch_bytes):
    """(HBM bytes per launch, kernel name) from the committed counter summary, if
    it was taken on the current kernel sources and this workload's bytes."""
    if not os.path.exists(TRAFFIC_SUMMARY):
        return None, None
    text = open(TRAFFIC_SUMMARY).read()
    m_sha = re.search(r"kernel_source_sha:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_wb = re.search(r"workload_bytes_per_launch:\s*([0-9.eE+]+)", text)
    m_k = re.search(r"kernel_name:\s*(\S+)", text)
    if not (m_sha and m_b and m_wb) or m_sha.group(1) != sha:
        return None, None
    if abs(float(m_wb.group(1)) - launch_bytes) > 1:
        return None, None
    return float(m_b.group(1)), (m_k.group(1) if m_k else None)


def cpu_baseline(bufs, w, sample, torch):
    """The oracle (lock-step ring simulator) on the first `sample` elements of each rank."""
    import numpy as np
    import oracle
    p = w["p"]
    m = min(sample, w["n"])
    xs = []
    for b in bufs:
        t = b[:m].cpu()
        if w["dtype"] == "bfloat16":
            xs.append(t.view(torch.int16).numpy().view(np.uint16).copy())
        else:
            xs.append(t.numpy().copy())
    item = {"int32": 4, "float32": 4, "bfloat16": 2}[w["dtype"]]
    t0 = time.perf_counter()
    oracle.ring_allreduce(xs, w["dtype"])
    dt = time.perf_counter() - t0
    gbps = 2 * p * m * item / dt / 1e9
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3), "host_cores_available": avail,
            "sample": (f"lock-step oracle (numpy, one thread) all-reducing the first {m:,} "
                       f"elements of each of the {p} rank buffers of the workload "
                       f"(p={p}, N={m:,} {w['dtype']}); rate on 2*p*S of that sample")}


def hier_group(p):
    """Ranks per node for the hierarchical algorithms here: the largest divisor of
    p that is at most 8 and leaves at least two nodes (p = 8: 2 nodes of 4;
    p = 9: 3 of 3; p = 64: 8 of 8).  The library's own default for p = 8 is one
    node of 8, where the hierarchy is the flat ring."""
    return max([g for g in range(1, min(8, p - 1) + 1) if p % g == 0] or [1])


def own_bytes(algo, p, S):
    """HBM bytes an all-reduce algorithm moves on p buffers of S bytes each.

    The fused passes read every buffer once and write it once: 2pS.  The
    slice-carrying pipelined ring reads every buffer once and writes each
    element position 2(p-1) times (the p-1 receivers' partials, then the
    all-gather's p-1 copies): (3p-2)S.  Every step-by-step algorithm moves
    5(p-1)S:
    * ring (and its flag-driven pipelined, channel and bidirectional forms): each
      reduce-scatter step reads two copies of a chunk and writes one, 3S over
      all ranks, and each all-gather step reads one and writes one, 2S;
      (p-1) steps of each;
    * binomial tree: p-1 pairwise adds of whole buffers (read 2S, write S) and
      p-1 whole-buffer copies (read S, write S);
    * two-level ring with g ranks per node and m = p/g nodes: 3(g-1)mS in the
      in-node reduce-scatter, 5(m-1)S in the g cross-node rings over S/g-byte
      shards, 2(g-1)mS in the in-node all-gather, which add up to 5(p-1)S."""
    if algo in ("fused", "hier_fused"):
        return 2 * p * S
    if algo == "ring_pipelined":
        return (3 * p - 2) * S
    return 5 * (p - 1) * S


def phase_bytes(call, algo, p, S):
    """(byte floor, bytes moved) of a standalone reduce-scatter or all-gather.

    The floors: (p+1)S for a reduce-scatter (every rank read, one owned chunk
    per rank written) and pS for an all-gather (every owned chunk read once,
    written p-1 times); the fused passes move exactly that.  The slice-carrying
    pipelined ring's reduce-scatter reads every rank once and writes the p-1
    receivers' partials of every chunk, (2p-1)S; its all-gather is the floor.
    The step-by-step phases move 3(p-1)S (p-1 steps that read two copies of
    each chunk and write one) and 2(p-1)S (p-1 steps that read one and write
    one)."""
    floor = (p + 1) * S if call == "reduce_scatter" else p * S
    if algo == "fused":
        return floor, floor
    if algo == "ring_pipelined":
        return floor, (2 * p - 1) * S if call == "reduce_scatter" else floor
    return floor, (3 if call == "reduce_scatter" else 2) * (p - 1) * S


def cpu_baseline_workloads(inputs):
    """The oracle (lock-step ring simulator, numpy, one thread) timed in full on
    every workload the host holds comfortably: the worked trace, the 1e6-element
    int32, the 1 MiB-per-rank and the 256 MiB-per-rank configurations.  The
    16 GB-per-rank one is sampled by cpu_baseline.  Input generation is not
    timed."""
    import oracle
    out = {}
    for name in ("trace_p4_fp32_n4", "p9_int32_n1000003", "p64_bf16_1MiB", "p8_fp32_256MiB"):
        w = inputs.WORKLOADS[name]
        xs = inputs.workload_inputs(name)
        t0 = time.perf_counter()
        oracle.ring_allreduce(xs, w["dtype"])
        dt = time.perf_counter() - t0
        S = w["n"] * inputs.ITEMSIZE[w["dtype"]]
        out[name] = {"seconds": round(dt, 4), "GBps_on_2pS": round(2 * w["p"] * S / dt / 1e9, 4),
                     "cores": 1}
        del xs
    return out


def per_workload(torch, B, inputs):
    """Effective GB/s and % of HBM peak for every workload that fits comfortably,
    per algorithm, all rated on 2pS, and as % of a plain copy of the same bytes
    (the streaming ceiling at that size).

    Each algorithm is timed twice: with a 1 GiB scratch buffer read before every
    call (cold: the read replaces the Infinity Cache's contents with clean lines,
    so nothing of the workload is cached and no write-back competes with the
    timed call) and back to back (warm: workloads whose 2pS is below the 256 MB
    cache are then partly cache-resident).  The rank tensors are marshalled once
    (RankBuffers), as a caller that all-reduces the same buffers every step would."""
    import numpy as np
    scratch = torch.ones(1 << 28, dtype=torch.int32, device="cuda")
    sink = torch.empty((), dtype=torch.int64, device="cuda")

    def flush():
        torch.sum(scratch, dim=0, dtype=torch.int64, out=sink)

    out = {}
    for name in ("p9_int32_n1000003", "p64_bf16_1MiB", "p8_fp32_256MiB"):
        w, bufs = alloc_workload(name, torch, B, inputs)
        p, n, dtype = w["p"], w["n"], w["dtype"]
        S = n * inputs.ITEMSIZE[dtype]
        two_ps = 2 * p * S
        rec = {"p": p, "n_per_rank": n, "dtype": dtype, "bytes_per_rank": S, "bytes_2pS": two_ps}
        # the streaming ceiling at this size: a plain copy of the same p*S bytes
        # (rounded down to 16) from one buffer to another, timed the same ways
        cb = p * S // 16 * 16
        src = torch.ones(cb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        fn = lambda: B.ra_stream_copy(dst, src)
        fn()
        cold, _ = time_calls(fn, 9, torch, flush=flush)
        warm, _ = time_calls(fn, 9, torch)
        tc, tw = float(np.median(cold[1:])), float(np.median(warm[1:]))
        rec["copy"] = {"ms_cold": round(tc, 4), "GBps_cold": round(2 * cb / (tc * 1e-3) / 1e9, 1),
                       "ms_warm": round(tw, 4), "GBps_warm": round(2 * cb / (tw * 1e-3) / 1e9, 1)}
        del src, dst
        ranks = B.RankBuffers(bufs)
        rec["hier_group"] = hier_group(p)
        for algo in ("fused", "ring_step", "ring_pipelined", "ring_pipelined_flags", "ring_bidir",
                     "ring_channels", "tree",
                     "hier", "hier_fused"):
            kw = {"group": hier_group(p)} if algo.startswith("hier") else {}
            fn = lambda a=algo, k=kw: B.ra_allreduce_ex(ranks, algo=a, **k)
            fn()
            B.ra_stream_status()
            cold, _ = time_calls(fn, 9, torch, flush=flush)
            warm, _ = time_calls(fn, 9, torch)
            B.ra_stream_status()
            tc = float(np.median(cold[1:]))
            tw = float(np.median(warm[1:]))
            rec[algo] = {"ms_cold": round(tc, 4), "GBps_cold": round(two_ps / (tc * 1e-3) / 1e9, 1),
                         "pct_peak_cold": round(100 * two_ps / (tc * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                         "pct_of_copy_cold": round(100 * rec["copy"]["ms_cold"] / tc, 1),
                         "ms_warm": round(tw, 4), "GBps_warm": round(two_ps / (tw * 1e-3) / 1e9, 1),
                         "pct_of_copy_warm": round(100 * rec["copy"]["ms_warm"] / tw, 1),
                         "hbm_bytes": own_bytes(algo, p, S)}
        out[name] = rec
        del bufs, ranks
        torch.cuda.empty_cache()
    del scratch, sink
    torch.cuda.empty_cache()
    return out


def phase_measure(bufs, S, p, torch, B):
    """Standalone reduce-scatter and all-gather on the workload's buffers, each
    rated on its own byte floor and on the bytes it moves (phase_bytes)."""
    out = {}
    # the fused all-gather twice: as the library picks it (read/write phases at
    # this workload) and with the phases turned off, on the same buffers
    for call, algo, name, flags in (
            ("reduce_scatter", "fused", "fused", 0), ("all_gather", "fused", "fused", 0),
            ("all_gather", "fused", "fused_no_phases", B.RA_FLAG_NO_PHASES),
            ("reduce_scatter", "ring_pipelined", "ring_pipelined", 0),
            ("all_gather", "ring_pipelined", "ring_pipelined", 0),
            ("reduce_scatter", "ring_step", "ring_step", 0),
            ("all_gather", "ring_step", "ring_step", 0)):
        floor, moved = phase_bytes(call, algo, p, S)
        f = B.ra_reduce_scatter_ex if call == "reduce_scatter" else B.ra_all_gather_ex
        fn = lambda f=f, a=algo, fl=flags: f(bufs, algo=a, flags=fl)
        fn()
        B.ra_stream_status()
        per, _ = time_calls(fn, 3, torch)
        B.ra_stream_status()
        t = sum(per) / len(per)
        out[f"{call}_{name}"] = {"ms": round(t, 3), "bytes_floor": floor,
                                 "GBps_on_floor": round(floor / (t * 1e-3) / 1e9, 1),
                                 "pct_peak": round(100 * floor / (t * 1e-3) / 1e9 / HBM_PEAK_GBPS, 2),
                                 "hbm_bytes": moved,
                                 "GBps_on_hbm_bytes": round(moved / (t * 1e-3) / 1e9, 1)}
    return out


def alpha_measure(torch, B, inputs):
    """Per-step latency of the step-by-step ring.

    (1) in-kernel: device wall-clock stamps as each step's barrier releases,
        tiny buffers (p=64, 1 KiB per rank): median step time, for the default
        launch (one workgroup at this size), for 8 channels, and for 64
        workgroups on the device-wide barrier.
    (2) fit: T(S) = 2(p-1) a + 2(p-1)/p * S / B over S from 1 KiB to 64 MiB per
        rank, p = 2 .. 64 (bf16), least squares per p, for the step-by-step,
        pipelined and channel rings; the tree under the same model (2 ceil(log2 p)
        steps of a + S / B) and the fused pass (a + 2pS/BW); the ring/tree
        crossover measured and from the fitted model; the sizes at which the
        pipelined ring beats the step-by-step one.
    """
    import numpy as np
    hz = B.ra_wallclock_hz()
    out = {}
    p = 64
    n = 512
    bufs = B.RankBuffers([torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(p)])
    ts = torch.zeros(2 * (p - 1) + 1, dtype=torch.int64, device="cuda")
    steps = []
    for _ in range(5):
        B.ra_allreduce_ex(bufs, algo="ring_step", step_ts=ts)
        B.ra_stream_status()
        v = ts.cpu().numpy().astype(np.float64)
        steps.append(np.diff(v) / hz * 1e6)
    out["in_kernel_step_us_p64_1KiB"] = round(float(np.median(np.concatenate(steps))), 3)
    # the same with 8 channels: each barrier spans an eighth of the grid
    steps = []
    for _ in range(5):
        B.ra_allreduce_ex(bufs, algo="ring_channels", channels=8, step_ts=ts)
        B.ra_stream_status()
        v = ts.cpu().numpy().astype(np.float64)
        steps.append(np.diff(v) / hz * 1e6)
    out["in_kernel_step_us_p64_1KiB_8channels"] = round(float(np.median(np.concatenate(steps))), 3)
    # the same steps on 64 workgroups synchronised by the device-wide barrier
    # (at this size the library runs them on one workgroup by default)
    steps = []
    for _ in range(5):
        B.ra_allreduce_ex(bufs, algo="ring_step", grid=64, step_ts=ts)
        B.ra_stream_status()
        v = ts.cpu().numpy().astype(np.float64)
        steps.append(np.diff(v) / hz * 1e6)
    out["in_kernel_step_us_p64_1KiB_grid64"] = round(float(np.median(np.concatenate(steps))), 3)
    # what a launch per step pays: 64 minimal launches (16-byte copies) queued back
    # to back on the stream, timed as one span (events between launches would add
    # their own cost)
    s16, d16 = torch.ones(16, dtype=torch.uint8, device="cuda"), torch.empty(16, dtype=torch.uint8,
                                                                              device="cuda")
    B.ra_stream_copy(d16, s16)
    spans = []
    for _ in range(5):
        _, span = time_calls(lambda: [B.ra_stream_copy(d16, s16) for _ in range(64)], 1, torch)
        spans.append(span / 64)
    out["launch_per_step_us"] = round(float(np.median(spans)) * 1e3, 3)
    fits = {}
    algos = ("ring_step", "ring_pipelined", "ring_pipelined_flags", "ring_channels", "tree", "fused")
    sizes = [1 << 10, 4 << 10, 16 << 10, 64 << 10, 256 << 10, 1 << 20, 4 << 20, 16 << 20,
             64 << 20]
    for p in (2, 4, 8, 9, 16, 32, 64):
        levels = max(1, (p - 1).bit_length())
        rows = []
        for per_rank in sizes:
            n = per_rank // 2
            bufs = B.RankBuffers([torch.zeros(n, dtype=torch.bfloat16, device="cuda")
                                  for _ in range(p)])
            row = {"S_per_rank": per_rank}
            for algo in algos:
                per, _ = time_calls(lambda a=algo: B.ra_allreduce_ex(bufs, algo=a), 7, torch)
                row[f"{algo}_ms"] = round(float(np.median(per[2:])), 4)
            rows.append(row)
            del bufs
        rec = {"sizes": rows}
        S = np.array([r["S_per_rank"] for r in rows], dtype=np.float64)
        # ring: T = 2(p-1) a + 2(p-1)/p * S / B ([Derive] Where it stops scaling)
        A = np.stack([np.full(len(S), 2.0 * (p - 1)), 2 * (p - 1) / p * S], axis=1)
        for algo in ("ring_step", "ring_pipelined_flags", "ring_channels"):
            y = np.array([r[f"{algo}_ms"] * 1e-3 for r in rows])
            (a, inv_b), *_ = np.linalg.lstsq(A, y, rcond=None)
            rec[algo] = {"alpha_us": round(a * 1e6, 3),
                         "B_GBps_per_rank": round(1.0 / inv_b / 1e9, 2) if inv_b > 0 else None}
        # tree under the same model: 2L steps, each alpha + S / B
        At = np.stack([np.full(len(S), 2.0 * levels), 2.0 * levels * S], axis=1)
        y = np.array([r["tree_ms"] * 1e-3 for r in rows])
        (at, inv_bt), *_ = np.linalg.lstsq(At, y, rcond=None)
        rec["tree"] = {"alpha_us": round(at * 1e6, 3),
                       "B_GBps_per_rank": round(1.0 / inv_bt / 1e9, 2) if inv_bt > 0 else None}
        # fused: one launch, T = a + 2pS / BW
        Af = np.stack([np.ones(len(S)), 2.0 * p * S], axis=1)
        y = np.array([r["fused_ms"] * 1e-3 for r in rows])
        (af, inv_bf), *_ = np.linalg.lstsq(Af, y, rcond=None)
        rec["fused"] = {"fixed_us": round(af * 1e6, 3),
                        "GBps": round(1.0 / inv_bf / 1e9, 1) if inv_bf > 0 else None}
        # crossovers: measured (largest size where the tree wins) and the pages'
        # model with the ring's fitted alpha and B: S* = B a (2(p-1) - 2L) / (2L - 2(p-1)/p)
        cross = None
        for r in rows:
            if r["tree_ms"] < r["ring_step_ms"]:
                cross = r["S_per_rank"]
        rec["largest_S_per_rank_where_tree_beats_ring"] = cross
        # where slicing the chunks pays ([InDepth] What real libraries add,
        # pipelining): sizes at which each pipelined ring beats one launch per step
        for algo in ("ring_pipelined", "ring_pipelined_flags"):
            rec[f"S_per_rank_where_{algo}_beats_ring_step"] = [
                r["S_per_rank"] for r in rows if r[f"{algo}_ms"] < r["ring_step_ms"]]
        a_r = rec["ring_step"]["alpha_us"] * 1e-6
        b_r = (rec["ring_step"]["B_GBps_per_rank"] or 0) * 1e9
        lat, bw = 2.0 * (p - 1) - 2.0 * levels, 2.0 * levels - 2.0 * (p - 1) / p
        rec["model_crossover_S_per_rank"] = (round(b_r * a_r * lat / bw)
                                             if lat > 0 and bw > 0 and b_r > 0 and a_r > 0 else None)
        # every size at which another algorithm's median beat the fused pass
        rec["not_fused_fastest"] = []
        for r in rows:
            best = min((r[f"{a}_ms"], a) for a in algos)
            if best[1] != "fused":
                rec["not_fused_fastest"].append(
                    [p, r["S_per_rank"], best[1], best[0], r["fused_ms"]])
        fits[f"p{p}"] = rec
    out["fit"] = fits
    torch.cuda.empty_cache()
    return out


# Keys of the final stdout line, which must stay short (a reader that keeps only
# the tail of stdout must still get it whole); everything else goes to the
# detail file.
SUMMARY_KEYS = ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "pct_of_hbm_peak", "busbw_emulated_GBps", "roofline", "cpu_baseline",
                "pct_of_copy_ceiling", "alpha_us", "detail_file")
SUMMARY_MAX_CHARS = 4096


def summary_line(result):
    """The one-line record printed last: the headline, its roofline and CPU
    baseline, the copy ceiling, the step latency, every algorithm's time on the
    headline workload and, per rank count, the ring/tree crossover (measured
    and from the pages' model)."""
    out = {k: result[k] for k in SUMMARY_KEYS if k in result}
    if "ceiling" in result:
        out["copy_ceiling_GBps"] = result["ceiling"].get("GBps")
        out["resident_copy_ceiling_GBps"] = result["ceiling"].get("resident_GBps")
    if "variants" in result:
        out["algos_ms"] = {k: v["ms"] for k, v in result["variants"].items()}
    fit = result.get("alpha", {}).get("fit")
    if fit:
        out["crossover_S_per_rank"] = {
            p: [rec.get("largest_S_per_rank_where_tree_beats_ring"),
                rec.get("model_crossover_S_per_rank")] for p, rec in fit.items()}
        out["fused_not_fastest"] = [x for rec in fit.values() for x in rec.get("not_fused_fastest", [])]
    line = json.dumps(out)
    if len(line) > SUMMARY_MAX_CHARS:
        # never let the headline grow past what a tail reader keeps
        for k in ("fused_not_fastest", "crossover_S_per_rank", "algos_ms"):
            out.pop(k, None)
            if len(json.dumps(out)) <= SUMMARY_MAX_CHARS:
                break
    return out


def write_detail(path, result):
    if not path:
        return
    os.makedirs(os.path.dirname(path) or ".", exist_ok=True)
    with open(path, "w") as f:
        json.dump(result, f, indent=1)
    log(f"full record in {path}")


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: the library runs the ring "
              "schedule's p virtual ranks inside ONE GPU's HBM; nothing crosses GPUs, so "
              "only --gpus 1 is measured.", file=sys.stderr)
        sys.exit(2)

    import torch
    from ring_all_reduce_schedule_amd import binding as B
    from ring_all_reduce_schedule_amd import inputs

    if not torch.cuda.is_available():
        print("bench.py needs a ROCm GPU", file=sys.stderr)
        sys.exit(1)
    B.lib()   # fails loudly if libra.so is missing
    torch.cuda.set_device(0)

    if args.mode == "copy":
        # counter calibration: one plain copy of 2 x 16 GiB traffic
        nbytes = 16 << 30
        src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(2):
            B.ra_stream_copy(dst, src)
        per, _ = time_calls(lambda: B.ra_stream_copy(dst, src), 3, torch)
        print(json.dumps({"mode": "copy", "bytes_read": nbytes, "bytes_written": nbytes,
                          "ms": [round(x, 3) for x in per],
                          "GBps": round(2 * nbytes / (min(per) * 1e-3) / 1e9, 1)}), flush=True)
        return

    log(f"allocating workload {args.workload}")
    w, bufs = alloc_workload(args.workload, torch, B, inputs)
    p, n, dtype = w["p"], w["n"], w["dtype"]
    item = inputs.ITEMSIZE[dtype]
    S = n * item
    min_bytes = 2 * p * S
    ranks = B.RankBuffers(bufs)   # checked and marshalled once; refills are in place

    step_opts = {k: v for k, v in (("grid", args.grid), ("channels", args.channels),
                                   ("group", args.group)) if v}

    if args.mode in ("reduce_scatter", "all_gather"):
        # one phase alone, for counter runs: its time and byte counts only
        f = B.ra_reduce_scatter_ex if args.mode == "reduce_scatter" else B.ra_all_gather_ex
        fn = lambda: f(ranks, algo=args.algo, **step_opts)
        for _ in range(args.warmup):
            fn()
        B.ra_stream_status()
        per, _ = time_calls(fn, args.steps, torch)
        B.ra_stream_status()
        floor, moved = phase_bytes(args.mode, args.algo, p, S)
        print(json.dumps({"mode": args.mode, "algo": args.algo, "workload": args.workload,
                          "ms": [round(x, 3) for x in per], "bytes_floor": floor,
                          "bytes_moved": moved}), flush=True)
        return

    def step():
        B.ra_allreduce_ex(ranks, algo=args.algo, **step_opts)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    B.ra_stream_status()
    # outputs of every rank must agree bit for bit
    for r in range(1, p):
        a, b = bufs[0], bufs[r]
        if dtype == "bfloat16":
            a, b = a.view(torch.int16), b.view(torch.int16)
        if not torch.equal(a, b):
            raise SystemExit(f"rank {r} differs from rank 0 after the all-reduce")

    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    per, span = time_calls(step, args.steps, torch)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    B.ra_stream_status()
    ms_per_step = span / args.steps
    value = min_bytes / (ms_per_step * 1e-3) / 1e9
    launch_ms = sum(per) / len(per)
    # the roofline rates the timed kernel on the bytes it must move itself
    # (2pS for the fused pass; the other algorithms move more, see own_bytes)
    kernel_bytes = own_bytes(args.algo, p, S)
    achieved = kernel_bytes / (launch_ms * 1e-3) / 1e9
    sha = kernel_source_sha()
    # the committed counter summary covers the fused kernel only
    traffic, traced = read_traffic(sha, min_bytes) if args.algo == "fused" else (None, None)
    # the kernel the counter run traced; without one, the one-pass family (the
    # library runs it in read/write phases where those pay, see include/ra.h)
    kernel = traced or (f"ra::k_fused<{dtype}>" if args.algo == "fused" else args.algo)

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": {"bfloat16": "bf16", "float32": "f32", "int32": "int32"}[dtype],
        "data": "synthetic (seeded normal/uniform draws, generated in HBM or on the host)",
        "config": {"workload": args.workload, "p": p, "n_per_rank": n,
                   "bytes_per_rank": S, "algo": args.algo, **step_opts,
                   "bytes_counted": "2*p*S (each rank buffer read once and written once)",
                   "bytes_per_step": min_bytes},
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        # nccl-tests' bus bandwidth, 2(p-1)/p * S / t: the rate each rank's links
        # would carry; here emulated, no link is involved
        "busbw_emulated_GBps": round(2 * (p - 1) / p * S / (ms_per_step * 1e-3) / 1e9, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic, "kernel": kernel,
                     "algorithmic_bytes": kernel_bytes,
                     "launch_ms_mean": round(launch_ms, 4),
                     "launch_ms_min": round(min(per), 4),
                     "kernel_source_sha": sha},
        "wall_s_timed": round(wall, 3),
    }

    if not args.no_extras:
        log("variants")
        fill_workload(args.workload, bufs, torch, inputs)
        variants = {}
        runs = [(a, a, {}) for a in ("ring_step", "ring_pipelined", "ring_pipelined_flags",
                                     "ring_bidir", "ring_channels",
                                     "tree")]
        runs += [(a, a, {"group": hier_group(p)}) for a in ("hier", "hier_fused")]
        # the step ring on one persistent grid with device-wide barriers between
        # steps (the library's default persistent grid: 3 workgroups per CU)
        cus = torch.cuda.get_device_properties(0).multi_processor_count
        runs += [("ring_step_persistent", "ring_step", {"grid": 3 * cus})]
        # the one-pass all-reduce without read/write phases (the library picks the
        # phases by itself for this workload)
        runs += [("fused_no_phases", "fused", {"flags": B.RA_FLAG_NO_PHASES})]
        runs += [("fused_wide_fp32_accumulate", "fused", {"wide": True}),
                 ("fused_avg", "fused", {"op": "avg"}), ("fused_max", "fused", {"op": "max"})]
        for name, algo, kw in runs:
            fn = lambda a=algo, k=kw: B.ra_allreduce_ex(ranks, algo=a, **k)
            fill_workload(args.workload, bufs, torch, inputs)
            fn()
            B.ra_stream_status()
            vper, _ = time_calls(fn, 3, torch)
            B.ra_stream_status()
            t = sum(vper) / len(vper)
            moved = own_bytes(algo, p, S)
            variants[name] = {"ms": round(t, 3), "GBps_on_2pS": round(min_bytes / (t * 1e-3) / 1e9, 1),
                              "hbm_bytes": moved,
                              "GBps_on_hbm_bytes": round(moved / (t * 1e-3) / 1e9, 1),
                              "pct_peak_on_hbm_bytes": round(100 * moved / (t * 1e-3) / 1e9
                                                             / HBM_PEAK_GBPS, 2)}
            if "group" in kw:
                variants[name]["group"] = kw["group"]
        result["variants"] = variants
        log("standalone phases")
        fill_workload(args.workload, bufs, torch, inputs)
        result["phases"] = phase_measure(ranks, S, p, torch, B)
        log("copy ceiling")
        # the same byte count as the all-reduce, read + write, through a plain copy
        half = min_bytes // 2
        chunk = min(half, 8 << 30)
        src = bufs[0].view(torch.int16)[: chunk // 2]
        dst = bufs[1].view(torch.int16)[: chunk // 2]
        cper, _ = time_calls(lambda: B.ra_stream_copy(dst, src), 5, torch)
        # the same copy on the persistent kernels' default resident grid, their
        # own streaming ceiling
        rper, _ = time_calls(lambda: B.ra_stream_copy_resident(dst, src), 5, torch)
        result["ceiling"] = {"kernel": "ra::k_copy", "bytes_moved": 2 * chunk,
                             "GBps": round(2 * chunk / (min(cper) * 1e-3) / 1e9, 1),
                             "resident_kernel": "ra::k_copy_resident",
                             "resident_GBps": round(2 * chunk / (min(rper) * 1e-3) / 1e9, 1)}
        for v in result["variants"].values():
            v["pct_of_copy_on_hbm_bytes"] = round(
                100 * v["GBps_on_hbm_bytes"] / result["ceiling"]["GBps"], 1)
        if "GBps" in result["ceiling"] and result["ceiling"]["GBps"]:
            result["pct_of_copy_ceiling"] = round(100.0 * value / result["ceiling"]["GBps"], 2)

    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        fill_workload(args.workload, bufs, torch, inputs)
        result["cpu_baseline"] = cpu_baseline(bufs, w, args.cpu_sample, torch)

    if not args.no_extras:
        del bufs, ranks
        torch.cuda.empty_cache()
        log("per-workload rates")
        result["per_workload"] = per_workload(torch, B, inputs)
        if not args.no_cpu_baseline:
            log("cpu baseline per workload (oracle, in full)")
            result["cpu_baseline_per_workload"] = cpu_baseline_workloads(inputs)
        log("alpha")
        result["alpha"] = alpha_measure(torch, B, inputs)
        result["alpha_us"] = result["alpha"]["in_kernel_step_us_p64_1KiB"]

    # everything measured goes to the detail file; stdout ends with the short line
    write_detail(args.detail, result)
    result["detail_file"] = os.path.relpath(args.detail, ROOT) if args.detail else None
    print(json.dumps(summary_line(result)), flush=True)


if __name__ == "__main__":
    main()
