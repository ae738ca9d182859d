"""GPU parity on the five named workloads at their full sizes (through the C ABI).

p8_bf16_16GB (128 GB of inputs) is drawn on the device and checked on sampled
windows: every chunk edge +-64 Ki elements, the windows around element 2**31
and 2**32 and around byte offset 2**32, and 16 random 1 Mi-element windows.
Inputs of every window are copied to the host before the all-reduce runs; the
oracle's windowed ring fold gives the expected values.  All p outputs are also
checked to be bitwise identical on the device.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff
from tests.test_gpu_parity import ALL, RING, expected as _expected, TOL

# every all-reduce algorithm and the order the oracle folds it in
WIDE_ALL = ALL + ["ring_channels", "hier", "hier_fused"]


def expected(xs, dtype, algo):
    if algo == "ring_channels":
        return oracle.ring_fold(xs, dtype)
    if algo in ("hier", "hier_fused"):
        return oracle.hier_fold(xs, dtype, _group(len(xs)))
    return _expected(xs, dtype, algo)


def _group(p):
    """The library's default ranks per node: the largest divisor of p up to 8."""
    return next(g for g in range(min(p, 8), 0, -1) if p % g == 0)

pytestmark = pytest.mark.gpu


def _run_full(name, algo):
    w = inputs.WORKLOADS[name]
    dtype = w["dtype"]
    xs = inputs.workload_inputs(name)
    want = expected(xs, dtype, algo)
    t = to_dev(xs, dtype)
    print(f"[case] workload={name} algo={algo}", flush=True)
    B.ra_allreduce_ex(t, algo=algo)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r, g in enumerate(got):
        assert same_bits(g, want, dtype), f"rank {r} first diff {first_diff(g, want, dtype)}"
    if algo == "tree" and dtype != "int32":
        err = oracle.normwise_error(oracle.as_values(got[0], dtype), oracle.exact_sum(xs, dtype))
        assert err <= TOL[dtype]
    del t
    torch.cuda.empty_cache()


@pytest.mark.parametrize("algo", WIDE_ALL)
def test_p9_int32(algo):
    require_gpu()
    _run_full("p9_int32_n1000003", algo)
    # integers: every algorithm gives the exact (wrapped) sum
    xs = inputs.workload_inputs("p9_int32_n1000003")
    assert np.array_equal(expected(xs, "int32", algo),
                          np.sum(np.stack(xs).astype(np.int64), axis=0).astype(np.int32))


@pytest.mark.parametrize("algo", WIDE_ALL)
def test_p64_bf16(algo):
    require_gpu()
    _run_full("p64_bf16_1MiB", algo)


@pytest.mark.parametrize("algo", WIDE_ALL)
def test_p8_fp32(algo):
    require_gpu()
    _run_full("p8_fp32_256MiB", algo)


def _windows(n, p, seed):
    bounds = oracle.chunk_bounds(n, p)
    half = 1 << 16
    wins = []
    for lo, _ in bounds[1:]:
        wins.append((lo - half, lo + half))
    for x in (2**31, 2**32, n - 1):     # elements 2^31 (= byte 2^32 of bf16) and 2^32
        wins.append((x - half, x + half))
    rng = np.random.default_rng(seed)
    for s in rng.integers(0, n - (1 << 20), 16):
        wins.append((int(s), int(s) + (1 << 20)))
    wins.append((0, 1 << 16))
    return sorted(set((max(0, a), min(n, b)) for a, b in wins))


@pytest.mark.parametrize("algo", ["fused", "hier_fused", "ring_step", "tree", "ring_bidir",
                                  "ring_channels", "ring_pipelined", "ring_pipelined_flags",
                                  "hier"])
def test_p8_bf16_16GB_windowed(algo):
    dev = require_gpu()
    w = inputs.WORKLOADS["p8_bf16_16GB"]
    p, n = w["p"], w["n"]
    free, _ = torch.cuda.mem_get_info(dev)
    need = p * n * 2
    assert free > need + (4 << 30), f"needs {need / 2**30:.0f} GiB of HBM, {free / 2**30:.0f} free"
    print(f"[case] workload=p8_bf16_16GB algo={algo}: drawing inputs", flush=True)
    t = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    inputs.device_normal_bf16(t, w["sigma"], w["seed"])
    wins = _windows(n, p, w["seed"])
    before = [[x[a:b].view(torch.int16).cpu().numpy().view(np.uint16) for x in t] for a, b in wins]
    torch.cuda.synchronize()
    # the hierarchical algorithms as two nodes of four ranks
    opts = {"group": 4} if algo.startswith("hier") else {}
    print(f"[case] workload=p8_bf16_16GB algo={algo} {opts}: running", flush=True)
    B.ra_allreduce_ex(t, algo=algo, **opts)
    B.ra_stream_status()
    for r in range(1, p):
        assert torch.equal(t[0].view(torch.int16), t[r].view(torch.int16)), f"rank {r} != rank 0"
    for (a, b), xw in zip(wins, before):
        if algo in ("hier_fused", "hier"):
            want = oracle.hier_fold_window(xw, a, n, "bfloat16", 4)
        elif algo == "ring_bidir":
            want = oracle.bidir_fold_window(xw, a, n, "bfloat16")
        elif algo == "tree":
            # the tree's order is the same for every element: fold whole windows
            want = oracle.tree_allreduce(xw, "bfloat16")[0][0]
        else:
            want = oracle.ring_fold_window(xw, a, n, "bfloat16")
        got = t[0][a:b].view(torch.int16).cpu().numpy().view(np.uint16)
        assert same_bits(got, want, "bfloat16"), f"window {a}:{b} first diff {first_diff(got, want, 'bfloat16')}"
    del t
    torch.cuda.empty_cache()
