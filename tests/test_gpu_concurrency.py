"""Concurrent callers (through the C ABI).

Four host threads, each with its own stream and its own rank buffers, issue
interleaved sequences of all-reduces with every algorithm.  The library keeps
its workspace per (device, stream) behind a lock and its error text per
thread; the default step launches use no workspace at all.  Persistent grids
(channels, flag-driven pipelined) are given 32 workgroups each so that all four can be
resident together.  Every result must equal the oracle's, bit for bit.
"""

import random
import threading

import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

ALGOS = ["fused", "ring_step", "tree", "ring_bidir", "hier", "hier_fused", "ring_channels",
         "ring_pipelined", "ring_pipelined_flags"]


def _want(xs, dtype, algo):
    if algo == "tree":
        return oracle.tree_allreduce(xs, dtype)[0][0]
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype)[0][0]
    if algo in ("hier", "hier_fused"):
        return oracle.hier_fold(xs, dtype, 2)
    return oracle.ring_fold(xs, dtype)


def _worker(tid, errors):
    try:
        rng = random.Random(1000 + tid)
        stream = torch.cuda.Stream()
        with torch.cuda.stream(stream):
            for k in range(12):
                p = rng.choice([4, 8])
                n = rng.choice([100, 3_000, 40_000, 200_003])
                dtype = rng.choice(["int32", "float32", "bfloat16"])
                algo = rng.choice(ALGOS)
                xs = inputs.make_inputs(p, n, dtype, seed=tid * 100 + k)
                t = to_dev(xs, dtype)
                opts = {"group": 2} if algo.startswith("hier") else {}
                if algo in ("ring_channels", "ring_pipelined_flags"):
                    opts["grid"] = 32
                B.ra_allreduce_ex(t, algo=algo, **opts)
                B.ra_stream_status(stream=stream)
                want = _want(xs, dtype, algo)
                for r, g in enumerate(from_dev(t, dtype)):
                    if not same_bits(g, want, dtype):
                        errors.append(f"thread {tid} call {k} {algo} p={p} n={n} {dtype} rank {r} "
                                      f"first diff {first_diff(g, want, dtype)}")
                        return
    except Exception as e:  # reported by the main thread
        errors.append(f"thread {tid}: {e!r}")


def test_four_threads_four_streams():
    require_gpu()
    print("[case] four threads, four streams, mixed algorithms", flush=True)
    errors = []
    threads = [threading.Thread(target=_worker, args=(i, errors)) for i in range(4)]
    for th in threads:
        th.start()
    for th in threads:
        th.join(timeout=240)
    assert not any(th.is_alive() for th in threads), "a worker thread did not finish"
    assert not errors, errors
