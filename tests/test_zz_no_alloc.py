"""ra_allreduce_noalloc (through the C ABI) against ra_allreduce_ex.

The entry point for callers that cannot allocate takes the persistent grids'
workspace from a fixed array in the library's device data instead of the
per-stream workspace.  Every result must equal ra_allreduce_ex's on the same
inputs bit for bit (and the oracle's), on two calls in a row, the second on a
smaller input; calls beyond the array's capacity are refused; a device-side
timeout stays sticky in the array until ra_stream_status reports it; and a call
captured in a HIP graph gives the eager result on every replay.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

CASES = [  # (algo, options): every kind of workspace use, and none
    ("ring_pipelined_flags", {}), ("ring_pipelined_flags", {"slice_elems": 4096, "grid": 64}),
    ("ring_step", {"grid": 64}), ("ring_step", {"grid": 1}), ("ring_channels", {}),
    ("ring_channels", {"channels": 3, "grid": 24}), ("tree", {"grid": 32}),
    ("ring_bidir", {"grid": 16}), ("hier", {"grid": 40, "group": 2}),
    ("ring_step", {"grid": 4}), ("ring_channels", {"channels": 2, "grid": 4}),
    ("ring_step", {}), ("fused", {}), ("ring_pipelined", {}),
]


def _clear():
    """Report and clear whatever an earlier failing call left in the array."""
    try:
        B.ra_stream_status()
    except B.RaError as e:
        assert e.code == B.RA_ERR_TIMEOUT


def _want(xs, dtype, algo, opts):
    if algo == "tree":
        return oracle.tree_allreduce(xs, dtype)[0][0]
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype)[0][0]
    if algo == "hier":
        return oracle.hier_fold(xs, dtype, opts["group"])
    return oracle.ring_fold(xs, dtype)


@pytest.mark.parametrize("algo,opts", CASES)
def test_noalloc_matches_allreduce_ex_twice(algo, opts):
    require_gpu()
    _clear()
    # the second call is smaller: fewer slices, fewer tiles, other chunk edges
    for k, (p, n, dtype) in enumerate([(8, 300_007, "bfloat16"), (4, 20_011, "float32")]):
        xs = inputs.make_inputs(p, n, dtype, seed=100 * k + len(algo), sigma=1.0)
        a, b = to_dev(xs, dtype), to_dev(xs, dtype)
        print(f"[case] noalloc call {k} algo={algo} {opts} p={p} n={n} {dtype}", flush=True)
        B.ra_allreduce_noalloc(a, algo=algo, **opts)
        B.ra_allreduce_ex(b, algo=algo, **opts)
        B.ra_stream_status()
        got, ref = from_dev(a, dtype), from_dev(b, dtype)
        want = _want(xs, dtype, algo, opts)
        for r in range(p):
            assert same_bits(got[r], ref[r], dtype), f"call {k} rank {r} at {first_diff(got[r], ref[r], dtype)}"
            assert same_bits(got[r], want, dtype), f"call {k} rank {r} vs oracle"


def test_noalloc_refuses_more_counters_than_it_holds():
    require_gpu()
    _clear()
    p, n = 8, 1 << 25
    t = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
    # slices of 8 elements round up to one 128-byte line (64 bfloat16): 65,536
    # per chunk, 524,288 counters
    with pytest.raises(B.RaError) as e:
        B.ra_allreduce_noalloc(t, algo="ring_pipelined_flags", slice_elems=8)
    assert e.value.code == B.RA_ERR_UNSUPPORTED
    B.ra_stream_status()
    # the ordinary entry point has no such limit
    B.ra_allreduce_ex(t, algo="ring_pipelined_flags", slice_elems=8)
    B.ra_stream_status()


def test_noalloc_counters_past_two_to_the_31_and_back():
    """The array's counter numbering jumps to 2^31 (test hook: the counters are
    zeroed by a kernel, not reallocated); calls before and after stay exact."""
    require_gpu()
    _clear()
    for k, flags in enumerate([0, B.RA_FLAG_RENEW_COUNTERS, 0, 0]):
        p, n = 8, 200_003 - 1000 * k
        xs = inputs.make_inputs(p, n, "bfloat16", seed=70 + k, sigma=1.0)
        t = to_dev(xs, "bfloat16")
        print(f"[case] noalloc counters call {k} flags={flags}", flush=True)
        B.ra_allreduce_noalloc(t, algo="ring_pipelined_flags", slice_elems=2048, flags=flags)
        B.ra_stream_status()
        want = oracle.ring_fold(xs, "bfloat16")
        for r, g in enumerate(from_dev(t, "bfloat16")):
            assert same_bits(g, want, "bfloat16"), f"call {k} rank {r}"


def test_noalloc_timeout_is_sticky_until_reported():
    require_gpu()
    _clear()
    p, n = 4, 40_000
    xs = inputs.make_inputs(p, n, "float32", seed=5)
    t = to_dev(xs, "float32")
    print("[case] noalloc forced timeout", flush=True)
    B.ra_allreduce_noalloc(t, algo="ring_step", grid=8, timeout_us=2000,
                           flags=B.RA_FLAG_FORCE_TIMEOUT)
    torch.cuda.synchronize()
    # a later persistent call on the same GPU does no work while the error stands
    u = to_dev(xs, "float32")
    B.ra_allreduce_noalloc(u, algo="ring_step", grid=8)
    with pytest.raises(B.RaError) as e:
        B.ra_stream_status()
    assert e.value.code == B.RA_ERR_TIMEOUT
    assert all(same_bits(g, x, "float32") for g, x in zip(from_dev(u, "float32"), xs))
    # cleared: the next call works
    B.ra_allreduce_noalloc(u, algo="ring_step", grid=8)
    B.ra_stream_status()
    want = oracle.ring_fold(xs, "float32")
    assert all(same_bits(g, want, "float32") for g in from_dev(u, "float32"))


@pytest.mark.parametrize("algo,opts", [("ring_step", {"grid": 64}), ("fused", {}),
                                       ("ring_pipelined", {}), ("ring_pipelined_flags", {}),
                                       ("ring_channels", {"channels": 8, "grid": 64})])
def test_noalloc_in_a_hip_graph(algo, opts):
    """Captured once, replayed three times with eager work and synchronisation
    between the replays; the maximum is idempotent, so every replay must give
    the eager result exactly."""
    require_gpu()
    _clear()
    p, n = 8, 100_003
    xs = inputs.make_inputs(p, n, "bfloat16", seed=9, sigma=1.0)
    eager = to_dev(xs, "bfloat16")
    B.ra_allreduce_noalloc(eager, algo=algo, op="max", **opts)   # also sets up the array
    B.ra_stream_status()
    want = from_dev(eager, "bfloat16")
    assert same_bits(want[0], oracle.ring_fold(xs, "bfloat16", op="max"), "bfloat16")
    t = to_dev(xs, "bfloat16")
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    print(f"[case] noalloc graph capture algo={algo}", flush=True)
    with torch.cuda.graph(g):
        B.ra_allreduce_noalloc(t, algo=algo, op="max", **opts)
    for rep in range(3):
        for r in range(p):
            t[r].copy_(to_dev([xs[r]], "bfloat16")[0])
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        B.ra_stream_status()
        got = from_dev(t, "bfloat16")
        for r in range(p):
            assert same_bits(got[r], want[r], "bfloat16"), f"replay {rep} rank {r}"
        # eager work between replays
        _ = (eager[0].float() * 2).sum().item()
