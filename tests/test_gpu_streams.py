"""Streams and graphs (through the C ABI).

* Two streams run all-reduces concurrently, each on its own buffers: the
  library keeps one workspace (barrier words, status) per (device, stream), so
  the grid barriers of concurrent step-by-step calls never mix.  Each call is
  given 64 workgroups so that both persistent grids are resident together.
* The same with the library's default launches (one launch per step), which
  use no workspace and need no co-residency.
* The one-pass algorithms, and the step algorithms' default launches (one
  workgroup for tiny steps, one launch per step otherwise), are ordinary
  kernels with no workspace, so they can be captured into a HIP graph -- on a
  stream that has never run a call; every replay (with eager work and
  synchronisation in between) must equal the eager result.
* Persistent grids (a caller's grid, channels, the flag-driven pipelined ring)
  are captured on a stream that has made such a call; replays alternate with
  eager flag-driven calls on the same stream.  Capturing one on a stream with no
  workspace fails cleanly.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("algo,grid", [("ring_step", 64), ("tree", 64), ("hier", 64),
                                       ("ring_channels", 64), ("ring_pipelined_flags", 64),
                                       ("ring_pipelined", 0),
                                       ("ring_step", 0), ("tree", 0), ("hier", 0), ("ring_bidir", 0)])
def test_two_streams_at_once(algo, grid):
    require_gpu()
    p, n, dtype = 8, 300_007, "float32"
    xa = inputs.make_inputs(p, n, dtype, seed=1)
    xb = inputs.make_inputs(p, n, dtype, seed=2)
    want = {"tree": lambda x: oracle.tree_allreduce(x, dtype)[0][0],
            "hier": lambda x: oracle.hier_fold(x, dtype, 8),
            "ring_bidir": lambda x: oracle.bidir_allreduce(x, dtype)[0][0]}.get(
                algo, lambda x: oracle.ring_fold(x, dtype))
    ta, tb = to_dev(xa, dtype), to_dev(xb, dtype)
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    print(f"[case] two streams algo={algo} grid={grid}", flush=True)
    for _ in range(3):
        # 64 workgroups each: both persistent grids fit on the GPU together
        with torch.cuda.stream(sa):
            B.ra_allreduce_ex(ta, algo=algo, grid=grid)
        with torch.cuda.stream(sb):
            B.ra_allreduce_ex(tb, algo=algo, grid=grid)
        B.ra_stream_status(stream=sa)
        B.ra_stream_status(stream=sb)
        # the next round starts from this round's result on both streams
        xa = [want(xa)] * p
        xb = [want(xb)] * p
        for r, g in enumerate(from_dev(ta, dtype)):
            assert same_bits(g, xa[0], dtype), f"stream a rank {r} at {first_diff(g, xa[0], dtype)}"
        for r, g in enumerate(from_dev(tb, dtype)):
            assert same_bits(g, xb[0], dtype), f"stream b rank {r} at {first_diff(g, xb[0], dtype)}"


STEP_CALLS = {"allreduce_ring_step": "ring_step", "allreduce_tree": "tree",
              "allreduce_hier": "hier", "allreduce_ring_bidir": "ring_bidir",
              "allreduce_ring_step_tiny": "ring_step", "allreduce_tree_tiny": "tree"}


def _graph_want(call, xs, dtype):
    algo = STEP_CALLS.get(call)
    if call == "allreduce_hier_fused" or algo == "hier":
        return oracle.hier_fold(xs, dtype, 3)
    if algo == "tree":
        return oracle.tree_allreduce(xs, dtype)[0][0]
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype)[0][0]
    return oracle.ring_fold(xs, dtype)


@pytest.mark.parametrize("call", ["allreduce_fused", "allreduce_hier_fused", "rs_then_ag_fused",
                                  "rs_then_ag_ring_step"] + list(STEP_CALLS))
def test_graph_capture_and_replay(call):
    require_gpu()
    p, n, dtype = 9, (200 if call.endswith("_tiny") else 100_003), "bfloat16"
    xs = inputs.make_inputs(p, n, dtype, seed=3)
    src = to_dev(xs, dtype)
    bufs = [torch.empty_like(s) for s in src]

    def run():
        if call == "allreduce_fused":
            B.ra_allreduce_ex(bufs, algo="fused")
        elif call == "allreduce_hier_fused":
            B.ra_allreduce_ex(bufs, algo="hier_fused", group=3)
        elif call in STEP_CALLS:
            B.ra_allreduce_ex(bufs, algo=STEP_CALLS[call], group=3)
        elif call == "rs_then_ag_ring_step":
            B.ra_reduce_scatter_ex(bufs, algo="ring_step")
            B.ra_all_gather_ex(bufs, algo="ring_step")
        else:
            B.ra_reduce_scatter_ex(bufs, algo="fused")
            B.ra_all_gather_ex(bufs, algo="fused")

    # eager reference (also warms the library up before capture)
    for b, s in zip(bufs, src):
        b.copy_(s)
    run()
    B.ra_stream_status()
    eager = from_dev(bufs, dtype)
    want = _graph_want(call, xs, dtype)
    assert all(same_bits(e, want, dtype) for e in eager)

    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    print(f"[case] graph capture {call}", flush=True)
    with torch.cuda.graph(g, stream=cap):
        run()
    torch.cuda.synchronize()
    for k in range(4):
        for b, s in zip(bufs, src):           # eager work between replays
            b.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, got in enumerate(from_dev(bufs, dtype)):
            assert same_bits(got, eager[r], dtype), f"replay {k} rank {r} at {first_diff(got, eager[r], dtype)}"


# Calls that run persistent grids use the stream's workspace (barrier words, tile
# counters, ready counters), so the stream must have made such a call once before
# capture; the flag-driven ring, captured, zeroes its ready counters with a
# captured fill kernel and numbers itself from 0, while eager calls keep numbering
# from 128 up.  Replays alternate with eager calls of the same kind on the same
# stream, and each must equal the eager result.
PERSISTENT_CALLS = {"allreduce_ring_pipelined_flags": ("ring_pipelined_flags", {}),
                    "allreduce_ring_pipelined_flags_small_slices":
                        ("ring_pipelined_flags", {"slice_elems": 2048, "grid": 64}),
                    "allreduce_ring_channels": ("ring_channels", {"channels": 8}),
                    "allreduce_ring_step_grid": ("ring_step", {"grid": 40}),
                    "allreduce_tree_grid": ("tree", {"grid": 48})}


@pytest.mark.parametrize("call", list(PERSISTENT_CALLS) + ["rs_then_ag_ring_pipelined_flags"])
def test_graph_capture_persistent_grids(call):
    require_gpu()
    p, n, dtype = 8, 1_000_003, "bfloat16"
    xs = inputs.make_inputs(p, n, dtype, seed=11)
    src = to_dev(xs, dtype)
    bufs = [torch.empty_like(s) for s in src]
    other = to_dev(inputs.make_inputs(p, 300_007, dtype, seed=12), dtype)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())

    def run():
        if call == "rs_then_ag_ring_pipelined_flags":
            B.ra_reduce_scatter_ex(bufs, algo="ring_pipelined_flags")
            B.ra_all_gather_ex(bufs, algo="ring_pipelined_flags")
        else:
            algo, opts = PERSISTENT_CALLS[call]
            B.ra_allreduce_ex(bufs, algo=algo, **opts)

    algo = "tree" if call == "allreduce_tree_grid" else "ring"
    want = oracle.tree_allreduce(xs, dtype)[0][0] if algo == "tree" else oracle.ring_fold(xs, dtype)
    with torch.cuda.stream(cap):
        for b, s in zip(bufs, src):
            b.copy_(s)
        run()                                   # eager, on the capture stream
        B.ra_stream_status(stream=cap)
    eager = from_dev(bufs, dtype)
    assert all(same_bits(e, want, dtype) for e in eager)
    g = torch.cuda.CUDAGraph()
    print(f"[case] graph capture {call}", flush=True)
    with torch.cuda.graph(g, stream=cap):
        run()
    torch.cuda.synchronize()
    for k in range(4):
        with torch.cuda.stream(cap):
            # an eager flag-driven call on the same stream between replays
            B.ra_allreduce_ex(other, algo="ring_pipelined_flags")
            for b, s in zip(bufs, src):
                b.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        B.ra_stream_status(stream=cap)
        for r, got in enumerate(from_dev(bufs, dtype)):
            assert same_bits(got, eager[r], dtype), f"replay {k} rank {r} at {first_diff(got, eager[r], dtype)}"


def test_graph_capture_needs_the_streams_workspace():
    """A persistent-grid call captured on a stream that never made one cannot
    allocate its workspace during capture: it fails before enqueueing anything."""
    require_gpu()
    bufs = to_dev(inputs.make_inputs(8, 100_003, "float32", seed=13), "float32")
    fresh = torch.cuda.Stream()
    fresh.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with pytest.raises(B.RaError) as e:
        with torch.cuda.graph(g, stream=fresh):
            B.ra_allreduce_ex(bufs, algo="ring_pipelined_flags")
    assert e.value.code == B.RA_ERR_UNSUPPORTED
    torch.cuda.synchronize()
