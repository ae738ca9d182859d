"""Barrier stress (through the C ABI): with RA_FLAG_STRESS every workgroup of the
step-by-step and pipelined kernels sleeps a pseudo-random 0-25 us before each
barrier arrival and each slice hop, a different pattern on every call.  The
results must stay bit-identical to the oracle: a missing wait or fence, or a
barrier that lets a workgroup through early, would show up as wrong values."""

import pytest

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

CASES = [  # (algo, options, oracle order)
    ("ring_step", {}, "ring"), ("ring_step", {"grid": 1024}, "ring"),
    ("ring_step", {"grid": 64}, "ring"), ("ring_pipelined_flags", {}, "ring"),
    ("ring_pipelined_flags", {"slice_elems": 4096}, "ring"), ("ring_pipelined", {}, "ring"),
    ("ring_bidir", {}, "bidir"),
    ("ring_channels", {"channels": 8}, "ring"), ("ring_channels", {"channels": 3}, "ring"),
    ("tree", {}, "tree"), ("hier", {"group": 4}, "hier"), ("hier", {"group": 2}, "hier"),
]


def want(xs, dtype, order, opts, op="sum"):
    if order == "ring":
        return oracle.ring_fold(xs, dtype, op=op)
    if order == "bidir":
        return oracle.bidir_allreduce(xs, dtype, op=op)[0][0]
    if order == "tree":
        return oracle.tree_allreduce(xs, dtype, op=op)[0][0]
    return oracle.hier_fold(xs, dtype, opts["group"], op=op)


@pytest.mark.parametrize("algo,opts,order", CASES)
@pytest.mark.parametrize("p,n,dtype", [(8, 1_000_003, "float32"), (16, 300_007, "bfloat16")])
def test_stressed_allreduce(algo, opts, order, p, n, dtype):
    require_gpu()
    xs = inputs.make_inputs(p, n, dtype, seed=p + n, sigma=1.0)
    expected = want(xs, dtype, order, opts)
    for rep in range(3):
        t = to_dev(xs, dtype)
        print(f"[case] stress algo={algo} {opts} p={p} n={n} rep={rep}", flush=True)
        B.ra_allreduce_ex(t, algo=algo, flags=B.RA_FLAG_STRESS, **opts)
        B.ra_stream_status()
        for r, g in enumerate(from_dev(t, dtype)):
            assert same_bits(g, expected, dtype), f"rank {r} at {first_diff(g, expected, dtype)}"


@pytest.mark.parametrize("algo,opts", [("ring_step", {}), ("ring_pipelined", {}),
                                       ("ring_pipelined_flags", {}),
                                       ("ring_channels", {"channels": 8})])
def test_stressed_reduce_scatter_states(algo, opts):
    require_gpu()
    p, n, dtype = 9, 500_009, "float16"
    xs = inputs.make_inputs(p, n, dtype, seed=5, sigma=1.0)
    t = to_dev(xs, dtype)
    print(f"[case] stress RS algo={algo} {opts}", flush=True)
    B.ra_reduce_scatter_ex(t, algo=algo, op="avg", flags=B.RA_FLAG_STRESS, **opts)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r in range(p):
        w = oracle.rs_partial(xs, dtype, r, op="avg")
        assert same_bits(got[r], w, dtype), f"rank {r} at {first_diff(got[r], w, dtype)}"
