"""GPU parity of the one-pass all-reduce run in read and write phases (through the C ABI).

RA_FLAG_PHASES forces the phased kernel at any size, so these cases reach it with
one rank, ragged chunks, chunk edge elements, more ranks than one batch of loads
(9, 16, 64), every element type and reduction and the wide accumulation; each
result must equal the oracle's ring order bit for bit, as the plain pass does.
The library picks the phases by itself only for all-reduces and all-gathers of 8
ranks of at least 12 GiB each: the full-size workload tests (8 x 16 GB bfloat16) check that default path,
and a 1.6 GB case here compares the phases with the plain pass on the same inputs.
"""

import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

PHASES = B.RA_FLAG_PHASES
NO_PHASES = B.RA_FLAG_NO_PHASES
DTYPES = ["int32", "int64", "float16", "bfloat16", "float32", "float64"]
FLOATS = ["float16", "bfloat16", "float32", "float64"]


def make(p, n, dtype, seed):
    if dtype == "int64":
        return inputs.make_inputs(p, n, dtype, seed, lo=-2**62, hi=2**62)
    return inputs.make_inputs(p, n, dtype, seed, sigma=3.0)


def check(xs, dtype, op="sum", wide=False, flags=PHASES):
    t = to_dev(xs, dtype)
    print(f"[case] fused phases flags={flags} op={op} wide={wide} p={len(xs)} n={len(xs[0])} "
          f"dtype={dtype}", flush=True)
    B.ra_allreduce_ex(t, algo="fused", op=op, wide=wide, flags=flags)
    B.ra_stream_status()
    want = oracle.ring_fold(xs, dtype, op=op, wide=wide)
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want, dtype), f"rank {r} first diff {first_diff(g, want, dtype)}"


SIZES = [(1, 1000), (2, 7), (3, 17), (4, 4096), (5, 1023), (8, 100_003), (8, 1 << 20),
         (9, 1_000_003), (16, 70_001), (64, 4097)]


@pytest.mark.parametrize("dtype", ["int32", "bfloat16", "float32"])
@pytest.mark.parametrize("p,n", SIZES)
def test_forced_phases_match_oracle(p, n, dtype):
    require_gpu()
    check(make(p, n, dtype, seed=7 * p + n), dtype)


DTYPE_OPS = [(d, o) for d in DTYPES for o in ("sum", "max", "avg") if o != "avg" or d in FLOATS]


@pytest.mark.parametrize("dtype,op", DTYPE_OPS)
def test_forced_phases_every_type_and_reduction(dtype, op):
    require_gpu()
    check(make(8, 100_003, dtype, seed=11), dtype, op=op)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
@pytest.mark.parametrize("op", ["sum", "avg"])
def test_forced_phases_wide_accumulation(dtype, op):
    require_gpu()
    check(make(6, 50_001, dtype, seed=13), dtype, op=op, wide=True)


def test_no_phases_wins_over_phases():
    require_gpu()
    check(make(8, 4099, "bfloat16", seed=17), "bfloat16", flags=PHASES | NO_PHASES)


def test_forced_phases_same_bits_as_plain_pass_large():
    """8 ranks x 200 MB bfloat16 (streaming, 48 rounds of the grid, so the
    default stays with the plain pass) forced into phases, against the plain
    pass on the same inputs and the oracle around every chunk boundary."""
    require_gpu()
    p, n = 8, 100_000_005          # ragged: edge elements at the chunk ends
    g = torch.Generator(device="cuda:0").manual_seed(23)
    src = [torch.randn(n, generator=g, device="cuda:0").mul_(1e-2).to(torch.bfloat16)
           for _ in range(p)]
    starts = [lo for lo, _ in oracle.chunk_bounds(n, p)][1:]
    wins = [(max(0, c - 40), min(n, c + 40)) for c in starts]
    xw = [[s[a:b].cpu().view(torch.int16).numpy().view("uint16").copy() for s in src]
          for a, b in wins]
    a = [s.clone() for s in src]
    print(f"[case] forced phases vs plain pass p={p} n={n} bfloat16", flush=True)
    B.ra_allreduce_ex(a, algo="fused", flags=PHASES)
    B.ra_stream_status()
    b = [s.clone() for s in src]
    B.ra_allreduce_ex(b, algo="fused", flags=NO_PHASES)
    B.ra_stream_status()
    for r in range(p):
        assert torch.equal(a[r].view(torch.int16), b[r].view(torch.int16)), f"rank {r}"
    for (lo, hi), x in zip(wins, xw):
        want = oracle.ring_fold_window(x, lo, n, "bfloat16")
        got = a[3][lo:hi].cpu().view(torch.int16).numpy().view("uint16")
        assert (got == want).all(), f"window {lo}"


def test_forced_phases_graph_replays():
    require_gpu()
    p, n, dtype = 8, 300_007, "bfloat16"
    xs = inputs.make_inputs(p, n, dtype, seed=29)
    src = to_dev(xs, dtype)
    bufs = [torch.empty_like(s) for s in src]
    for b, s in zip(bufs, src):
        b.copy_(s)
    B.ra_allreduce_ex(bufs, algo="fused", flags=PHASES)
    B.ra_stream_status()
    want = oracle.ring_fold(xs, dtype)
    assert all(same_bits(e, want, dtype) for e in from_dev(bufs, dtype))
    g = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    print("[case] graph capture of the phased pass", flush=True)
    with torch.cuda.graph(g, stream=cap):
        B.ra_allreduce_ex(bufs, algo="fused", flags=PHASES)
    torch.cuda.synchronize()
    for k in range(4):
        for b, s in zip(bufs, src):           # eager work between replays
            b.copy_(s)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for r, got in enumerate(from_dev(bufs, dtype)):
            assert same_bits(got, want, dtype), f"replay {k} rank {r} at {first_diff(got, want, dtype)}"


@pytest.mark.parametrize("p,n,dtype", [(2, 7, "float32"), (3, 1_003, "int32"),
                                       (8, 100_003, "bfloat16"), (9, 300_001, "float32"),
                                       (16, 70_001, "bfloat16")])
def test_forced_phases_reduce_scatter_then_all_gather(p, n, dtype):
    """The fused reduce-scatter (each rank's owned chunk folded in ring order, the
    other chunks left as they were) and the fused all-gather (each owner's chunk
    copied to the other ranks) in phases, against the oracle."""
    require_gpu()
    xs = inputs.make_inputs(p, n, dtype, seed=31 * p + n, sigma=1.0)
    t = to_dev(xs, dtype)
    print(f"[case] RS/AG fused phases p={p} n={n} dtype={dtype}", flush=True)
    B.ra_reduce_scatter_ex(t, algo="fused", flags=PHASES)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r in range(p):
        want = oracle.rs_owned(xs, dtype, r)
        assert same_bits(got[r], want, dtype), f"rank {r} at {first_diff(got[r], want, dtype)}"
    B.ra_all_gather_ex(t, algo="fused", flags=PHASES)
    B.ra_stream_status()
    want = oracle.ring_fold(xs, dtype)
    for r, f in enumerate(from_dev(t, dtype)):
        assert same_bits(f, want, dtype), f"rank {r} at {first_diff(f, want, dtype)}"
    # the all-gather alone on buffers that hold arbitrary values
    t = to_dev(xs, dtype)
    B.ra_all_gather_ex(t, algo="fused", flags=PHASES)
    B.ra_stream_status()
    want, _ = oracle.all_gather(xs, dtype)
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want[r], dtype), f"all-gather rank {r} at {first_diff(g, want[r], dtype)}"


def test_forced_phases_on_two_streams_at_once():
    """Two phased all-reduces on separate buffers and streams, enqueued together:
    their grids share the compute units (the kernel has no waits between
    workgroups, so a workgroup that starts late only joins a later window), and
    each result must still equal the oracle's."""
    require_gpu()
    dtype = "bfloat16"
    cases = [inputs.make_inputs(8, 400_003, dtype, seed=41), inputs.make_inputs(8, 250_001, dtype, seed=43)]
    devs = [to_dev(xs, dtype) for xs in cases]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    print("[case] two streams, forced phases", flush=True)
    torch.cuda.synchronize()
    for t, st in zip(devs, streams):
        B.ra_allreduce_ex(t, algo="fused", flags=PHASES, stream=st)
    for st in streams:
        B.ra_stream_status(st)
    torch.cuda.synchronize()
    for xs, t in zip(cases, devs):
        want = oracle.ring_fold(xs, dtype)
        for r, g in enumerate(from_dev(t, dtype)):
            assert same_bits(g, want, dtype), f"rank {r} first diff {first_diff(g, want, dtype)}"
