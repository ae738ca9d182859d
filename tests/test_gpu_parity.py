"""GPU parity: every algorithm of libra.so against the CPU oracle (through the C ABI).

Ring-ordered algorithms (ring_step, both pipelined rings, fused) and the bidirectional
rings must match the oracle bit for bit; the tree must match the oracle's tree
bit for bit and be within the normwise tolerance of the float64 sum (1e-5 for
float32, 1e-2 for bfloat16).  Integer results are exact for every algorithm.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

RING = ["fused", "ring_step", "ring_pipelined", "ring_pipelined_flags"]
ALL = RING + ["ring_bidir", "tree"]
TOL = {"float32": 1e-5, "bfloat16": 1e-2, "int32": 0.0}


def expected(xs, dtype, algo):
    """Oracle result (identical on every rank) for `algo`."""
    if algo in RING:
        return oracle.ring_fold(xs, dtype)
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype)[0][0]
    if algo == "tree":
        return oracle.tree_allreduce(xs, dtype)[0][0]
    raise ValueError(algo)


def run(xs, dtype, algo, **opts):
    t = to_dev(xs, dtype)
    print(f"[case] algo={algo} p={len(xs)} n={len(xs[0])} dtype={dtype} {opts}", flush=True)
    B.ra_allreduce_ex(t, algo=algo, **opts)
    B.ra_stream_status()
    return from_dev(t, dtype)


def check(xs, dtype, algo, **opts):
    got = run(xs, dtype, algo, **opts)
    want = expected(xs, dtype, algo)
    for r, g in enumerate(got):
        assert same_bits(g, want, dtype), f"rank {r} differs first at {first_diff(g, want, dtype)}"
    # the normwise measure needs many elements: for a handful, one sum that
    # nearly cancels makes max|exact| tiny; bit-exactness against the oracle's
    # tree order is the check that holds at every size
    if algo == "tree" and dtype in TOL and dtype != "int32" and len(want) >= 1000:
        err = oracle.normwise_error(oracle.as_values(got[0], dtype), oracle.exact_sum(xs, dtype))
        assert err <= TOL[dtype]


# ------------------------------------------------------------ worked trace

@pytest.mark.parametrize("algo", ALL)
def test_worked_trace(algo, golden):
    require_gpu()
    g = golden("trace_p4_n4.json")
    got = run(inputs.trace_inputs(), "float32", algo)
    for r in range(4):
        assert got[r].tolist() == g["expected_final_every_rank"]


# ------------------------------------------------------------ small sweep

SMALL = [(p, n) for p in (2, 3, 4, 5, 8, 9, 16, 64)
         for n in (1, 3, 7, 8, 9, 17, 100, 1023, 4097, 70_001)]


@pytest.mark.parametrize("dtype", ["int32", "float32", "bfloat16"])
@pytest.mark.parametrize("p,n", SMALL)
def test_small_sweep(p, n, dtype):
    require_gpu()
    xs = inputs.make_inputs(p, n, dtype, seed=1000 * p + n, sigma=2.0)
    for algo in ALL:
        check(xs, dtype, algo)


# Small steps run on one workgroup (its own barrier between steps); a grid
# forced above one keeps them on the device-wide barriers.  Both must agree
# with the oracle, at and around the size where the choice flips (p = 8 bf16:
# one workgroup up to 256 whole vectors per step, a chunk of 256 elements).
@pytest.mark.parametrize("grid", [0, 5])
@pytest.mark.parametrize("p,n", [(3, 1), (3, 4097), (8, 9), (8, 2048), (8, 2049), (8, 2112),
                                 (8, 2300), (64, 1023), (64, 70_001)])
def test_small_steps_one_workgroup_and_grid(p, n, grid):
    require_gpu()
    xs = inputs.make_inputs(p, n, "bfloat16", seed=7 * p + n + grid, sigma=2.0)
    for algo in ("ring_step", "ring_bidir", "tree"):
        check(xs, "bfloat16", algo, grid=grid)


# Copy steps (all-gather, tree broadcast) whose widest segment holds 8192 or more
# whole vectors launch with two vectors per thread, every other step with one.
# Sizes straddle that bound for each vector width (8 bf16, 4 int32, 2 float64
# elements), with ragged and unaligned chunk edges.
@pytest.mark.parametrize("dtype,V", [("bfloat16", 8), ("int32", 4), ("float64", 2)])
@pytest.mark.parametrize("delta", [-25, -1, 0, 5, 61])
def test_copy_steps_two_vectors_per_thread(dtype, V, delta):
    require_gpu()
    p = 3
    n = p * 8192 * V + delta
    xs = inputs.make_inputs(p, n, dtype, seed=V * 1000 + delta + 50, sigma=2.0)
    for algo in ("ring_step", "ring_bidir"):
        check(xs, dtype, algo)
    # the tree's segments are whole buffers: straddle the bound with n itself
    xt = inputs.make_inputs(2, 8192 * V + delta, dtype, seed=V + delta + 90, sigma=2.0)
    check(xt, dtype, "tree")
    # the hierarchy (2 nodes of 2): in-node chunks of n/2, cross-node pieces of n/4
    xh = inputs.make_inputs(4, 2 * 8192 * V + delta, dtype, seed=V + delta + 130, sigma=2.0)
    t = to_dev(xh, dtype)
    print(f"[case] algo=hier p=4 n={len(xh[0])} dtype={dtype}", flush=True)
    B.ra_allreduce_ex(t, algo="hier", group=2)
    B.ra_stream_status()
    want = oracle.hier_fold(xh, dtype, 2)
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want, dtype), f"hier rank {r} first diff {first_diff(g, want, dtype)}"
    # the all-gather phase alone, on buffers that hold arbitrary values
    t = to_dev(xs, dtype)
    print(f"[case] all_gather ring_step p={p} n={n} dtype={dtype}", flush=True)
    B.ra_all_gather_ex(t, algo="ring_step")
    B.ra_stream_status()
    want, _ = oracle.all_gather(xs, dtype)
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want[r], dtype), f"all-gather rank {r} first diff {first_diff(g, want[r], dtype)}"


@pytest.mark.parametrize("slice_elems,grid", [(8, 0), (24, 16), (1000, 0), (4096, 64),
                                              (1 << 20, 0), (64, 8)])
@pytest.mark.parametrize("dtype", ["float32", "bfloat16"])
def test_pipelined_slices_and_grids(slice_elems, grid, dtype):
    require_gpu()
    p, n = 9, 100_003
    xs = inputs.make_inputs(p, n, dtype, seed=slice_elems + grid, sigma=1.0)
    check(xs, dtype, "ring_pipelined_flags", slice_elems=slice_elems, grid=grid)


# The slice-carrying pipelined ring: a workgroup carries one or more 256-vector
# tiles of a chunk through all hops; chunk edges ride with slice 0.  Slices of
# 1, 2 and many tiles, chunks shorter than a tile, ragged edges.
@pytest.mark.parametrize("slice_elems", [0, 1, 2048, 2049, 5000, 1 << 20])
@pytest.mark.parametrize("p,n,dtype", [(9, 100_003, "bfloat16"), (3, 70_001, "float32"),
                                       (64, 8_195, "bfloat16"), (5, 40_960, "int32"),
                                       (2, 4_111, "float64")])
def test_pipelined_rider_slices(slice_elems, p, n, dtype):
    require_gpu()
    xs = inputs.make_inputs(p, n, dtype, seed=slice_elems % 1000 + p + n, sigma=1.0)
    check(xs, dtype, "ring_pipelined", slice_elems=slice_elems)
    # the reduce-scatter alone leaves the step-by-step partials on every chunk
    t = to_dev(xs, dtype)
    print(f"[case] RS ring_pipelined slice={slice_elems} p={p} n={n} {dtype}", flush=True)
    B.ra_reduce_scatter_ex(t, algo="ring_pipelined", slice_elems=slice_elems)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r in range(p):
        want = oracle.rs_partial(xs, dtype, r)
        assert same_bits(got[r], want, dtype), f"rank {r} at {first_diff(got[r], want, dtype)}"


def test_pipelined_flags_counters_numbered_past_two_to_the_31():
    """Ready counters compared against targets above 2^31: a fresh (zeroed)
    counter buffer must still read as 'not ready'.  The test hook reallocates
    the counters and numbers the call from 2^31; later calls continue from
    there, one of them on a larger buffer (the counters grow again)."""
    require_gpu()
    stream = torch.cuda.current_stream()
    for k, (p, n, flags) in enumerate([(8, 300_007, B.RA_FLAG_RENEW_COUNTERS), (8, 300_007, 0),
                                       (9, 2_000_003, 0), (4, 50_001, B.RA_FLAG_RENEW_COUNTERS)]):
        xs = inputs.make_inputs(p, n, "bfloat16", seed=40 + k, sigma=1.0)
        t = to_dev(xs, "bfloat16")
        print(f"[case] flag counters call {k} p={p} n={n} flags={flags}", flush=True)
        B.ra_allreduce_ex(t, algo="ring_pipelined_flags", flags=flags, slice_elems=2048,
                          stream=stream)
        B.ra_stream_status(stream=stream)
        want = oracle.ring_fold(xs, "bfloat16")
        for r, g in enumerate(from_dev(t, "bfloat16")):
            assert same_bits(g, want, "bfloat16"), f"call {k} rank {r} at {first_diff(g, want, 'bfloat16')}"


@pytest.mark.parametrize("algo", ["ring_step", "ring_bidir", "tree"])
@pytest.mark.parametrize("grid", [1, 3, 37])
def test_step_kernels_any_grid(algo, grid):
    require_gpu()
    p, n = 8, 50_001
    xs = inputs.make_inputs(p, n, "bfloat16", seed=grid, sigma=1.0)
    check(xs, "bfloat16", algo, grid=grid)


# Persistent grids take a large step's tiles (8 or more per workgroup) in order
# from tile counters, one contiguous range per group of workgroups (one group per
# XCD a channel runs on), and smaller steps in a fixed stride.  These shapes reach
# the counters with 1, 2, 4 and 8 groups per channel, groups of unequal size
# (grids that the group count does not divide), steps exactly at the threshold
# (8 and 16 channels), and launches that mix both kinds of step (the tree's
# levels hold 4, 2 and 1 pairs; the hierarchy's in-node and cross-node steps
# differ in width).  A second, smaller call on the same stream starts from
# freshly zeroed counters.
HANDOUT = [("ring_step", {"grid": 40}), ("ring_step", {"grid": 44}), ("ring_step", {"grid": 6}),
           ("ring_channels", {"channels": 2, "grid": 40}),
           ("ring_channels", {"channels": 3, "grid": 45}),
           ("ring_channels", {"channels": 5, "grid": 40}),
           ("ring_channels", {"channels": 8, "grid": 64}),
           ("ring_channels", {"channels": 16, "grid": 64}),
           ("tree", {"grid": 100}), ("ring_bidir", {"grid": 24}), ("hier", {"group": 4, "grid": 56})]


@pytest.mark.parametrize("algo,opts", HANDOUT)
def test_persistent_tile_handout(algo, opts):
    require_gpu()
    for k, (p, n, dtype) in enumerate([(8, 4_000_003, "bfloat16"), (8, 1_000_037, "int32")]):
        xs = inputs.make_inputs(p, n, dtype, seed=HANDOUT.index((algo, opts)) + 50 * k, sigma=1.0)
        print(f"[case] tile hand-out call {k} algo={algo} {opts} p={p} n={n} {dtype}", flush=True)
        got = run(xs, dtype, algo, **opts)
        if algo == "hier":
            want = oracle.hier_fold(xs, dtype, opts["group"])
        elif algo == "ring_channels":
            want = oracle.ring_fold(xs, dtype)
        else:
            want = expected(xs, dtype, algo)
        for r, g in enumerate(got):
            assert same_bits(g, want, dtype), f"call {k} rank {r} at {first_diff(g, want, dtype)}"


# Persistent grids the library sizes itself take 512-thread workgroups from 4 MiB per
# rank and 1024-thread ones from 16 MiB (up to 256 MiB, 64 MiB above 16 ranks); ragged
# sizes, every mode that reaches such a grid without a caller-set grid.
SHAPES = [("ring_channels", {"channels": 0}, 8, 2_500_003, "float32"),
          ("ring_channels", {"channels": 3}, 5, 3_000_001, "bfloat16"),
          ("ring_step", {"step_ts": True}, 9, 1_500_007, "int32"),
          ("ring_channels", {"channels": 0}, 8, 5_000_011, "float32"),
          ("ring_channels", {"channels": 8}, 4, 10_000_019, "bfloat16"),
          ("ring_channels", {"channels": 0, "flags": B.RA_FLAG_STRESS}, 8, 4_200_017, "int32"),
          ("ring_step", {"step_ts": True}, 17, 4_500_001, "float32"),
          ("ring_bidir", {"step_ts": True}, 8, 4_400_009, "float32"),
          ("tree", {"step_ts": True}, 6, 4_300_013, "float32"),
          ("hier", {"group": 4, "step_ts": True}, 8, 4_100_003, "bfloat16")]


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_persistent_workgroup_shapes(case):
    require_gpu()
    algo, opts, p, n, dtype = SHAPES[case]
    opts = dict(opts)
    if opts.pop("step_ts", False):
        opts["step_ts"] = torch.zeros(512, dtype=torch.int64, device="cuda")
    xs = inputs.make_inputs(p, n, dtype, seed=70 + case, sigma=1.0)
    got = run(xs, dtype, algo, **opts)
    if algo == "hier":
        want = oracle.hier_fold(xs, dtype, opts["group"])
    elif algo == "ring_channels":
        want = oracle.ring_fold(xs, dtype)
    else:
        want = expected(xs, dtype, algo)
    for r, g in enumerate(got):
        assert same_bits(g, want, dtype), f"rank {r} at {first_diff(g, want, dtype)}"


def test_noop_cases():
    require_gpu()
    x = [torch.arange(10, dtype=torch.float32, device="cuda")]
    B.ra_allreduce(x)
    assert x[0].tolist() == list(range(10))
    e = [torch.empty(0, device="cuda") for _ in range(4)]
    for algo in ALL:
        B.ra_allreduce_ex(e, algo=algo)
    B.ra_stream_status()


# ------------------------------------------------------------ reduce-scatter / all-gather

@pytest.mark.parametrize("algo", ["ring_step", "ring_pipelined", "ring_pipelined_flags"])
@pytest.mark.parametrize("p,n,dtype", [(4, 4, "float32"), (9, 1_003, "int32"),
                                       (9, 100_003, "bfloat16"), (16, 70_001, "float32")])
def test_reduce_scatter_states_then_all_gather(algo, p, n, dtype):
    require_gpu()
    xs = inputs.make_inputs(p, n, dtype, seed=p + n, sigma=1.0)
    t = to_dev(xs, dtype)
    print(f"[case] RS/AG algo={algo} p={p} n={n} dtype={dtype}", flush=True)
    B.ra_reduce_scatter_ex(t, algo=algo)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r in range(p):
        # every chunk of every rank: the ring's partial sums after p-1 steps
        want = oracle.rs_partial(xs, dtype, r)
        assert same_bits(got[r], want, dtype), f"rank {r} at {first_diff(got[r], want, dtype)}"
    B.ra_all_gather_ex(t, algo=algo)
    B.ra_stream_status()
    final = from_dev(t, dtype)
    want = oracle.ring_fold(xs, dtype)
    assert all(same_bits(f, want, dtype) for f in final)


def test_default_entry_points():
    require_gpu()
    p, n = 5, 12_345
    xs = inputs.make_inputs(p, n, "float32", seed=3)
    t = to_dev(xs, "float32")
    B.ra_reduce_scatter(t)
    B.ra_all_gather(t)
    B.ra_stream_status()
    want = oracle.ring_fold(xs, "float32")
    assert all(same_bits(f, want, "float32") for f in from_dev(t, "float32"))
    t = to_dev(xs, "float32")
    B.ra_allreduce(t)
    B.ra_stream_status()
    assert all(same_bits(f, want, "float32") for f in from_dev(t, "float32"))


# ------------------------------------------------------------ failure handling

@pytest.mark.parametrize("algo", ["ring_step", "ring_pipelined_flags", "tree"])
def test_forced_timeout_is_reported_and_cleared(algo):
    # the host asks the first device wait to expect an arrival that never comes;
    # with a 2 ms budget every workgroup gives up and exits, and the error shows
    # up on the stream instead of a hang
    require_gpu()
    p, n = 4, 4096
    xs = inputs.make_inputs(p, n, "float32", seed=1)
    t = to_dev(xs, "float32")
    print(f"[case] forced timeout algo={algo}", flush=True)
    B.ra_allreduce_ex(t, algo=algo, timeout_us=2000, flags=B.RA_FLAG_FORCE_TIMEOUT)
    with pytest.raises(B.RaError) as e:
        B.ra_stream_status()
    assert e.value.code == B.RA_ERR_TIMEOUT
    # cleared: the next call on the stream works
    t = to_dev(xs, "float32")
    B.ra_allreduce_ex(t, algo=algo)
    B.ra_stream_status()
    want = expected(xs, "float32", algo)
    assert all(same_bits(f, want, "float32") for f in from_dev(t, "float32"))


def test_step_timestamps():
    require_gpu()
    p, n = 8, 1 << 20
    t = to_dev(inputs.make_inputs(p, n, "float32", seed=2), "float32")
    ts = torch.zeros(2 * (p - 1) + 1, dtype=torch.int64, device="cuda")
    B.ra_allreduce_ex(t, algo="ring_step", step_ts=ts)
    B.ra_stream_status()
    v = ts.cpu().numpy()
    assert np.all(v > 0) and np.all(np.diff(v) >= 0)
    assert B.ra_wallclock_hz() > 0


def test_binding_rejects_mismatched_tensors():
    require_gpu()
    a = torch.zeros(16, device="cuda")
    with pytest.raises(ValueError):
        B.ra_allreduce([a, torch.zeros(17, device="cuda")])
    with pytest.raises(ValueError):
        B.ra_allreduce([a, torch.zeros(16, device="cuda", dtype=torch.int32)])
    with pytest.raises(TypeError):
        B.ra_allreduce([torch.zeros(16, device="cuda", dtype=torch.uint8) for _ in range(2)])
    with pytest.raises(B.RaError) as e:
        B.ra_allreduce([a, a])
    assert e.value.code == B.RA_ERR_ALIAS


def test_rank_buffers_match_lists_on_every_entry_point():
    """A RankBuffers (checked and marshalled once) gives the same bits as the list
    it was made from, through every entry point, and is reused across calls."""
    require_gpu()
    p, n = 9, 10_007
    xs = inputs.make_inputs(p, n, "float32", seed=11)
    want = oracle.ring_fold(xs, "float32")
    t = to_dev(xs, "float32")
    ranks = B.RankBuffers(t)
    assert len(ranks) == p and ranks.n == n
    for call in (lambda: B.ra_allreduce(ranks), lambda: B.ra_allreduce_ex(ranks, algo="ring_step")):
        for r in range(p):
            t[r].copy_(torch.from_numpy(xs[r]))
        call()
        B.ra_stream_status()
        got = from_dev(t, "float32")
        for r in range(p):
            assert same_bits(got[r], want, "float32"), r
    # reduce-scatter then all-gather through the same object
    for r in range(p):
        t[r].copy_(torch.from_numpy(xs[r]))
    B.ra_reduce_scatter(ranks)
    B.ra_all_gather(ranks)
    B.ra_reduce_scatter_ex(ranks, algo="fused")
    B.ra_all_gather_ex(ranks, algo="fused")
    B.ra_stream_status()
    # the second round re-reduces the already-reduced buffers: compare with the oracle's
    # two rounds
    want2 = oracle.ring_fold([want] * p, "float32")
    got = from_dev(t, "float32")
    for r in range(p):
        assert same_bits(got[r], want2, "float32"), r


def test_rank_buffers_rejects_bad_inputs_and_resized_tensors():
    require_gpu()
    a = torch.zeros(16, device="cuda")
    with pytest.raises(ValueError):
        B.RankBuffers([a, torch.zeros(17, device="cuda")])
    with pytest.raises(ValueError):
        B.RankBuffers([a, torch.zeros(32, device="cuda")[::2]])
    b = torch.zeros(16, device="cuda")
    ranks = B.RankBuffers([b, torch.zeros(16, device="cuda")])
    b.resize_(1 << 20)   # the first rank now lives elsewhere
    with pytest.raises(ValueError):
        B.ra_allreduce(ranks)
    with pytest.raises(B.RaError) as e:
        B.ra_allreduce(B.RankBuffers([a, a]))
    assert e.value.code == B.RA_ERR_ALIAS


def test_stream_copy():
    require_gpu()
    src = torch.randn(1 << 20, device="cuda")
    dst = torch.zeros_like(src)
    B.ra_stream_copy(dst, src)
    torch.cuda.synchronize()
    assert torch.equal(dst, src)


@pytest.mark.parametrize("nbytes,grid", [(16, 1), (16 << 10, 3), ((16 << 10) + 48, 7),
                                         ((1 << 24) + 4096 + 16, 0), (1 << 26, 1000),
                                         ((1 << 22) + 80, 9), ((5 << 20) + 16, 13)])
def test_stream_copy_resident(nbytes, grid):
    # whole 16 KiB tiles handed out per XCD group (grids that 8 does not divide
    # give the groups unequal shares), the vectors past them one per thread; a
    # second, smaller call on the same stream starts from freshly zeroed counters
    require_gpu()
    for k, nb in enumerate((nbytes, max(16, nbytes // 2 // 16 * 16))):
        src = torch.randint(-2**31, 2**31 - 1, (nb // 4,), dtype=torch.int32, device="cuda")
        dst = torch.zeros(nb // 4 + 64, dtype=torch.int32, device="cuda")
        print(f"[case] resident copy call {k} bytes={nb} grid={grid}", flush=True)
        B.ra_stream_copy_resident(dst, src, grid=grid)
        torch.cuda.synchronize()
        assert torch.equal(dst[: nb // 4], src)
        assert not dst[nb // 4:].any()
