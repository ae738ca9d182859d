"""GPU parity on seeded random cases (through the C ABI).

A fixed list of 1000 pseudo-random configurations spans the choices the library
makes per call, so that every code path meets odd combinations:

* p from 2 to 64, n from 0 to about 60 000 (below, at and above the size where
  the step algorithms switch from one workgroup to one launch per step, and
  chunk edges at every alignment);
* all six element types and the three reductions (average on floats only);
* every all-reduce algorithm, with grids, channel counts, hierarchy group sizes
  and slice lengths drawn at random where they apply;
* reduce-scatter followed by all-gather with independently drawn algorithms.

A second list of 60 cases draws n from 100 000 to 3 000 000 elements, where
the launch shapes that only large buffers get (two vectors per thread for copy
steps, eight or more pipelined slices per chunk, whole-buffer tree launches)
come into play.

Each result must equal the oracle's result for that algorithm's order bit for
bit.  The lists are generated from fixed seeds, so a failure names a
reproducible case.
"""

import random

import pytest

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

DTYPES = ["int32", "int64", "float16", "bfloat16", "float32", "float64"]
FLOATS = {"float16", "bfloat16", "float32", "float64"}
ALL_REDUCE = ["fused", "ring_step", "ring_pipelined", "ring_channels", "ring_bidir", "tree",
              "hier", "hier_fused", "auto"]
PHASE = ["fused", "ring_step", "ring_pipelined", "ring_channels"]
RING_ORDER = {"fused", "ring_step", "ring_pipelined", "ring_pipelined_flags", "ring_channels",
              "auto"}


def _divisors(p):
    return [g for g in range(1, p + 1) if p % g == 0]


def _cases(count=1000, seed=20261202):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        p = rng.choice([2, 3, 4, 5, 7, 8, 9, 12, 16, 31, 32, 64])
        n = rng.choice([0, 1, p - 1, p, p + 1, rng.randrange(2, 300), rng.randrange(300, 4000),
                        rng.randrange(4000, 60_000)])
        dtype = rng.choice(DTYPES)
        op = rng.choice(["sum", "max", "avg"] if dtype in FLOATS else ["sum", "max"])
        kind = rng.random()
        if kind < 0.8:
            algo = rng.choice(ALL_REDUCE)
            opts = {}
            if algo in ("ring_step", "ring_bidir", "tree", "hier") and rng.random() < 0.3:
                opts["grid"] = rng.choice([1, 2, 7, 16, 64])
            if algo == "ring_channels":
                opts["channels"] = rng.choice([0, 1, 2, 3, 8, 16])
                if rng.random() < 0.3:
                    opts["grid"] = rng.choice([8, 24, 64])
            if algo == "ring_pipelined" and rng.random() < 0.5:
                opts["slice_elems"] = rng.choice([8, 64, 1000, 4096])
            if algo == "ring_pipelined" and i % 2 == 0:
                algo = "ring_pipelined_flags"   # both pipelined forms, same draws
            if algo in ("hier", "hier_fused"):
                opts["group"] = rng.choice(_divisors(p))
            out.append(("allreduce", i, p, n, dtype, op, algo, None, opts))
        else:
            rs, ag = rng.choice(PHASE), rng.choice(PHASE)
            if i % 2 == 0:
                rs, ag = (a + "_flags" if a == "ring_pipelined" else a for a in (rs, ag))
            out.append(("rs_ag", i, p, n, dtype, op, rs, ag, {}))
    return out


def _want(xs, dtype, op, algo, opts):
    if algo in RING_ORDER:
        return oracle.ring_fold(xs, dtype, op=op)
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype, op=op)[0][0]
    if algo == "tree":
        return oracle.tree_allreduce(xs, dtype, op=op)[0][0]
    return oracle.hier_fold(xs, dtype, opts["group"], op=op)


@pytest.mark.parametrize("case", _cases(), ids=lambda c: f"case{c[1]}")
def test_random_case(case):
    require_gpu()
    call, i, p, n, dtype, op, algo, algo2, opts = case
    if dtype == "int64":
        xs = inputs.make_inputs(p, n, dtype, seed=i, lo=-2**62, hi=2**62)
    else:
        xs = inputs.make_inputs(p, n, dtype, seed=i, sigma=2.0)
    t = to_dev(xs, dtype)
    print(f"[case] {case}", flush=True)
    if call == "allreduce":
        B.ra_allreduce_ex(t, algo=algo, op=op, **opts)
        want = _want(xs, dtype, op, algo, opts)
    else:
        B.ra_reduce_scatter_ex(t, algo=algo, op=op)
        B.ra_all_gather_ex(t, algo=algo2)
        want = oracle.ring_fold(xs, dtype, op=op)
    B.ra_stream_status()
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want, dtype), f"rank {r} first diff {first_diff(g, want, dtype)}"


# Larger buffers (up to a few million elements), where copy steps take two
# vectors per thread, pipelined chunks are cut into eight or more slices with
# workers in multiples of 8, and whole-buffer tree steps run as large launches.
def _large_cases(count=60, seed=20261203):
    rng = random.Random(seed)
    out = []
    for i in range(count):
        p = rng.choice([2, 3, 4, 8, 9, 16])
        n = rng.randrange(100_000, 3_000_000)
        dtype = rng.choice(DTYPES)
        op = rng.choice(["sum", "max", "avg"] if dtype in FLOATS else ["sum", "max"])
        algo = rng.choice(["ring_step", "ring_pipelined", "ring_bidir", "tree", "hier", "auto"])
        opts = {}
        if algo == "ring_pipelined" and rng.random() < 0.5:
            opts["slice_elems"] = rng.choice([1024, 4096, 65536])
        if algo == "ring_pipelined" and rng.random() < 0.3:
            opts["grid"] = rng.choice([64, 200, 512])
        if algo == "ring_pipelined" and ("grid" in opts or i % 2 == 0):
            algo = "ring_pipelined_flags"       # grids are the flag ring's option
        if algo == "hier":
            opts["group"] = rng.choice(_divisors(p))
        out.append(("allreduce", 1000 + i, p, n, dtype, op, algo, None, opts))
    return out


@pytest.mark.parametrize("case", _large_cases(), ids=lambda c: f"large{c[1]}")
def test_random_large_case(case):
    test_random_case(case)
