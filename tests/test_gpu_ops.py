"""GPU parity of every element type and reduction (through the C ABI).

Element types int32, int64, float16, bfloat16, float32, float64; reductions sum,
max and avg (pre-divided, floats only); the fused pass also with wide
accumulation.  Every algorithm must match the oracle's result for its own order
bit for bit: ring order for fused, ring_step, both pipelined rings and ring_channels,
the bidirectional rings' halves for ring_bidir, the binomial tree for tree.
"""

import numpy as np
import pytest
import torch

import oracle
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

DTYPES = ["int32", "int64", "float16", "bfloat16", "float32", "float64"]
FLOATS = ["float16", "bfloat16", "float32", "float64"]
ALGOS = ["fused", "ring_step", "ring_pipelined", "ring_pipelined_flags", "ring_channels",
         "ring_bidir", "tree"]
RING = ["fused", "ring_step", "ring_pipelined", "ring_pipelined_flags", "ring_channels"]


def expected(xs, dtype, algo, op, wide=False):
    if algo in RING:
        return oracle.ring_fold(xs, dtype, op=op, wide=wide)
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype, op=op)[0][0]
    return oracle.tree_allreduce(xs, dtype, op=op)[0][0]


def make(p, n, dtype, seed):
    if dtype == "int64":
        return inputs.make_inputs(p, n, dtype, seed, lo=-2**62, hi=2**62)
    return inputs.make_inputs(p, n, dtype, seed, sigma=3.0)


def check_all_reduce(xs, dtype, algo, op, wide=False):
    t = to_dev(xs, dtype)
    print(f"[case] algo={algo} op={op} wide={wide} p={len(xs)} n={len(xs[0])} dtype={dtype}",
          flush=True)
    B.ra_allreduce_ex(t, algo=algo, op=op, wide=wide)
    B.ra_stream_status()
    want = expected(xs, dtype, algo, op, wide)
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want, dtype), f"rank {r} first diff {first_diff(g, want, dtype)}"


# avg is defined for floating-point types only (the library refuses it on
# integers, a CPU test checks that)
DTYPE_OPS = [(d, o) for d in DTYPES for o in ("sum", "max", "avg") if o != "avg" or d in FLOATS]


@pytest.mark.parametrize("dtype,op", DTYPE_OPS)
@pytest.mark.parametrize("p,n", [(2, 7), (5, 1023), (9, 70_001), (64, 4097)])
def test_every_algorithm(dtype, op, p, n):
    require_gpu()
    xs = make(p, n, dtype, seed=p * 131 + n)
    for algo in ALGOS:
        check_all_reduce(xs, dtype, algo, op)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
@pytest.mark.parametrize("op", ["sum", "avg", "max"])
@pytest.mark.parametrize("p,n", [(3, 17), (8, 100_003), (64, 4097)])
def test_wide_accumulation(dtype, op, p, n):
    require_gpu()
    xs = make(p, n, dtype, seed=p + n)
    check_all_reduce(xs, dtype, "fused", op, wide=True)


@pytest.mark.parametrize("dtype", ["float16", "bfloat16", "float32"])
@pytest.mark.parametrize("op", ["sum", "avg"])
def test_wide_reduce_scatter(dtype, op):
    require_gpu()
    p, n = 9, 10_007
    xs = make(p, n, dtype, seed=41)
    t = to_dev(xs, dtype)
    print(f"[case] wide fused RS op={op} dtype={dtype}", flush=True)
    B.ra_reduce_scatter_ex(t, algo="fused", op=op, wide=True)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r in range(p):
        want = oracle.rs_owned(xs, dtype, r, op=op, wide=True)
        assert same_bits(got[r], want, dtype), f"rank {r} at {first_diff(got[r], want, dtype)}"


@pytest.mark.parametrize("algo", ["ring_step", "ring_pipelined", "ring_pipelined_flags",
                                  "ring_channels", "fused"])
@pytest.mark.parametrize("op", ["max", "avg"])
@pytest.mark.parametrize("dtype", ["float16", "float64"])
def test_reduce_scatter_states_with_ops(algo, op, dtype):
    # step-by-step reduce-scatters leave the partial folds of the (divided)
    # terms; the fused one leaves non-owned chunks untouched
    require_gpu()
    p, n = 7, 20_011
    xs = make(p, n, dtype, seed=43)
    t = to_dev(xs, dtype)
    print(f"[case] RS states algo={algo} op={op} dtype={dtype}", flush=True)
    B.ra_reduce_scatter_ex(t, algo=algo, op=op)
    B.ra_stream_status()
    got = from_dev(t, dtype)
    for r in range(p):
        want = (oracle.rs_owned(xs, dtype, r, op=op) if algo == "fused"
                else oracle.rs_partial(xs, dtype, r, op=op))
        assert same_bits(got[r], want, dtype), f"rank {r} at {first_diff(got[r], want, dtype)}"
    B.ra_all_gather_ex(t, algo=algo)
    B.ra_stream_status()
    want = oracle.ring_fold(xs, dtype, op=op)
    assert all(same_bits(g, want, dtype) for g in from_dev(t, dtype))


def test_float16_overflow_and_its_remedies():
    # 8 ranks of 8192: the fp16 sum overflows (65536 > 65504); pre-divided
    # averages stay exact (1024 each, 8192 in total)
    require_gpu()
    p, n = 8, 4096
    xs = [np.full(n, 8192.0, np.float16) for _ in range(p)]
    for algo in ALGOS:
        t = to_dev(xs, "float16")
        print(f"[case] fp16 overflow algo={algo}", flush=True)
        B.ra_allreduce_ex(t, algo=algo, op="sum")
        B.ra_stream_status()
        assert all(np.all(np.isinf(g)) for g in from_dev(t, "float16"))
        t = to_dev(xs, "float16")
        B.ra_allreduce_ex(t, algo=algo, op="avg")
        B.ra_stream_status()
        assert all(np.all(g == 8192.0) for g in from_dev(t, "float16"))


def test_int64_wraps():
    require_gpu()
    p, n = 4, 1001
    big = np.iinfo(np.int64).max
    xs = [np.full(n, big, np.int64) for _ in range(p)]
    want = np.full(n, np.int64(-4), np.int64)      # 4 * (2^63 - 1) mod 2^64 = 2^64 - 4
    for algo in ALGOS:
        t = to_dev(xs, "int64")
        B.ra_allreduce_ex(t, algo=algo)
        B.ra_stream_status()
        assert all(np.array_equal(g, want) for g in from_dev(t, "int64"))


def test_binding_accepts_new_dtypes():
    require_gpu()
    for dt in (torch.float16, torch.float64, torch.int64):
        x = [torch.ones(33, dtype=dt, device="cuda") for _ in range(3)]
        B.ra_allreduce(x)
        B.ra_stream_status()
        assert all(torch.equal(v, torch.full_like(v, 3)) for v in x)


def special_values(p, n, dtype, seed):
    """Normals mixed with +-0, +-inf and NaNs of both signs and several payloads."""
    rng = np.random.default_rng(seed)
    xs = make(p, n, dtype, seed)
    bits_t = {"float16": np.uint16, "bfloat16": np.uint16, "float32": np.uint32,
              "float64": np.uint64}[dtype]
    width = 8 * np.dtype(bits_t).itemsize
    exp_mask = {"float16": 0x7C00, "bfloat16": 0x7F80, "float32": 0x7F800000,
                "float64": 0x7FF0000000000000}[dtype]
    sign = 1 << (width - 1)
    pool = [0, sign, exp_mask, exp_mask | sign, exp_mask | 1, exp_mask | 1 | sign,
            exp_mask | (exp_mask >> 1 & ~exp_mask), (1 << (width - 1)) - 1]
    out = []
    for x in xs:
        b = np.array(x, copy=True).view(bits_t)
        idx = rng.random(n) < 0.2
        b[idx] = np.array(pool, dtype=np.uint64).astype(bits_t)[rng.integers(0, len(pool), idx.sum())]
        out.append(b.view(x.dtype))
    return out


@pytest.mark.parametrize("dtype", FLOATS)
def test_max_with_nan_signed_zero_and_infinity(dtype):
    # every algorithm's maximum equals the oracle's bit for bit on inputs full of
    # +-0, +-inf and NaNs (any NaN gives the canonical quiet NaN; +0 > -0)
    require_gpu()
    p, n = 9, 20_011
    xs = special_values(p, n, dtype, seed=5)
    for algo in ALGOS + ["hier", "hier_fused"]:
        t = to_dev(xs, dtype)
        print(f"[case] max specials algo={algo} dtype={dtype}", flush=True)
        B.ra_allreduce_ex(t, algo=algo, op="max", group=3)
        B.ra_stream_status()
        want = oracle.ring_fold(xs, dtype, op="max")
        for r, g in enumerate(from_dev(t, dtype)):
            assert same_bits(g, want, dtype), f"{algo} rank {r} first diff {first_diff(g, want, dtype)}"
