"""GPU parity on constructed edge cases (through the C ABI), every algorithm.

* subnormal inputs and sums (float32, bfloat16, float16, float64): values that
  are small multiples of the smallest subnormal, and odd multiples that round
  once they are normal -- a kernel that flushed subnormals to zero, or rounded
  them differently, would differ from the oracle;
* round-half-even ties on every element (bfloat16 through the float32 add and
  the packed narrowing convert, float16 through the half add): two ranks hold
  A and B whose sum lies exactly halfway between two neighbours, every other
  rank holds +0, so every algorithm's one inexact hop is that tie, and half of
  the ties round down to even, half up;
* int32 sums that wrap past 2**31 both ways;
* chunk edges: sizes where most chunks start and end inside a 16-byte vector,
  up to p = 64, so the one-pass, two-level and slice-carrying kernels fold edge
  elements in every edge wave of several edge workgroups, in each of their
  modes (all-reduce, reduce-scatter, all-gather) and reductions;
* short last tiles: sizes at which those launches number each chunk's short
  last tile after the others, with and without edge workgroups, and sizes just
  outside that rule;
* p = 2 with 35 * 2**30 bfloat16 elements per rank (70 GiB, 140 GiB in all):
  more tiles than one dispatch can hold, so the one-pass, pipelined and step
  kernels take their grid-stride loops; checked on windows against the oracle.

Expected values are the oracle's (each algorithm against its own order).
"""

import numpy as np
import pytest
import torch

import oracle
from oracle.arith import f32_to_bf16_bits
from ring_all_reduce_schedule_amd import binding as B
from ring_all_reduce_schedule_amd import inputs
from tests.gpu_util import require_gpu, to_dev, from_dev, same_bits, first_diff

pytestmark = pytest.mark.gpu

ALGOS = ["fused", "ring_step", "ring_pipelined", "ring_pipelined_flags", "ring_channels",
         "ring_bidir", "tree", "hier", "hier_fused"]
def _group(p):
    """Ranks per node for the hierarchical algorithms: 2, or 3 when 2 does not divide p."""
    return 2 if p % 2 == 0 else 3


def _want(xs, dtype, algo):
    if algo == "tree":
        return oracle.tree_allreduce(xs, dtype)[0][0]
    if algo == "ring_bidir":
        return oracle.bidir_allreduce(xs, dtype)[0][0]
    if algo in ("hier", "hier_fused"):
        return oracle.hier_fold(xs, dtype, _group(len(xs)))
    return oracle.ring_fold(xs, dtype)


def _check(xs, dtype, algo, tag):
    t = to_dev(xs, dtype)
    opts = {"group": _group(len(xs))} if algo.startswith("hier") else {}
    print(f"[case] {tag} algo={algo} p={len(xs)} n={len(xs[0])} {dtype}", flush=True)
    B.ra_allreduce_ex(t, algo=algo, **opts)
    B.ra_stream_status()
    want = _want(xs, dtype, algo)
    for r, g in enumerate(from_dev(t, dtype)):
        assert same_bits(g, want, dtype), f"{tag} rank {r} first diff {first_diff(g, want, dtype)}"
    return want


# (precision in bits including the leading one, smallest normal exponent)
FORMATS = {"float32": (24, -126), "bfloat16": (8, -126), "float16": (11, -14),
           "float64": (53, -1022)}


def _subnormal_inputs(p, n, dtype, seed):
    prec, emin = FORMATS[dtype]
    tiny = 2.0 ** (emin - prec + 1)
    rng = np.random.default_rng(seed)
    xs = []
    for r in range(p):
        k = rng.integers(-2 ** (prec - 1), 2 ** (prec - 1), n)
        odd = (2 * rng.integers(-2 ** (prec - 2), 2 ** (prec - 2), n) + 1) * rng.integers(1, 5, n)
        v = np.where(rng.random(n) < 0.5, k * tiny, odd * tiny)
        if dtype == "bfloat16":
            xs.append(f32_to_bf16_bits(v.astype(np.float32)))
        else:
            xs.append(v.astype({"float32": np.float32, "float16": np.float16,
                                "float64": np.float64}[dtype]))
    return xs


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["float32", "bfloat16", "float16", "float64"])
def test_subnormal_inputs_and_sums(algo, dtype):
    require_gpu()
    p, n = 8, 10_007
    xs = _subnormal_inputs(p, n, dtype, seed=10 * ALGOS.index(algo) + list(FORMATS).index(dtype))
    want = _check(xs, dtype, algo, "subnormal")
    prec, emin = FORMATS[dtype]
    v = np.abs(oracle.as_values(want, dtype))
    # the case is what it claims: many results are subnormal and nonzero
    assert np.count_nonzero((v > 0) & (v < 2.0 ** emin)) > n // 10


def _tie_inputs(p, n, dtype, seed):
    """Ranks a and b hold A and B with A + B exactly halfway between two
    neighbours of the element type; every other rank holds +0."""
    rng = np.random.default_rng(seed)
    prec = FORMATS[dtype][0]
    # A: a value with `prec` significant bits, exponent e; B: half an ulp of A
    e = rng.integers(-8, 8, n)
    mant = rng.integers(2 ** (prec - 1), 2 ** prec, n)          # includes odd and even
    sign = np.where(rng.random(n) < 0.5, -1.0, 1.0)
    A = sign * mant * 2.0 ** (e - (prec - 1))
    B = sign * 2.0 ** (e - prec)                                  # half an ulp, same sign
    a, b = rng.choice(p, 2, replace=False)
    xs = []
    for r in range(p):
        v = A if r == a else B if r == b else np.zeros(n)
        if dtype == "bfloat16":
            xs.append(f32_to_bf16_bits(v.astype(np.float32)))
        else:
            xs.append(v.astype(np.float16))
    return xs, mant


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["bfloat16", "float16"])
@pytest.mark.parametrize("p", [2, 8])
def test_round_half_even_ties(algo, dtype, p):
    require_gpu()
    n = 20_011
    xs, mant = _tie_inputs(p, n, dtype, seed=p * 31 + len(algo))
    want = _check(xs, dtype, algo, "ties")
    # every element was a tie: even significands stay, odd ones move up by one ulp
    got = np.abs(oracle.as_values(want, dtype))
    a_abs = np.abs(np.maximum.reduce([np.abs(oracle.as_values(x, dtype)) for x in xs]))
    ulp = a_abs / mant                                            # 2**(e-(prec-1))
    expect = np.where(mant % 2 == 0, a_abs, a_abs + ulp)
    assert np.array_equal(got, expect)
    assert 0.3 < np.mean(mant % 2) < 0.7


@pytest.mark.parametrize("algo", ALGOS)
def test_int32_wraps(algo):
    require_gpu()
    p, n = 9, 30_011
    rng = np.random.default_rng(17)
    xs = [rng.integers(2 ** 30, 2 ** 31 - 1, n, dtype=np.int64).astype(np.int32) *
          np.where(rng.random(n) < 0.7, 1, -1).astype(np.int32) for _ in range(p)]
    want = _check(xs, "int32", algo, "int32 wrap")
    exact = np.sum(np.stack(xs).astype(np.int64), axis=0)
    assert np.array_equal(want.astype(np.int64), (exact + 2 ** 31) % 2 ** 32 - 2 ** 31)
    assert np.count_nonzero(np.abs(exact) >= 2 ** 31) > n // 4


# ------------------------------------------------------------ chunk edges

VEC = {"int32": 4, "float32": 4, "bfloat16": 8, "float16": 8, "float64": 2, "int64": 2}
EDGE_CASES = [(2, 37, "bfloat16", "sum"), (5, 1_003, "int64", "sum"),
              (13, 20_011, "float16", "avg"), (33, 10_007, "float64", "avg"),
              (63, 65_537, "bfloat16", "sum"), (64, 4_133, "float32", "max"),
              (64, 524_365, "bfloat16", "sum")]


def _edge_chunks(n, p, dtype):
    v = VEC[dtype]
    return sum(1 for lo, hi in oracle.chunk_bounds(n, p) if hi > lo and (lo % v or hi % v))


@pytest.mark.parametrize("p,n,dtype,op", EDGE_CASES)
def test_chunk_edges_every_mode(p, n, dtype, op):
    require_gpu()
    # the case is what it claims: most chunks have edge elements
    assert _edge_chunks(n, p, dtype) >= p // 2
    xs = inputs.make_inputs(p, n, dtype, seed=p * 7 + n, sigma=1.0)
    g = next(d for d in range(2, p + 1) if p % d == 0)      # ranks per node
    ring = oracle.ring_fold(xs, dtype, op=op)
    for algo, want in (("fused", ring), ("ring_pipelined", ring),
                       ("hier_fused", oracle.hier_fold(xs, dtype, g, op=op))):
        t = to_dev(xs, dtype)
        print(f"[case] edges AR algo={algo} p={p} n={n} {dtype} {op}", flush=True)
        B.ra_allreduce_ex(t, algo=algo, op=op, **({"group": g} if algo == "hier_fused" else {}))
        B.ra_stream_status()
        for r, got in enumerate(from_dev(t, dtype)):
            assert same_bits(got, want, dtype), f"{algo} rank {r} at {first_diff(got, want, dtype)}"
    # reduce-scatter: the one-pass kernel writes owned chunks only, the
    # slice-carrying ring leaves the step-by-step partials (checked where the
    # oracle's closed form for every rank stays quick)
    for algo in ("fused", "ring_pipelined"):
        if algo == "ring_pipelined" and p * p * n > 50_000_000:
            continue
        t = to_dev(xs, dtype)
        print(f"[case] edges RS algo={algo} p={p} n={n} {dtype} {op}", flush=True)
        B.ra_reduce_scatter_ex(t, algo=algo, op=op)
        B.ra_stream_status()
        for r, got in enumerate(from_dev(t, dtype)):
            want = (oracle.rs_owned(xs, dtype, r, op=op) if algo == "fused"
                    else oracle.rs_partial(xs, dtype, r, op=op))
            assert same_bits(got, want, dtype), f"{algo} RS rank {r} at {first_diff(got, want, dtype)}"
    # all-gather on arbitrary buffers: only owned chunks may be read
    gathered, _ = oracle.all_gather(xs, dtype)
    for algo in ("fused", "ring_pipelined"):
        t = to_dev(xs, dtype)
        print(f"[case] edges AG algo={algo} p={p} n={n} {dtype}", flush=True)
        B.ra_all_gather_ex(t, algo=algo)
        B.ra_stream_status()
        for r, got in enumerate(from_dev(t, dtype)):
            assert same_bits(got, gathered[r], dtype), f"{algo} AG rank {r} at {first_diff(got, gathered[r], dtype)}"


# Sizes at which the one-pass, two-level and slice-carrying launches number each
# chunk's short last tile after the others (at most 2048 tiles, last tiles at
# most half full), with and without edge workgroups between the whole and the
# short tiles, and one where the last tiles are fuller and the order is plain.
SHORT_TAIL_CASES = [(64, 528_384, "bfloat16"),      # 5 tiles per chunk, the last 8 vectors
                    (64, 524_365, "bfloat16"),      # the same with edge elements
                    (16, 2_097_215, "float32"),     # 129 tiles per chunk: more than 2048 in all
                    (64, 1_000_003, "bfloat16"),    # last tiles 62% full, edge elements
                    (5, 5 * 1029 * 4, "int32")]     # 5 tiles per chunk, the last a few vectors


@pytest.mark.parametrize("p,n,dtype", SHORT_TAIL_CASES)
def test_short_last_tiles_every_mode(p, n, dtype):
    require_gpu()
    xs = inputs.make_inputs(p, n, dtype, seed=p * 13 + n, sigma=1.0)
    g = next(d for d in range(2, p + 1) if p % d == 0)
    ring = oracle.ring_fold(xs, dtype)
    for algo, want in (("fused", ring), ("ring_pipelined", ring),
                       ("hier_fused", oracle.hier_fold(xs, dtype, g))):
        t = to_dev(xs, dtype)
        print(f"[case] short tail AR algo={algo} p={p} n={n} {dtype}", flush=True)
        B.ra_allreduce_ex(t, algo=algo, **({"group": g} if algo == "hier_fused" else {}))
        B.ra_stream_status()
        for r, got in enumerate(from_dev(t, dtype)):
            assert same_bits(got, want, dtype), f"{algo} rank {r} at {first_diff(got, want, dtype)}"
    t = to_dev(xs, dtype)
    print(f"[case] short tail RS fused p={p} n={n} {dtype}", flush=True)
    B.ra_reduce_scatter_ex(t, algo="fused")
    B.ra_stream_status()
    for r, got in enumerate(from_dev(t, dtype)):
        want = oracle.rs_owned(xs, dtype, r)
        assert same_bits(got, want, dtype), f"fused RS rank {r} at {first_diff(got, want, dtype)}"
    gathered, _ = oracle.all_gather(xs, dtype)
    for algo in ("fused", "ring_pipelined"):
        t = to_dev(xs, dtype)
        print(f"[case] short tail AG algo={algo} p={p} n={n} {dtype}", flush=True)
        B.ra_all_gather_ex(t, algo=algo)
        B.ra_stream_status()
        for r, got in enumerate(from_dev(t, dtype)):
            assert same_bits(got, gathered[r], dtype), f"{algo} AG rank {r}"


# ------------------------------------------------------------ beyond one dispatch

N_HUGE = 35 << 30          # bf16 elements per rank: 70 GiB, 2**24 + tiles of 4 KiB per chunk


def _huge_windows(n, p, seed):
    half = 1 << 15
    wins = [(0, 1 << 15), (n - (1 << 15), n)]
    for lo, _ in oracle.chunk_bounds(n, p)[1:]:
        wins.append((lo - half, lo + half))
    for x in (2 ** 31, 2 ** 32, 2 ** 33, 2 ** 34):
        wins.append((x - half, x + half))
    rng = np.random.default_rng(seed)
    for s in rng.integers(0, n - (1 << 18), 8):
        wins.append((int(s), int(s) + (1 << 18)))
    return sorted(set(wins))


@pytest.mark.parametrize("algo", ["fused", "ring_pipelined", "ring_step", "tree"])
def test_two_ranks_beyond_one_dispatch(algo):
    dev = require_gpu()
    p, n = 2, N_HUGE
    free, _ = torch.cuda.mem_get_info(dev)
    need = p * n * 2
    assert free > need + (4 << 30), f"needs {need / 2**30:.0f} GiB, {free / 2**30:.0f} free"
    # the one-pass kernel's tiles (4 KiB of every chunk each) exceed one dispatch's
    # 2**32 / 256 workgroups
    assert p * ((n // p) // (8 * 256)) > 0xFFFFFFFF // 256
    print(f"[case] p=2 n={n} bf16 algo={algo}: drawing inputs", flush=True)
    t = [torch.empty(n, dtype=torch.bfloat16, device=dev) for _ in range(p)]
    inputs.device_normal_bf16(t, 1e-3, 5)
    wins = _huge_windows(n, p, 5)
    before = [[x[a:b].view(torch.int16).cpu().numpy().view(np.uint16) for x in t] for a, b in wins]
    torch.cuda.synchronize()
    print(f"[case] p=2 n={n} bf16 algo={algo}: running", flush=True)
    B.ra_allreduce_ex(t, algo=algo)
    B.ra_stream_status()
    assert torch.equal(t[0].view(torch.int16), t[1].view(torch.int16)), "ranks differ"
    for (a, b), xw in zip(wins, before):
        if algo == "tree":
            want = oracle.tree_allreduce(xw, "bfloat16")[0][0]
        else:
            want = oracle.ring_fold_window(xw, a, n, "bfloat16")
        got = t[0][a:b].view(torch.int16).cpu().numpy().view(np.uint16)
        assert same_bits(got, want, "bfloat16"), f"window {a}:{b} first diff {first_diff(got, want, 'bfloat16')}"
    del t
    torch.cuda.empty_cache()
