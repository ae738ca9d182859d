"""Seeded synthetic inputs shared by the tests, the benchmark and the parity checks.

Nothing in this module performs any step of the all-reduce: it only draws the
p per-rank input buffers.  Both the CPU oracle (via the tests) and the HIP path
receive exactly the arrays produced here.

Workloads (p virtual ranks, N elements per rank):

  trace_p4_fp32_n4        p=4,  N=4 fp32, rank r holds (r+1) * [1, 10, 100, 1000]
                          (the worked trace in "Ring All-Reduce, in depth",
                          section "Tracing four GPUs")
  p9_int32_n1000003       p=9,  N=1,000,003 int32, uniform on [-1000, 1000], seed 0
  p64_bf16_1MiB           p=64, N=524,288 bf16 (1 MiB per rank), normal(0, 1), seed 1
  p8_fp32_256MiB          p=8,  N=67,108,864 fp32 (256 MiB per rank), normal(0, 1e-2), seed 2
  p8_bf16_16GB            p=8,  N=8e9 bf16 (16 GB per rank, 128 GB in all), normal(0, 1e-3),
                          seed 3, drawn on the device (see ``device_normal_bf16``)

Recipe: ``numpy.random.default_rng(seed)``; ranks drawn one after another,
r = 0 .. p-1.  Integers: ``integers(lo, hi, N, endpoint=True)``.  Normals:
``standard_normal(N, float32) * float32(sigma)``, and for bf16 the float32
draw is narrowed by torch's CPU float32 -> bfloat16 conversion (round to
nearest even).  bf16 arrays are returned as uint16 bit patterns.
"""

import numpy as np


WORKLOADS = {
    "trace_p4_fp32_n4": dict(p=4, n=4, dtype="float32", kind="trace"),
    "p9_int32_n1000003": dict(p=9, n=1_000_003, dtype="int32", kind="uniform_int",
                              lo=-1000, hi=1000, seed=0),
    "p64_bf16_1MiB": dict(p=64, n=524_288, dtype="bfloat16", kind="normal",
                          sigma=1.0, seed=1),
    "p8_fp32_256MiB": dict(p=8, n=67_108_864, dtype="float32", kind="normal",
                           sigma=1e-2, seed=2),
    "p8_bf16_16GB": dict(p=8, n=8_000_000_000, dtype="bfloat16", kind="normal",
                         sigma=1e-3, seed=3, on_device=True),
}

ITEMSIZE = {"int32": 4, "float32": 4, "bfloat16": 2, "float16": 2, "float64": 8, "int64": 8}
INTS = ("int32", "int64")


def f32_to_bf16_bits_torch(x):
    """float32 numpy array -> bf16 bit patterns via torch's CPU conversion."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def trace_inputs():
    """p=4, N=4: rank r holds (r + 1) * [1, 10, 100, 1000]."""
    base = np.array([1, 10, 100, 1000], dtype=np.float32)
    return [np.float32(r + 1) * base for r in range(4)]


def uniform_int(p, n, lo, hi, seed, dtype="int32"):
    rng = np.random.default_rng(seed)
    t = np.int64 if dtype == "int64" else np.int32
    return [rng.integers(lo, hi, n, endpoint=True, dtype=t) for _ in range(p)]


def _store(x32, dtype):
    """float32 draws in the storage of ``dtype`` (bf16 as bit patterns)."""
    if dtype == "bfloat16":
        return f32_to_bf16_bits_torch(x32)
    if dtype == "float16":
        return x32.astype(np.float16)
    return x32


def normal(p, n, sigma, seed, dtype):
    """normal(0, sigma) draws: float64 drawn in float64, the rest as float32
    draws narrowed to the element type (round to nearest even)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(p):
        if dtype == "float64":
            out.append(rng.standard_normal(n) * float(sigma))
        else:
            out.append(_store(rng.standard_normal(n, dtype=np.float32) * np.float32(sigma), dtype))
    return out


def small_int_valued(p, n, dtype, lo, hi, seed):
    """Integer-valued inputs stored in ``dtype`` (exactly representable)."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(p):
        v = rng.integers(lo, hi, n, endpoint=True)
        if dtype in INTS:
            out.append(v.astype(np.int64 if dtype == "int64" else np.int32))
        elif dtype == "float64":
            out.append(v.astype(np.float64))
        else:
            out.append(_store(v.astype(np.float32), dtype))
    return out


def make_inputs(p, n, dtype, seed, kind="normal", sigma=1.0, lo=-1000, hi=1000):
    """Generic host inputs for a (p, n, dtype) case."""
    if kind == "trace":
        return trace_inputs()
    if dtype in INTS or kind == "uniform_int":
        return uniform_int(p, n, lo, hi, seed, dtype if dtype in INTS else "int32")
    if kind == "small_int":
        return small_int_valued(p, n, dtype, lo, hi, seed)
    return normal(p, n, sigma, seed, dtype)


def workload_inputs(name):
    """Host inputs of a named workload (not for the on-device one)."""
    w = WORKLOADS[name]
    if w.get("on_device"):
        raise ValueError(f"{name} is drawn on the device; use device_normal_bf16")
    return make_inputs(w["p"], w["n"], w["dtype"], w.get("seed", 0), w["kind"],
                       w.get("sigma", 1.0), w.get("lo", -1000), w.get("hi", 1000))


DEVICE_BLOCK = 1 << 28     # float32 elements per device draw (1 GiB)


def device_normal_bf16(tensors, sigma, seed):
    """Fill bf16 CUDA tensors (one per rank) with normal(0, sigma) draws on the device.

    torch's device generator seeded with ``seed`` draws float32 normals in
    blocks of 2**28 elements, rank after rank and block after block; each block
    is scaled by float32(sigma) and narrowed to bf16 by torch.  Windows of the
    result are copied to the host for the oracle before any all-reduce runs.
    """
    import torch
    dev = tensors[0].device
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    for t in tensors:
        flat = t.view(-1)
        n = flat.numel()
        for lo in range(0, n, DEVICE_BLOCK):
            hi = min(n, lo + DEVICE_BLOCK)
            blk = torch.randn(hi - lo, generator=g, device=dev, dtype=torch.float32)
            blk.mul_(sigma)
            flat[lo:hi].copy_(blk)
            del blk
