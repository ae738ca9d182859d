"""Host-side checks of libra.so that need no GPU: it loads, exports every symbol
include/ra.h declares, and its host logic (chunk partition, argument checks)
agrees with the oracle and the header's contract.  No call here reaches a kernel."""

import ctypes
import os

import pytest

import oracle
from ring_all_reduce_schedule_amd import binding as B


def test_library_exports_every_header_symbol():
    names = B.header_symbols()
    assert len(names) >= 12
    lib = B.lib()
    for name in names:
        assert hasattr(lib, name), name
    # and the binding wraps each of them under the same name
    for name in names:
        assert name in B._SIGNATURES, name
        assert hasattr(B, name), name


@pytest.mark.parametrize("n,p", [(n, p) for p in (1, 2, 3, 4, 8, 9, 64)
                                 for n in (0, 1, 3, 4, 63, 64, 65, 1000, 1_000_003,
                                           67_108_864, 8_000_000_000, 2**40 + 7)])
def test_chunk_bounds_matches_oracle(n, p):
    starts = B.ra_chunk_bounds(n, p)
    assert list(zip(starts[:-1], starts[1:])) == oracle.chunk_bounds(n, p)


def test_chunk_bounds_errors():
    for n, p, code in [(4, 0, B.RA_ERR_INVALID_ARG), (-1, 4, B.RA_ERR_INVALID_ARG),
                       (4, 65, B.RA_ERR_UNSUPPORTED)]:
        with pytest.raises(B.RaError) as e:
            B.ra_chunk_bounds(n, p)
        assert e.value.code == code
    assert B.lib().ra_chunk_bounds(4, 2, None) == B.RA_ERR_INVALID_ARG


def _ptrs(addrs):
    return (ctypes.c_void_p * len(addrs))(*addrs)


def _call(addrs, n, dtype=B.RA_FLOAT32, op=B.RA_SUM, algo=-1, p=None):
    lib = B.lib()
    p = len(addrs) if p is None else p
    return lib.ra_allreduce_ex(_ptrs(addrs) if addrs is not None else None, p, n, dtype, op,
                               algo, None, None)


MiB = 1 << 20


def test_argument_errors_are_reported_before_any_gpu_work():
    base = 0x7f0000000000
    ok = [base + i * MiB for i in range(4)]
    assert _call(None, 16, p=4) == B.RA_ERR_INVALID_ARG
    assert _call(ok, 16, p=0) == B.RA_ERR_INVALID_ARG
    assert _call(ok, -1) == B.RA_ERR_INVALID_ARG
    assert _call(ok, 16, dtype=7) == B.RA_ERR_INVALID_ARG
    assert _call(ok, 16, op=7) == B.RA_ERR_UNSUPPORTED
    # averages need a floating-point type
    for dt in (B.RA_INT32, B.RA_INT64):
        assert _call(ok, 16, dtype=dt, op=B.RA_AVG) == B.RA_ERR_UNSUPPORTED
    # wide accumulation: the fused pass on bf16 / fp16 / fp32 only
    lib = B.lib()
    o = B._options(wide=True)
    for algo, dt in ((B.ALGOS["ring_step"], B.RA_BFLOAT16), (B.ALGOS["tree"], B.RA_FLOAT32),
                     (B.ALGOS["fused"], B.RA_INT32), (B.ALGOS["fused"], B.RA_FLOAT64)):
        assert lib.ra_allreduce_ex(_ptrs(ok), 4, 16, dt, 0, algo, ctypes.byref(o), None) == B.RA_ERR_UNSUPPORTED
    assert _call(ok, 16, algo=99) == B.RA_ERR_INVALID_ARG
    assert _call([base + i * MiB for i in range(65)], 16) == B.RA_ERR_UNSUPPORTED
    assert _call([ok[0], 0, ok[2], ok[3]], 16) == B.RA_ERR_INVALID_ARG
    assert _call([ok[0], ok[1] + 8, ok[2], ok[3]], 16) == B.RA_ERR_MISALIGNED
    # 16 float32 = 64 bytes: buffers 32 bytes apart overlap
    assert _call([base, base + 32, base + 4096, base + 8192], 16) == B.RA_ERR_ALIAS
    assert "overlap" in B.ra_last_error()
    # ... 64 bytes apart do not (and n = 0 never touches the device)
    assert _call([base, base + 64, base + 128, base + 192], 0) == B.RA_OK
    # a world of one is a no-op
    assert _call([base], 1 << 20) == B.RA_OK
    # empty buffers may be NULL (nothing is read or written)
    assert _call([0, 0, 0], 0) == B.RA_OK
    lib = B.lib()
    assert lib.ra_reduce_scatter_ex(_ptrs(ok), 4, 16, 0, 0, B.ALGOS["tree"], None, None) == B.RA_ERR_UNSUPPORTED
    assert lib.ra_all_gather_ex(_ptrs(ok), 4, 16, 0, B.ALGOS["ring_bidir"], None, None) == B.RA_ERR_UNSUPPORTED
    for bad in (-1, 65):
        o = B._options(channels=bad)
        assert lib.ra_allreduce_ex(_ptrs(ok), 4, 16, 1, 0, B.ALGOS["ring_channels"],
                                   ctypes.byref(o), None) == B.RA_ERR_INVALID_ARG
        assert lib.ra_reduce_scatter_ex(_ptrs(ok), 4, 16, 1, 0, B.ALGOS["ring_channels"],
                                        ctypes.byref(o), None) == B.RA_ERR_INVALID_ARG
    assert lib.ra_stream_copy(None, None, 16, None) == B.RA_ERR_INVALID_ARG
    assert lib.ra_stream_copy(base, base + 4096, 15, None) == B.RA_ERR_INVALID_ARG
    assert lib.ra_stream_copy_resident(None, None, 16, 8, None) == B.RA_ERR_INVALID_ARG
    assert lib.ra_stream_copy_resident(base, base + 4096, 15, 8, None) == B.RA_ERR_INVALID_ARG
    assert lib.ra_stream_copy_resident(base, base + 4096, 16, -1, None) == B.RA_ERR_INVALID_ARG
    assert lib.ra_stream_copy_resident(base + 8, base + 4096, 16, 8, None) == B.RA_ERR_MISALIGNED


def test_status_strings():
    names = ["RA_OK", "RA_ERR_INVALID_ARG", "RA_ERR_UNSUPPORTED", "RA_ERR_ALIAS",
             "RA_ERR_MISALIGNED", "RA_ERR_HIP", "RA_ERR_TIMEOUT"]
    assert [B.ra_status_string(i) for i in range(7)] == names
    assert B.ra_status_string(99) == "RA_ERR_UNKNOWN"


def test_options_struct_layout():
    # int64, int64, int32, uint32, pointer, int32, int32, double, double: 56 bytes
    assert ctypes.sizeof(B.ra_options) == 56
    assert B.ra_options.step_ts.offset == 24
    assert B.ra_options.channels.offset == 32
    assert B.ra_options.group.offset == 36
    assert B.ra_options.link_alpha_us.offset == 40


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    monkeypatch.setattr(B, "_lib", None)
    monkeypatch.setattr(B, "LIB_PATH", str(tmp_path / "absent.so"))
    with pytest.raises(RuntimeError, match="no fallback"):
        B.lib()


@pytest.mark.parametrize("p", [1, 2, 3, 4, 8, 9, 16, 64])
def test_select_algo_follows_the_cost_model(p):
    # the library's AUTO choice against the oracle's pricing of the same call
    for dtype, item in (("int32", 4), ("float32", 4), ("bfloat16", 2)):
        for n in (0, 1, 1000, 65_536, 524_288, 10**7, 8 * 10**9):
            for alpha_us in (1.0, 10.0, 20.0):
                for gbps in (25.0, 50.0, 450.0):
                    s = n * item
                    tr = oracle.cost.t_ring(p, s, gbps * 1e9, alpha_us * 1e-6)
                    tt = oracle.cost.t_tree(p, s, gbps * 1e9, alpha_us * 1e-6)
                    if tr > 0 and abs(tr - tt) / tr < 1e-9:
                        continue        # a tie up to rounding: either answer is right
                    want = oracle.cost.choose_ring_or_tree(p, s, gbps * 1e9, alpha_us * 1e-6)
                    got = B.ra_select_algo(p, n, dtype, link_alpha_us=alpha_us, link_GBps=gbps)
                    assert got == {"ring": "ring_step", "tree": "tree"}[want], (p, n, dtype, alpha_us, gbps)
    # no link model: the one-memory fused pass
    assert B.ra_select_algo(p, 1 << 20, "bfloat16") == "fused"


def test_select_algo_errors():
    lib = B.lib()
    out = ctypes.c_int()
    for args, code in [((0, 16, 1), B.RA_ERR_INVALID_ARG), ((4, -1, 1), B.RA_ERR_INVALID_ARG),
                       ((4, 16, 9), B.RA_ERR_INVALID_ARG), ((65, 16, 1), B.RA_ERR_UNSUPPORTED)]:
        assert lib.ra_select_algo(*args, None, ctypes.byref(out)) == code
    assert lib.ra_select_algo(4, 16, 1, None, None) == B.RA_ERR_INVALID_ARG
    for a, b in ((-1.0, 50.0), (10.0, -5.0), (float("nan"), 50.0), (float("inf"), 50.0)):
        o = B._options(link_alpha_us=a, link_GBps=b)
        assert lib.ra_select_algo(4, 16, 1, ctypes.byref(o), ctypes.byref(out)) == B.RA_ERR_INVALID_ARG
    # AUTO is an all-reduce choice only
    base = 0x7f0000000000
    ptrs = (ctypes.c_void_p * 4)(*[base + i * (1 << 20) for i in range(4)])
    assert lib.ra_reduce_scatter_ex(ptrs, 4, 16, 1, 0, B.ALGOS["auto"], None, None) == B.RA_ERR_UNSUPPORTED


def test_hier_group_errors():
    lib = B.lib()
    base = 0x7f0000000000
    ptrs = (ctypes.c_void_p * 8)(*[base + i * (1 << 20) for i in range(8)])
    for bad in (-1, 3, 9):
        o = B._options(group=bad)
        for algo in ("hier", "hier_fused"):
            assert lib.ra_allreduce_ex(ptrs, 8, 16, 1, 0, B.ALGOS[algo], ctypes.byref(o),
                                       None) == B.RA_ERR_INVALID_ARG
    o = B._options(wide=True, group=4)
    assert lib.ra_allreduce_ex(ptrs, 8, 16, 2, 0, B.ALGOS["hier_fused"], ctypes.byref(o),
                               None) == B.RA_ERR_UNSUPPORTED


def test_rank_buffers_rejects_host_tensors_and_empty_lists():
    """The binding's marshalling checks run before any library call."""
    import torch
    with pytest.raises(ValueError):
        B.RankBuffers([])
    with pytest.raises(ValueError):
        B.RankBuffers([torch.zeros(4), torch.zeros(4)])
    with pytest.raises(ValueError):
        B.ra_allreduce([torch.zeros(4)])
