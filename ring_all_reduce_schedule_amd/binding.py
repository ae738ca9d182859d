"""Thin ctypes binding of libra.so: the C ABI of include/ra.h under the same names.

Only argument marshalling happens here: torch tensors are turned into device
pointers, element counts, dtype codes and the current HIP stream, and nonzero
status codes are raised as ``RaError``.  Every step of the all-reduce runs in the
library's HIP kernels.  If libra.so has not been built, the first call raises:
there is no fallback path.
"""

import array
import ctypes
import os
import re

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libra.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "ra.h")

RA_OK, RA_ERR_INVALID_ARG, RA_ERR_UNSUPPORTED, RA_ERR_ALIAS = 0, 1, 2, 3
RA_ERR_MISALIGNED, RA_ERR_HIP, RA_ERR_TIMEOUT = 4, 5, 6
RA_INT32, RA_FLOAT32, RA_BFLOAT16, RA_FLOAT16, RA_FLOAT64, RA_INT64 = 0, 1, 2, 3, 4, 5
RA_SUM, RA_MAX, RA_AVG = 0, 1, 2
RA_MAX_RANKS = 64
RA_FLAG_FORCE_TIMEOUT = 1
RA_FLAG_WIDE_ACCUM = 2
RA_FLAG_STRESS = 4
RA_FLAG_RENEW_COUNTERS = 8
RA_FLAG_PHASES = 16
RA_FLAG_NO_PHASES = 32
OPS = {"sum": RA_SUM, "max": RA_MAX, "avg": RA_AVG}

ALGOS = {"default": -1, "ring_step": 0, "ring_pipelined": 1, "ring_bidir": 2,
         "fused": 3, "tree": 4, "ring_channels": 5, "auto": 6, "hier": 7,
         "hier_fused": 8, "ring_pipelined_flags": 9}
ALGO_NAMES = {v: k for k, v in ALGOS.items()}
DTYPE_NAMES = {"int32": RA_INT32, "float32": RA_FLOAT32, "bfloat16": RA_BFLOAT16,
               "float16": RA_FLOAT16, "float64": RA_FLOAT64, "int64": RA_INT64}


class RaError(RuntimeError):
    """A libra.so call returned a nonzero status."""

    def __init__(self, code, name, message):
        super().__init__(f"{name}: {message}")
        self.code, self.name, self.message = code, name, message


class ra_options(ctypes.Structure):
    _fields_ = [("slice_elems", ctypes.c_int64),
                ("timeout_us", ctypes.c_int64),
                ("grid", ctypes.c_int32),
                ("flags", ctypes.c_uint32),
                ("step_ts", ctypes.c_void_p),
                ("channels", ctypes.c_int32),
                ("group", ctypes.c_int32),
                ("link_alpha_us", ctypes.c_double),
                ("link_GBps", ctypes.c_double)]


_lib = None
_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_int = ctypes.c_int

_SIGNATURES = {
    "ra_chunk_bounds": (_int, [_i64, _int, ctypes.POINTER(ctypes.c_int64)]),
    "ra_reduce_scatter": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _int, _vp]),
    "ra_all_gather": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _vp]),
    "ra_allreduce": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _int, _vp]),
    "ra_allreduce_ex": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _int, _int,
                               ctypes.POINTER(ra_options), _vp]),
    "ra_allreduce_noalloc": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _int, _int,
                                    ctypes.POINTER(ra_options), _vp]),
    "ra_reduce_scatter_ex": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _int, _int,
                                    ctypes.POINTER(ra_options), _vp]),
    "ra_all_gather_ex": (_int, [ctypes.POINTER(_vp), _int, _i64, _int, _int,
                                ctypes.POINTER(ra_options), _vp]),
    "ra_stream_status": (_int, [_vp]),
    "ra_select_algo": (_int, [_int, _i64, _int, ctypes.POINTER(ra_options),
                              ctypes.POINTER(_int)]),
    "ra_status_string": (ctypes.c_char_p, [_int]),
    "ra_last_error": (ctypes.c_char_p, []),
    "ra_wallclock_hz": (_int, [ctypes.POINTER(ctypes.c_int64)]),
    "ra_stream_copy": (_int, [_vp, _vp, _i64, _vp]),
    "ra_stream_copy_resident": (_int, [_vp, _vp, _i64, _int, _vp]),
}


def lib():
    """The loaded libra.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} not found: build it with "
                "`python -m ring_all_reduce_schedule_amd.build` (there is no fallback)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype, fn.argtypes = res, args
        _lib = handle
    return _lib


def header_symbols():
    """Function names declared in include/ra.h."""
    with open(HEADER_PATH) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(ra_\w+)\s*\(", text, re.M)))


def ra_status_string(code):
    return lib().ra_status_string(int(code)).decode()


def ra_last_error():
    return lib().ra_last_error().decode()


def _check(code):
    if code != RA_OK:
        raise RaError(code, ra_status_string(code), ra_last_error())
    return code


# ---------------------------------------------------------------- marshalling

def _torch():
    import torch
    return torch


def dtype_code(t):
    torch = _torch()
    codes = {torch.int32: RA_INT32, torch.float32: RA_FLOAT32, torch.bfloat16: RA_BFLOAT16,
             torch.float16: RA_FLOAT16, torch.float64: RA_FLOAT64, torch.int64: RA_INT64}
    if t.dtype not in codes:
        raise TypeError(f"unsupported dtype {t.dtype} "
                        "(int32, int64, float16, bfloat16, float32, float64)")
    return codes[t.dtype]


def _stream_handle(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _marshal_list(tensors):
    """(pointer array, p, n, dtype code, device) for a sequence of rank tensors,
    checked: same dtype, length and device, contiguous, on a GPU.  The pointer
    array is a ctypes view of an array.array, which is several times cheaper to
    build than a ctypes array from a list."""
    if len(tensors) == 0:
        raise ValueError("need at least one rank buffer")
    t0 = tensors[0]
    if not t0.is_cuda:
        raise ValueError("rank buffers must be device tensors")
    dt, n, dev = t0.dtype, t0.numel(), t0.get_device()
    for t in tensors:
        if t.dtype is not dt or t.numel() != n or t.get_device() != dev:
            raise ValueError("rank buffers must share dtype, length and device")
        if not t.is_contiguous():
            raise ValueError("rank buffers must be contiguous")
    code = dtype_code(t0)
    table = array.array("Q", [t.data_ptr() for t in tensors])
    ptrs = (ctypes.c_void_p * len(tensors)).from_buffer(table)
    return ptrs, len(tensors), n, code, t0.device


class RankBuffers:
    """p rank tensors checked and marshalled once, for repeated calls.

    Every entry point accepts one in place of a list of tensors.  A list is
    checked and turned into a pointer table on every call, which costs about
    0.8 us of host time per rank (about 50 us at p = 64, more than a fused
    all-reduce of 1 MiB per rank takes on the GPU); this object does it once.
    It holds references to the tensors, so their memory stays allocated while it
    lives.  The tensors must not be resized or re-pointed (``resize_``,
    ``set_``) meanwhile: the table holds the addresses they had when it was made,
    and a call raises if the first rank's address or length has changed."""

    __slots__ = ("tensors", "ptrs", "p", "n", "dtype", "device", "_first")

    def __init__(self, tensors):
        self.tensors = tuple(tensors)
        self.ptrs, self.p, self.n, self.dtype, self.device = _marshal_list(self.tensors)
        self._first = (self.tensors[0].data_ptr(), self.n)

    def __len__(self):
        return self.p


def _marshal(tensors):
    """(pointer array, p, n, dtype code, device) for a list of rank tensors or a
    RankBuffers."""
    if isinstance(tensors, RankBuffers):
        t0 = tensors.tensors[0]
        if (t0.data_ptr(), t0.numel()) != tensors._first:
            raise ValueError("a rank tensor of this RankBuffers was resized or re-pointed")
        return tensors.ptrs, tensors.p, tensors.n, tensors.dtype, tensors.device
    return _marshal_list(tensors)


def _options(slice_elems=0, timeout_us=0, grid=0, flags=0, step_ts=None, channels=0,
             link_alpha_us=0.0, link_GBps=0.0, wide=False, group=0):
    o = ra_options()
    o.slice_elems = int(slice_elems)
    o.timeout_us = int(timeout_us)
    o.grid = int(grid)
    o.flags = int(flags) | (RA_FLAG_WIDE_ACCUM if wide else 0)
    o.step_ts = None if step_ts is None else int(step_ts.data_ptr())
    o.channels = int(channels)
    o.group = int(group)
    o.link_alpha_us = float(link_alpha_us)
    o.link_GBps = float(link_GBps)
    return o


def _algo(algo):
    return ALGOS[algo] if isinstance(algo, str) else int(algo)


def _op(op):
    if isinstance(op, str):
        return OPS.get(op, -1)
    return int(op)


# ---------------------------------------------------------------- entry points

def ra_chunk_bounds(n, p):
    """List of p + 1 chunk starts (host only)."""
    starts = (ctypes.c_int64 * (max(p, 0) + 1))()
    _check(lib().ra_chunk_bounds(int(n), int(p), starts))
    return list(starts)


def ra_allreduce(tensors, op="sum", stream=None):
    ptrs, p, n, dt, dev = _marshal(tensors)
    return _check(lib().ra_allreduce(ptrs, p, n, dt, _op(op), _stream_handle(stream, dev)))


def ra_allreduce_ex(tensors, algo="default", op="sum", stream=None, **opts):
    ptrs, p, n, dt, dev = _marshal(tensors)
    o = _options(**opts)
    return _check(lib().ra_allreduce_ex(ptrs, p, n, dt, _op(op), _algo(algo), ctypes.byref(o),
                                        _stream_handle(stream, dev)))


def ra_allreduce_noalloc(tensors, algo="default", op="sum", stream=None, **opts):
    ptrs, p, n, dt, dev = _marshal(tensors)
    o = _options(**opts)
    return _check(lib().ra_allreduce_noalloc(ptrs, p, n, dt, _op(op), _algo(algo), ctypes.byref(o),
                                             _stream_handle(stream, dev)))


def ra_reduce_scatter(tensors, op="sum", stream=None):
    ptrs, p, n, dt, dev = _marshal(tensors)
    return _check(lib().ra_reduce_scatter(ptrs, p, n, dt, _op(op), _stream_handle(stream, dev)))


def ra_reduce_scatter_ex(tensors, algo="default", op="sum", stream=None, **opts):
    ptrs, p, n, dt, dev = _marshal(tensors)
    o = _options(**opts)
    return _check(lib().ra_reduce_scatter_ex(ptrs, p, n, dt, _op(op), _algo(algo),
                                             ctypes.byref(o), _stream_handle(stream, dev)))


def ra_all_gather(tensors, stream=None):
    ptrs, p, n, dt, dev = _marshal(tensors)
    return _check(lib().ra_all_gather(ptrs, p, n, dt, _stream_handle(stream, dev)))


def ra_all_gather_ex(tensors, algo="default", stream=None, **opts):
    ptrs, p, n, dt, dev = _marshal(tensors)
    o = _options(**opts)
    return _check(lib().ra_all_gather_ex(ptrs, p, n, dt, _algo(algo), ctypes.byref(o),
                                         _stream_handle(stream, dev)))


def ra_select_algo(p, n, dtype, **opts):
    """Name of the algorithm RA_ALGO_AUTO would run (host only)."""
    code = DTYPE_NAMES[dtype] if isinstance(dtype, str) else int(dtype)
    o = _options(**opts)
    out = ctypes.c_int(-1)
    _check(lib().ra_select_algo(int(p), int(n), code, ctypes.byref(o), ctypes.byref(out)))
    return ALGO_NAMES[out.value]


def ra_stream_status(stream=None, device=None):
    torch = _torch()
    dev = device if device is not None else torch.cuda.current_device()
    return _check(lib().ra_stream_status(_stream_handle(stream, dev)))


def ra_wallclock_hz():
    hz = ctypes.c_int64()
    _check(lib().ra_wallclock_hz(ctypes.byref(hz)))
    return hz.value


def ra_stream_copy(dst, src, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    return _check(lib().ra_stream_copy(ctypes.c_void_p(dst.data_ptr()),
                                       ctypes.c_void_p(src.data_ptr()), nbytes,
                                       _stream_handle(stream, src.device)))


def ra_stream_copy_resident(dst, src, grid=0, stream=None):
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst smaller than src")
    return _check(lib().ra_stream_copy_resident(ctypes.c_void_p(dst.data_ptr()),
                                                ctypes.c_void_p(src.data_ptr()), nbytes,
                                                int(grid), _stream_handle(stream, src.device)))
