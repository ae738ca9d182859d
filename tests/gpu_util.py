"""Helpers for the GPU tests: host arrays <-> rank tensors on cuda:0."""

import numpy as np
import torch

TORCH_DTYPE = {"int32": torch.int32, "float32": torch.float32, "bfloat16": torch.bfloat16,
               "float16": torch.float16, "float64": torch.float64, "int64": torch.int64}
UINT_VIEW = {"int32": np.uint32, "float32": np.uint32, "bfloat16": np.uint16,
             "float16": np.uint16, "float64": np.uint64, "int64": np.uint64}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return torch.device("cuda:0")


def to_dev(arrs, dtype, device="cuda:0"):
    out = []
    for a in arrs:
        if dtype == "bfloat16":
            t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(np.ascontiguousarray(a))
        out.append(t.to(device))
    return out


def from_dev(tensors, dtype):
    out = []
    for t in tensors:
        t = t.detach().cpu()
        if dtype == "bfloat16":
            out.append(t.view(torch.int16).numpy().view(np.uint16).copy())
        else:
            out.append(t.numpy().copy())
    return out


def same_bits(a, b, dtype):
    a = np.asarray(a)
    b = np.asarray(b)
    return a.shape == b.shape and np.array_equal(a.view(UINT_VIEW[dtype]), b.view(UINT_VIEW[dtype]))


def first_diff(a, b, dtype):
    u = UINT_VIEW[dtype]
    idx = np.nonzero(np.asarray(a).view(u) != np.asarray(b).view(u))[0]
    return None if idx.size == 0 else int(idx[0])
