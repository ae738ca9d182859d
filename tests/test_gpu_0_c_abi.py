"""The C ABI from plain C (tests/c/abi_check.c, built by build()): device buffers
from hipMalloc, no Python binding and no torch.  It checks every algorithm's int32
all-reduce against the closed-form sum, the reduce-scatter's owned chunks, the
all-gather, and the argument errors.

The check runs as a child process before this test process touches the GPU (the
module sorts first among the GPU tests and imports no GPU library)."""

import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "abi_check")


def test_c_program_uses_the_abi():
    torch = sys.modules.get("torch")
    if torch is not None and torch.cuda.is_initialized():
        pytest.skip("the GPU is already initialised in this process; run this module first")
    assert os.path.exists(BIN), "tests/c/abi_check is missing: run build() first"
    print("[case] tests/c/abi_check", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "PASSED" in res.stdout
