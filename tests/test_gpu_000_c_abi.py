"""The C ABI from plain C (tests/c/abi_check.c, built by build()): device buffers
from hipMalloc, no Python binding and no torch.  It checks every algorithm's int32
all-reduce against the closed-form sum, the reduce-scatter's owned chunks, the
all-gather, and the argument errors.

The check runs as a child process.  The module sorts first among the GPU tests and
imports no GPU library, so the child normally has the GPU to itself; every launch
the library makes is an ordinary one, so it also runs beside a test process that
already holds the GPU."""

import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "abi_check")


def test_c_program_uses_the_abi():
    assert os.path.exists(BIN), "tests/c/abi_check is missing: run build() first"
    print("[case] tests/c/abi_check", flush=True)
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=120)
    print(res.stdout)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "PASSED" in res.stdout
