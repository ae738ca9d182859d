"""The C ABI's host code under AddressSanitizer (CPU only).

tests/c/host_check.cpp drives every entry point's argument checks, chunk bounds,
overlap detection on 2000 random pointer sets, and algorithm selection, against
a copy of the library's host code built with -fsanitize=address (build()
compiles it).  Any heap or stack misuse aborts the program."""

import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
BIN = os.path.join(ROOT, "tests", "c", "host_check")


def test_host_code_is_clean_under_asan():
    assert os.path.exists(BIN), "tests/c/host_check is missing: run build() first"
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1")
    res = subprocess.run([BIN], capture_output=True, text=True, timeout=300, env=env)
    assert res.returncode == 0, res.stdout[-4000:] + res.stderr[-4000:]
    assert "PASSED" in res.stdout
