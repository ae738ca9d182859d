"""Build libra.so (HIP, gfx950) in-tree with hipcc.

    python -m ring_all_reduce_schedule_amd.build

Every call compiles from source.  Flags:
  --offload-arch=gfx950              MI355X only, no other targets
  -Xclang -target-feature -Xclang -packed-fp32-ops
                                     no packed fp32 instructions are generated
  -ffp-contract=off                  each hop's add is rounded on its own
"""

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libra.so")

SOURCES = ["ra_fused.hip", "ra_steps.hip", "ra_copy.hip", "ra_api.cpp"]
HEADERS = ["ra_elem.h", "ra_sync.h", "ra_internal.h"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libra.so")
    return exe


def command(out=LIB):
    return [hipcc(), "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
            "-x", "hip", "-ffp-contract=off",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wno-unused-command-line-argument",
            "-I", INCLUDE, "-I", CSRC,
            *[os.path.join(CSRC, s) for s in SOURCES], "-o", out]


def build(verbose=False):
    tmp = LIB + ".tmp"
    cmd = command(tmp)
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libra.so")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    noise = [ln for ln in res.stderr.splitlines() if ln.strip()
             and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
