"""Build libra.so (HIP, gfx950) in-tree with hipcc.

    python -m ring_all_reduce_schedule_amd.build

Every call compiles every source from scratch (one hipcc per source, in
parallel, objects under _build/) and links them.  Flags:
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

SOURCES = ["ra_fused.hip", "ra_rider.hip", "ra_steps.hip", "ra_copy.hip", "ra_api.cpp"]
HEADERS = ["ra_elem.h", "ra_sync.h", "ra_internal.h"]


def hipcc():
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; ROCm is required to build libra.so")
    return exe


BUILD = os.path.join(ROOT, "_build")

FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-ffp-contract=off",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def compile_command(src, obj):
    return [hipcc(), *FLAGS, "-x", "hip", "-I", INCLUDE, "-I", CSRC, "-c",
            os.path.join(CSRC, src), "-o", obj]


def link_command(objs, out):
    return [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", out]


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(" ".join(cmd) + "\n" + res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libra.so")
    # hipcc's host pass warns that it does not know the packed-fp32 feature
    return [ln for ln in res.stderr.splitlines() if ln.strip()
            and "packed-fp32-ops" not in ln and "not a recognized feature" not in ln]


C_CHECK_SRC = os.path.join(ROOT, "tests", "c", "abi_check.c")
C_CHECK_BIN = os.path.join(ROOT, "tests", "c", "abi_check")


def c_check_command(out=C_CHECK_BIN):
    """The plain-C user of the ABI: gcc, no HIP compiler, linked against libra.so
    (found next to the package through an rpath relative to the binary)."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    return ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
            "-I", INCLUDE, "-I", os.path.join(rocm, "include"), C_CHECK_SRC,
            "-L", PKG, "-lra", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
            "-Wl,-rpath,$ORIGIN/../../ring_all_reduce_schedule_amd",
            "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", out]


HOST_CHECK_SRC = os.path.join(ROOT, "tests", "c", "host_check.cpp")
HOST_CHECK_BIN = os.path.join(ROOT, "tests", "c", "host_check")


def host_check_commands(objs, out=HOST_CHECK_BIN):
    """The host side of the ABI under AddressSanitizer: ra_api.cpp again with the
    sanitizer on its host code only (each -fsanitize= right after -Xarch_host),
    linked by g++ with the kernels' objects into a program that needs no GPU."""
    rocm = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    api = os.path.join(BUILD, "ra_api_asan.o")
    main = os.path.join(BUILD, "host_check.o")
    kernels = [o for o in objs if not o.endswith("ra_api.o")]
    return [
        [hipcc(), *FLAGS, "-x", "hip", "-I", INCLUDE, "-I", CSRC, "-Xarch_host", "-fsanitize=address",
         "-Xarch_host", "-fno-omit-frame-pointer", "-c", os.path.join(CSRC, "ra_api.cpp"), "-o", api],
        ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address", "-fno-omit-frame-pointer",
         "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(rocm, "include"), "-c",
         HOST_CHECK_SRC, "-o", main],
        ["g++", "-fsanitize=address", main, api, *kernels, "-L", os.path.join(rocm, "lib"),
         "-lamdhip64", "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", out],
    ]


def build(verbose=False):
    """Compile every source (in parallel) and link libra.so; always from scratch.
    Then build the plain-C ABI check against it."""
    from concurrent.futures import ThreadPoolExecutor
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, os.path.splitext(src)[0] + ".o") for src in SOURCES]
    cmds = [compile_command(src, obj) for src, obj in zip(SOURCES, objs)]
    if verbose:
        for c in cmds:
            print(" ".join(c), flush=True)
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 1)) as ex:
        noise = [ln for out in ex.map(_run, cmds) for ln in out]
    tmp = LIB + ".tmp"
    noise += _run(link_command(objs, tmp))
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    os.replace(tmp, LIB)
    noise += _run(c_check_command())
    for cmd in host_check_commands(objs):
        noise += _run(cmd)
    if verbose and noise:
        sys.stderr.write("\n".join(noise) + "\n")
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
