"""Which launches the step algorithms and the one-pass calls choose (through the C
ABI, RA_DEBUG=1).

With RA_DEBUG=1 the library prints one line per call with the grid and the
number of kernel launches.  A child process runs a few calls and the test checks
the documented choices:

* steps that move at most 256 vectors: one launch of one workgroup;
* larger steps: one launch per step (2(p-1) for the ring, 2*ceil(log2 p) for
  the tree);
* a caller's grid, or channels: one persistent launch of that many workgroups;
* the library's own persistent grids: 256-thread workgroups, 512-thread ones
  from 4 MiB per rank, 1024-thread ones from 16 MiB (1 per compute unit);
* the slice-carrying pipelined ring: one launch, one workgroup per 4 KiB slice
  of every chunk.
* the one-pass all-reduce and all-gather of 8 ranks of at least 12 GiB each:
  8 workgroups per compute unit (read/write phases); averages, reduce-scatters,
  other rank counts and smaller calls: one workgroup per tile, unless
  RA_FLAG_PHASES forces the phases.

Every launch is an ordinary one (persistent grids are sized to stay resident,
not launched cooperatively), so the child can run while the test process holds
the GPU too.
"""

import os
import re
import subprocess
import sys

import pytest
import torch

from tests.gpu_util import require_gpu

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from ring_all_reduce_schedule_amd import binding as B
def bufs(p, n):
    return [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
B.ra_allreduce_ex(bufs(8, 512), algo="ring_step")                # tiny: one workgroup
B.ra_allreduce_ex(bufs(8, 1 << 20), algo="ring_step")            # large: a launch per step
B.ra_allreduce_ex(bufs(8, 1 << 20), algo="tree")
B.ra_allreduce_ex(bufs(8, 1 << 20), algo="ring_step", grid=16)   # caller's grid: persistent
B.ra_allreduce_ex(bufs(8, 1 << 20), algo="ring_channels", channels=8)
B.ra_allreduce_ex(bufs(8, 1 << 20), algo="ring_pipelined")       # one launch, a slice per workgroup
B.ra_allreduce_ex(bufs(8, 3 << 20), algo="ring_channels")        # 6 MiB per rank: 512 threads
B.ra_allreduce_ex(bufs(8, 10 << 20), algo="ring_channels")       # 20 MiB per rank: 1024 threads
B.ra_stream_status()
torch.cuda.synchronize()
"""


def test_step_launch_choices():
    require_gpu()
    env = dict(os.environ, RA_DEBUG="1")
    print("[case] child process with RA_DEBUG=1", flush=True)
    res = subprocess.run([sys.executable, "-c", CHILD, ROOT], env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    lines = [ln for ln in res.stderr.splitlines() if ln.startswith("[ra] allreduce")]
    got = []
    for ln in lines:
        m = re.search(r"algo=(\w+) p=(\d+) n=(\d+) dtype=\d+ grid=(\d+) launches=(\d+)", ln)
        assert m, ln
        got.append((m.group(1), int(m.group(3)), int(m.group(4)), int(m.group(5))))
    assert len(got) == 8, lines
    (a0, n0, g0, l0), (a1, n1, g1, l1), (a2, n2, g2, l2), (a3, n3, g3, l3), (a4, n4, g4, l4) = got[:5]
    assert (a0, g0, l0) == ("ring_step", 1, 1)
    assert (a1, l1) == ("ring_step", 14) and g1 > 1
    assert (a2, l2) == ("tree", 6) and g2 > 1
    assert (a3, g3, l3) == ("ring_step", 16, 1)
    assert a4 == "ring_channels" and l4 == 1 and g4 % 8 == 0
    # 2^20 bf16 per rank: 8 chunks of 16384 vectors, 64 tiles of 256 each
    assert got[5] == ("ring_pipelined", 1 << 20, 8 * 64, 1)
    # 3 Mi bf16 per rank: chunks of 49,152 vectors, 24 tiles of 512 x 4 each, 8 chunks
    assert got[6] == ("ring_channels", 3 << 20, 8 * 24, 1)
    # 10 Mi bf16 per rank: 40 tiles of 1024 x 4 per chunk, one workgroup per compute unit
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert got[7] == ("ring_channels", 10 << 20, min(cus, 8 * 40), 1)


PHASE_CHILD = r"""
import sys, torch
sys.path.insert(0, sys.argv[1])
from ring_all_reduce_schedule_amd import binding as B
def bufs(p, n):
    return [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(p)]
big = bufs(8, 6 << 30)              # 12 GiB per rank: the smallest the phases are picked for
B.ra_allreduce_ex(big, algo="fused")                                   # phases
B.ra_allreduce_ex(big, algo="fused", flags=B.RA_FLAG_NO_PHASES)        # one-shot
B.ra_allreduce_ex(big, algo="fused", op="avg")                         # averages: one-shot
B.ra_all_gather_ex(big, algo="fused")                                  # phases
B.ra_reduce_scatter_ex(big, algo="fused")                              # one-shot
B.ra_allreduce_ex(big[:7], algo="fused")                               # 7 ranks: one-shot
del big
small = bufs(8, 1 << 23)            # 128 MiB in all: cached, 4096 tiles
B.ra_allreduce_ex(small, algo="fused")                                 # one-shot
B.ra_allreduce_ex(small, algo="fused", flags=B.RA_FLAG_PHASES)         # forced
B.ra_stream_status()
torch.cuda.synchronize()
"""


def test_fused_phase_choices():
    """The one-pass calls that run in read/write phases show the phased grid,
    8 workgroups per compute unit; the others one workgroup per tile."""
    require_gpu()
    env = dict(os.environ, RA_DEBUG="1")
    print("[case] child process with RA_DEBUG=1 (phase choices)", flush=True)
    res = subprocess.run([sys.executable, "-c", PHASE_CHILD, ROOT], env=env, capture_output=True,
                         text=True, timeout=300)
    assert res.returncode == 0, res.stderr[-2000:]
    got = []
    for ln in res.stderr.splitlines():
        m = re.match(r"\[ra\] (\w+) algo=(\w+) p=(\d+) n=(\d+) dtype=\d+ grid=(\d+)", ln)
        if m:
            got.append((m.group(1), int(m.group(3)), int(m.group(5))))
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    phased = 8 * cus
    tiles = 8 * ((6 << 30) // 8 // 8 // 256)
    assert got[0] == ("allreduce", 8, phased)
    assert got[1] == ("allreduce", 8, tiles)
    assert got[2] == ("allreduce", 8, tiles)
    assert got[3] == ("all_gather", 8, phased)
    assert got[4] == ("reduce_scatter", 8, tiles)
    assert got[5][:2] == ("allreduce", 7) and got[5][2] > phased
    assert got[6] == ("allreduce", 8, 8 * ((1 << 23) // 8 // 8 // 256))
    assert got[7] == ("allreduce", 8, min(phased, 4096))
    assert len(got) == 8, got
