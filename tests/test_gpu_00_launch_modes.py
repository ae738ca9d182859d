"""Which launches the step algorithms choose (through the C ABI, RA_DEBUG=1).

With RA_DEBUG=1 the library prints one line per call with the grid and the
number of kernel launches.  A child process runs a few calls and the test checks
the documented choices:

* steps that move at most 256 vectors: one launch of one workgroup;
* larger steps: one launch per step (2(p-1) for the ring, 2*ceil(log2 p) for
  the tree);
* a caller's grid, or channels: one persistent launch of that many workgroups;
* the slice-carrying pipelined ring: one launch, one workgroup per 4 KiB slice
  of every chunk.

Every launch is an ordinary one (persistent grids are sized to stay resident,
not launched cooperatively), so the child can run while the test process holds
the GPU too.
"""

import os
import re
import subprocess
import sys

import pytest

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
    assert len(got) == 6, lines
    (a0, n0, g0, l0), (a1, n1, g1, l1), (a2, n2, g2, l2), (a3, n3, g3, l3), (a4, n4, g4, l4) = got[:5]
    assert (a0, g0, l0) == ("ring_step", 1, 1)
    assert (a1, l1) == ("ring_step", 14) and g1 > 1
    assert (a2, l2) == ("tree", 6) and g2 > 1
    assert (a3, g3, l3) == ("ring_step", 16, 1)
    assert a4 == "ring_channels" and l4 == 1 and g4 % 8 == 0
    # 2^20 bf16 per rank: 8 chunks of 16384 vectors, 64 tiles of 256 each
    assert got[5] == ("ring_pipelined", 1 << 20, 8 * 64, 1)
