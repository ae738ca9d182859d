"""Lock-step simulator of the ring all-reduce (oracle; test infrastructure only).

Follows [InDepth] "The schedule" and the simulator idea of [InDepth] "An
implementation": every step first collects all of its messages from the state
the ranks hold *before* the step (each message carries a copy of the chunk), and
only then delivers them, so all sends of a step happen at once.  Delivery adds
into the receiver's chunk during the reduce-scatter and overwrites it during the
all-gather ([InDepth] "The schedule"; [Deepinsea] "Phase 1: Reduce-Scatter",
"Phase 2: All-Gather").  Unlike the page's simulator, which widens everything to
float64, each hop here rounds to the buffer's element type (see ``arith``); the
float64 sum is kept separately as ``exact.exact_sum``.

Besides the buffers the simulator returns what the tests pin against the pages:
the number of elements each rank sent ([InDepth] "The schedule"; [Derive] "A
strong answer"), the element reads and writes the schedule implies for buffers
that live in one memory (a receive-add reads the incoming chunk and the
receiver's chunk and writes the receiver's chunk; a receive-copy reads one chunk
and writes one), and the chunk indices sent at every step.

Reductions other than the sum ([Deepinsea] "AllReduce 语义"): "max" delivers
with the exact maximum instead of the add; "avg" divides every rank's buffer by
p before the first step ([InDepth] "Failure modes": pre-divide), then sums.

Failure: [InDepth] "Failure modes" -- a dead rank never sends, its right
neighbour waits for a message that does not come, and the job should fail fast
on a timeout instead of hanging.  ``dead_rank=k`` models that: rank k's messages
are never delivered and the receiver gives up after ``max_polls`` empty polls of
its inbox by raising ``RingTimeout``.
"""

import numpy as np

from .arith import combine, pre_divide
from .schedule import (chunk_bounds, rs_send_chunk, ag_send_chunk, right_of,
                       left_of)


class RingTimeout(RuntimeError):
    """A receive found no message within its poll budget."""

    def __init__(self, rank, phase, step):
        super().__init__(f"rank {rank} timed out waiting in {phase} step {step}")
        self.rank, self.phase, self.step = rank, phase, step


class Trace:
    """What happened during a run of the simulator."""

    def __init__(self, p, keep_states=False):
        self.keep_states = keep_states
        self.states = []              # copies of all buffers after every step
        self.sent = [0] * p           # elements sent, per rank
        self.reads = 0                # element reads, all ranks
        self.writes = 0               # element writes, all ranks
        self.rs_table = []            # rs_table[s][r] = chunk rank r sent at RS step s
        self.ag_table = []            # ag_table[s][r] = chunk rank r sent at AG step s
        self.steps = 0


def _deliver(inbox, rank, phase, step, max_polls):
    """Poll ``inbox`` for the message addressed to ``rank``; time out if absent."""
    for _ in range(max_polls):
        if rank in inbox:
            return inbox.pop(rank)
    raise RingTimeout(rank, phase, step)


def _phase(bufs, dtype, direction, phase, trace, dead_rank, max_polls, op="sum"):
    p = len(bufs)
    n = len(bufs[0])
    bounds = chunk_bounds(n, p)
    pick = rs_send_chunk if phase == "reduce-scatter" else ag_send_chunk
    table = trace.rs_table if phase == "reduce-scatter" else trace.ag_table
    for s in range(p - 1):
        # 1. every rank reads the chunk it sends from the pre-step state
        inbox = {}
        sent_chunks = []
        for r in range(p):
            c = pick(r, s, p, direction)
            lo, hi = bounds[c]
            sent_chunks.append(c)
            if r == dead_rank:
                continue
            inbox[right_of(r, p, direction)] = (c, bufs[r][lo:hi].copy())
            trace.sent[r] += hi - lo
        table.append(sent_chunks)
        # a rank never writes the chunk it is sending in the same step, so the
        # in-place update below cannot clobber a message before it is read
        for r in range(p):
            incoming = sent_chunks[left_of(r, p, direction)]
            assert incoming != sent_chunks[r], "read/write overlap inside a step"
        # 2. every receiver applies what arrived
        for dst in range(p):
            c, data = _deliver(inbox, dst, phase, s, max_polls)
            lo, hi = bounds[c]
            if phase == "reduce-scatter":
                bufs[dst][lo:hi] = combine(bufs[dst][lo:hi], data, dtype, op)
                trace.reads += 2 * (hi - lo)
            else:
                bufs[dst][lo:hi] = data
                trace.reads += hi - lo
            trace.writes += hi - lo
        trace.steps += 1
        if trace.keep_states:
            trace.states.append([b.copy() for b in bufs])
    return bufs


def reduce_scatter(bufs, dtype, direction=1, dead_rank=None, max_polls=3,
                   trace=None, op="sum"):
    """Run the p - 1 reduce-scatter steps in place on copies of ``bufs``.

    Returns (buffers, trace).  Afterwards rank r holds the full sum of chunk
    ``owned_chunk(r, p, direction)``; its other chunks hold ring partial sums.
    With op "avg" the buffers are divided by p first.
    """
    p = len(bufs)
    bufs = [np.array(b, copy=True) for b in bufs]
    if op == "avg":
        bufs = [pre_divide(b, dtype, p) for b in bufs]
    trace = trace or Trace(p)
    _phase(bufs, dtype, direction, "reduce-scatter", trace, dead_rank, max_polls, op)
    return bufs, trace


def all_gather(bufs, dtype, direction=1, dead_rank=None, max_polls=3,
               trace=None):
    """Run the p - 1 all-gather steps: owned chunks are copied round the ring."""
    bufs = [np.array(b, copy=True) for b in bufs]
    trace = trace or Trace(len(bufs))
    _phase(bufs, dtype, direction, "all-gather", trace, dead_rank, max_polls)
    return bufs, trace


def ring_allreduce(bufs, dtype, direction=1, dead_rank=None, max_polls=3,
                   keep_states=False, op="sum"):
    """Reduce-scatter then all-gather.

    Returns (final buffers, buffers after the reduce-scatter, trace); with
    ``keep_states`` the trace also holds every rank's buffer after each step.  With one
    rank there is nothing to send and the buffer is returned unchanged
    ([InDepth] "An implementation": a world of one is a no-op).
    """
    trace = Trace(len(bufs), keep_states)
    after_rs, _ = reduce_scatter(bufs, dtype, direction, dead_rank, max_polls,
                                 trace, op)
    final, _ = all_gather(after_rs, dtype, direction, dead_rank, max_polls,
                          trace)
    return final, after_rs, trace
