"""CPU oracle for the ring all-reduce chunk schedule (TEST INFRASTRUCTURE ONLY).

This package is a plain, slow, obviously-correct restatement of what the ring
all-reduce computes, written with numpy from the pages' descriptions.  It is the
parity reference for the HIP path and nothing else: only the test-suite, the
smoke check in ``__graft_entry__.py`` and the CPU-baseline leg of ``bench.py``
may import it.  The
product path (the C-ABI library and its Python binding) never imports, links or
calls anything in here, and this package imports nothing from the product.

Sources, cited by page title and section throughout:

* [InDepth]   "Ring All-Reduce, in depth: the chunk schedule step by step, a
              working implementation, pipelining, multi-ring and hierarchical
              variants" (aicassindra.com) -- sections "The schedule", "Tracing
              four GPUs", "An implementation", "What real libraries add",
              "Failure modes".
* [Derive]    "Derive the cost of a ring all-reduce" (aiinfrainterviews.com) --
              "TL;DR", "A strong answer", "Where it stops scaling", "What
              interviewers probe next".
* [Deepinsea] "AllReduce 与 Ring 通信算法详解" (deepinsea.top) -- "AllReduce 语义",
              "Phase 1: Reduce-Scatter", "Phase 2: All-Gather", "通信量分析".
* [Fable]     "Ring All-Reduce" fable of the Jade Ring Pond (fables.day) --
              "What it is", "Metaphor mapping".

Element storage: int32 / int64 / float16 / float32 / float64 -> the numpy type
of that name, bfloat16 -> numpy uint16 holding the bf16 bit pattern.

Modules
  schedule  chunk partition and the send/receive index rules
  arith     per-hop addition rounded to the buffer's element type
  ring      lock-step simulator of reduce-scatter / all-gather (both directions)
  fold      closed form of the ring's accumulation order, per element
  tree      binomial-tree all-reduce (reduce up, broadcast down)
  bidir     two counter-rotating rings on the two halves of the buffer
  hier      two-level ring: reduce-scatter in a node, all-reduce across nodes, all-gather
  exact     float64 reference sum and the normwise error measure
  cost      step / traffic counts and the latency-bandwidth cost model

Every function here has a pin in ``tests/test_oracle_*.py`` that checks it
against something other than itself (printed values, closed forms, library
routines, brute force); none is "parity unpinned".
"""

from .schedule import (chunk_bounds, chunk_of, rs_send_chunk, ag_send_chunk,
                       owned_chunk, right_of, left_of)
from .arith import (DTYPES, STORAGE, add_rounded, bf16_bits_to_f32,
                    f32_to_bf16_bits, as_values)
from .ring import (RingTimeout, reduce_scatter, all_gather, ring_allreduce)
from .fold import ring_fold, ring_fold_window, rs_partial, rs_owned
from .tree import tree_allreduce
from .bidir import bidir_allreduce, bidir_halves, bidir_fold_window
from .hier import hier_allreduce, hier_fold, hier_fold_window, hier_layout
from .exact import exact_sum, normwise_error
from . import cost

__all__ = [
    "chunk_bounds", "chunk_of", "rs_send_chunk", "ag_send_chunk", "owned_chunk",
    "right_of", "left_of", "DTYPES", "STORAGE", "add_rounded",
    "bf16_bits_to_f32", "f32_to_bf16_bits", "as_values", "RingTimeout",
    "reduce_scatter", "all_gather", "ring_allreduce", "ring_fold",
    "ring_fold_window", "rs_partial", "rs_owned", "tree_allreduce", "bidir_allreduce",
    "bidir_halves", "bidir_fold_window", "hier_allreduce", "hier_fold", "hier_fold_window", "hier_layout", "exact_sum", "normwise_error", "cost",
]
