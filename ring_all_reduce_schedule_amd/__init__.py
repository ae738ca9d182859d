"""Ring all-reduce chunk schedule on one MI355X (gfx950): p virtual ranks in HBM.

The compute path is the C-ABI library ``libra.so`` (hand-written HIP kernels);
``binding`` is a thin ctypes layer over it with the same function names.
``inputs`` draws the seeded synthetic workloads.  Importing this package does
not load the library; the first call into ``binding`` does, and raises if the
library has not been built.
"""

__all__ = ["binding", "inputs"]
