"""Decode attention over a prefix-shared KV tree (ChunkAttention's two-phase
partition) for AMD Instinct MI355X (gfx950).

The compute path lives in ``libpkvt.so`` (C++ prefix tree and planner, HIP
kernels) behind the C ABI declared in ``include/pkvt.h``.  ``binding`` is a
thin ctypes layer with the same function names; ``workloads`` draws the
seeded synthetic inputs.  Importing this package loads nothing; the library
is loaded on first use of ``binding``.
"""
__all__ = ["binding", "workloads"]
