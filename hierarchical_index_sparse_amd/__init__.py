"""Hierarchical block-then-token sparse attention for AMD MI355X (gfx950).

The compute path is libhsa_sparse.so (hand-written HIP kernels behind a
C ABI, see include/hsa_sparse.h); ``_lib`` is its ctypes binding and
``pipeline`` chains the entry points.  ``datagen`` and ``workloads`` make
the seeded synthetic inputs.
"""
from .workloads import WORKLOADS, Workload  # noqa: F401
