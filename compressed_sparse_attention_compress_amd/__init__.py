"""CSA2 (Compressed Sparse Attention 2) layer hot path for AMD MI355X (gfx950).

The compute lives in libcsa2.so (hand-written HIP kernels behind the C ABI in
include/csa2.h); ``csa2`` is its thin Python binding.
"""
from . import csa2  # noqa: F401

__all__ = ["csa2"]
