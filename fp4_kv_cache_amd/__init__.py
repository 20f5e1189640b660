"""libcsa2 for AMD MI355X: decode-time Compressed Sparse Attention 2 with an
FP4 main-KV cache.  The compute path is the HIP library `libcsa2.so`
(C ABI in include/csa2.h); `csa2` is its thin ctypes binding.
"""
from . import csa2  # noqa: F401

__all__ = ["csa2"]
