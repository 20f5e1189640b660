"""CPU oracle for the CSA2 decode path (float64 NumPy).

TEST INFRASTRUCTURE ONLY: only tests/, the smoke check and the benchmark's
CPU-baseline leg may import it.  It shares no code with the GPU library
(`fp4_kv_cache_amd`) and never imports it.
"""
from . import formats, csa2, accounting  # noqa: F401
