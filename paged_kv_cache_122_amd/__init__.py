"""PagedAttention decode for AMD MI355X (gfx950).

The compute path is ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``).  This package holds its Python binding
(argument marshalling only), the cache layout helpers, the host block manager
and prefix cache, and the seeded workload generator.
"""

from . import blockpool, layout, prefix_cache, sizing, workloads  # noqa: F401

__all__ = ["blockpool", "layout", "prefix_cache", "sizing", "workloads"]
