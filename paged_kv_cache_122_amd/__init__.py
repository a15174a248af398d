"""PagedAttention decode for AMD MI355X (gfx950).

The compute path is ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``).  This package holds its Python binding
(argument marshalling only), the cache layout helpers, the host block manager
and the seeded workload generator.
"""

from . import blockpool, layout, sizing, workloads  # noqa: F401

__all__ = ["blockpool", "layout", "sizing", "workloads"]
