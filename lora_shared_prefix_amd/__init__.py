"""ResidualAttention over a copy-on-write forked, disaggregated paged KV cache, for MI355X.

The work runs in ``libforkkv.so`` (C ABI declared in ``include/forkkv.h``; HIP kernels for
gfx950).  ``forkkv`` is the ctypes binding; ``session`` uploads a workload and drives the
library from PyTorch device memory and streams.
"""
from . import forkkv  # noqa: F401
