"""Quest query-aware sparse decode attention over a paged KV cache, for AMD
Instinct MI355X (gfx950).

The compute lives in libquest.so (hand-written HIP kernels behind the C ABI in
include/quest.h); ``quest`` is its ctypes binding and ``workloads`` draws the
seeded synthetic inputs.
"""
from . import quest, workloads  # noqa: F401

__all__ = ["quest", "workloads"]
