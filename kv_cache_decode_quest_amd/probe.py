"""ctypes binding of libquest_probe.so (include/quest_probe.h): HBM read
probes for the benchmark, which times what plain reads of the Quest step's
two access patterns (a contiguous scan, scattered page chunks) achieve on the
GPU.  Argument marshalling only; raises if the library is missing or a call
fails."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libquest_probe.so")
EXPORTS = ("quest_probe_stream_read", "quest_probe_gather_read")
NEVER = 0x9E3779B9            # sink value no probe input produces in practice

_lib = None


def load(path: str = LIB_PATH):
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run __graft_entry__.build()")
    L = ctypes.CDLL(path)
    vp, i32, sz, u32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_uint32
    L.quest_probe_stream_read.argtypes = [vp, sz, i32, u32, vp, vp]
    L.quest_probe_gather_read.argtypes = [vp, vp, vp, i32, i32, i32, u32, vp, vp]
    for name in EXPORTS:
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def stream_read(buf: torch.Tensor, sink: torch.Tensor, work_groups: int = 0):
    """Read all of `buf` once, contiguously.  work_groups = 0: one 16-byte
    load per thread (the fastest shape measured on an MI355X: 131 MB in
    21.2 us, against 25.8 us with 4096 work-groups of 8 loads per thread)."""
    nbytes = buf.numel() * buf.element_size()
    if work_groups <= 0:
        work_groups = max(1, min((nbytes // 16 + 255) // 256, 1 << 20))
    st = load().quest_probe_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, work_groups,
                                        NEVER, ctypes.c_void_p(sink.data_ptr()), _stream(buf))
    if st != 0:
        raise RuntimeError(f"quest_probe_stream_read failed: {st}")


def gather_read(a: torch.Tensor, b: torch.Tensor, offsets16: torch.Tensor, chunk_bytes: int,
                sink: torch.Tensor, work_groups: int = 2048):
    """Read chunk pairs of chunk_bytes at 16-byte element offsets
    offsets16 (int64, device) of a and of b."""
    if offsets16.dtype != torch.int64 or not offsets16.is_contiguous():
        raise TypeError("offsets16: contiguous int64 expected")
    st = load().quest_probe_gather_read(ctypes.c_void_p(a.data_ptr()),
                                        ctypes.c_void_p(b.data_ptr()),
                                        ctypes.c_void_p(offsets16.data_ptr()),
                                        int(offsets16.numel()), int(chunk_bytes), work_groups,
                                        NEVER, ctypes.c_void_p(sink.data_ptr()), _stream(a))
    if st != 0:
        raise RuntimeError(f"quest_probe_gather_read failed: {st}")
