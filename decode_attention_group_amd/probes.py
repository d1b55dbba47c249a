"""Python binding of libkvq_probes.so (include/kvq_probes.h): the stream-read and
MFMA-loop probes that measure attainable ceilings on the GPU.  Argument
marshalling only; the caller times the launches with events."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libkvq_probes.so")
EXPORTS = ("kvq_probe_stream_read", "kvq_probe_segment_read", "kvq_probe_mfma_bf16", "kvq_probe_mfma_flops_per_iter")
_lib = None


def load_library(path: str = LIB_PATH):
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(path)
        P, i32 = ctypes.c_void_p, ctypes.c_int32
        lib.kvq_probe_stream_read.argtypes = [P, ctypes.c_size_t, i32, i32, P, P]
        lib.kvq_probe_stream_read.restype = ctypes.c_int
        lib.kvq_probe_segment_read.argtypes = [P, ctypes.c_size_t, i32, i32, P, P]
        lib.kvq_probe_segment_read.restype = ctypes.c_int
        lib.kvq_probe_mfma_bf16.argtypes = [i32, i32, i32, P, P]
        lib.kvq_probe_mfma_bf16.restype = ctypes.c_int
        lib.kvq_probe_mfma_flops_per_iter.argtypes = [i32, i32]
        lib.kvq_probe_mfma_flops_per_iter.restype = ctypes.c_double
        _lib = lib
    return _lib


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def stream_read(src: torch.Tensor, blocks: int, nontemporal: bool, sink: torch.Tensor):
    nbytes = src.numel() * src.element_size()
    st = load_library().kvq_probe_stream_read(src.data_ptr(), nbytes, blocks, int(nontemporal),
                                              sink.data_ptr(), _stream())
    if st:
        raise RuntimeError(f"kvq_probe_stream_read: status {st}")


def segment_read(src: torch.Tensor, segment_bytes: int, blocks: int, nontemporal: bool, sink: torch.Tensor):
    if blocks * segment_bytes > src.numel() * src.element_size():
        raise ValueError("segments past the buffer")
    st = load_library().kvq_probe_segment_read(src.data_ptr(), segment_bytes, blocks, int(nontemporal),
                                               sink.data_ptr(), _stream())
    if st:
        raise RuntimeError(f"kvq_probe_segment_read: status {st}")


def mfma_bf16(shape: int, iters: int, blocks: int, sink: torch.Tensor) -> float:
    """Launch the MFMA loop; returns the FLOPs it performs."""
    lib = load_library()
    st = lib.kvq_probe_mfma_bf16(shape, iters, blocks, sink.data_ptr(), _stream())
    if st:
        raise RuntimeError(f"kvq_probe_mfma_bf16: status {st}")
    return lib.kvq_probe_mfma_flops_per_iter(shape, blocks) * iters
