"""ctypes binding of libpaprobe.so (include/pa_probe.h): the bench's plain
read and copy kernels.  Argument marshalling only; raises if the library is
missing or a call fails."""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpaprobe.so")
HEADER = os.path.join(os.path.dirname(_HERE), "include", "pa_probe.h")

_lib = None


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"HIP library not built: {LIB_PATH} (run __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.pa_probe_read.argtypes = [P, ctypes.c_int64, P, P]
    lib.pa_probe_read.restype = ctypes.c_int
    lib.pa_probe_copy.argtypes = [P, P, ctypes.c_int64, P]
    lib.pa_probe_copy.restype = ctypes.c_int
    _lib = lib
    return lib


def _stream(stream):
    return ctypes.c_void_p((stream or torch.cuda.current_stream()).cuda_stream)


def read(buf: torch.Tensor, sink: torch.Tensor, stream=None) -> None:
    """Stream buf once (all its bytes) with the read probe kernel."""
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("sink must hold at least 1 KiB")
    rc = load().pa_probe_read(ctypes.c_void_p(buf.data_ptr()), buf.numel() * buf.element_size(),
                              ctypes.c_void_p(sink.data_ptr()), _stream(stream))
    if rc != 0:
        raise RuntimeError(f"pa_probe_read failed ({rc})")


def copy(src: torch.Tensor, dst: torch.Tensor, stream=None) -> None:
    """dst[:] = src[:] (same byte size) with the copy probe kernel."""
    n = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != n:
        raise ValueError("src and dst sizes differ")
    rc = load().pa_probe_copy(ctypes.c_void_p(src.data_ptr()), ctypes.c_void_p(dst.data_ptr()), n,
                              _stream(stream))
    if rc != 0:
        raise RuntimeError(f"pa_probe_copy failed ({rc})")
