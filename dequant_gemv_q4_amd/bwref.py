"""ctypes front of libqgbw.so, the benchmark's bandwidth reference (a plain 16-byte-load read
kernel in grid-stride or contiguous-chunk order, bw_read.hip).  Not part of the GEMV library: bench.py times it beside the GEMV kernels to
state how much of the attainable HBM read rate they reach."""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libqgbw.so")
_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libqgbw.so not built ({LIB_PATH}); run "
                               "`python -m dequant_gemv_q4_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        L.qgbw_read.restype = ctypes.c_int
        L.qgbw_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int,
                                ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
        _lib = L
    return _lib


def read(buf, nbytes: int, out, grid: int, threads: int, chunked: bool = False, stream=None):
    """Read nbytes of the device tensor buf, in grid-stride order or (chunked) one contiguous
    chunk per workgroup; out (a device tensor) takes grid * threads / 64 words."""
    import torch
    if out.numel() * out.element_size() < grid * threads // 64 * 4:
        raise ValueError("out too small for this launch shape")
    if buf.numel() * buf.element_size() < nbytes:
        raise ValueError("buffer smaller than the requested read")
    s = stream if stream is not None else torch.cuda.current_stream().cuda_stream
    rc = lib().qgbw_read(buf.data_ptr(), nbytes, out.data_ptr(), grid, threads, int(chunked), s)
    if rc != 0:
        raise RuntimeError(f"qgbw_read failed: hip error {rc}")
