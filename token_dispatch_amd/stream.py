"""Python binding of libmoonep_stream.so: plain sequential read, write and copy
kernels that measure the practical HBM ceilings the data moves are compared with
(include/moonep_stream.h). Argument marshalling only; tensors are torch device
tensors, the stream is the tensors' current stream unless given."""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoonep_stream.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build the HIP libraries first")

_lib = ctypes.CDLL(LIB_PATH)
_vp, _i64, _u32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32
_lib.moonep_stream_read.argtypes = [_vp, _i64, _i64, _vp, _vp]
_lib.moonep_stream_write.argtypes = [_vp, _i64, _i64, _u32, _vp]
_lib.moonep_stream_copy.argtypes = [_vp, _vp, _i64, _i64, _vp]
for _n in ("moonep_stream_read", "moonep_stream_write", "moonep_stream_copy"):
    getattr(_lib, _n).restype = ctypes.c_int

ENTRY_POINTS = ("moonep_stream_read", "moonep_stream_write", "moonep_stream_copy")


def _stream(t, stream):
    import torch
    return (stream if stream is not None else torch.cuda.current_stream(t.device)).cuda_stream


def _nbytes(t) -> int:
    if not t.is_contiguous() or t.device.type != "cuda":
        raise ValueError("a contiguous GPU tensor is needed")
    return t.numel() * t.element_size()


def _check(rc, where):
    if rc != 0:
        raise RuntimeError(f"{where} failed (rc={rc})")


def stream_read(src, sink, chunk_bytes: int = 0, stream=None) -> None:
    """Read every byte of src once (sink: a 16-byte device tensor). chunk_bytes: 0
    for one resident grid, else one workgroup per chunk of that many bytes."""
    _check(_lib.moonep_stream_read(src.data_ptr(), _nbytes(src), chunk_bytes, sink.data_ptr(),
                                   _stream(src, stream)), "moonep_stream_read")


def stream_write(dst, pattern: int = 0, chunk_bytes: int = 0, stream=None) -> None:
    _check(_lib.moonep_stream_write(dst.data_ptr(), _nbytes(dst), chunk_bytes,
                                    pattern & 0xffffffff, _stream(dst, stream)),
           "moonep_stream_write")


def stream_copy(dst, src, chunk_bytes: int = 0, stream=None) -> None:
    n = _nbytes(src)
    if _nbytes(dst) < n:
        raise ValueError("dst is smaller than src")
    _check(_lib.moonep_stream_copy(dst.data_ptr(), src.data_ptr(), n, chunk_bytes,
                                   _stream(src, stream)), "moonep_stream_copy")
