"""ctypes binding of libsaga_probe.so (include/saga_probe.h): the HBM
measurement kernels that calibrate the decode library's roofline.  Argument
marshalling only; the kernels are in ``hbm_probe.hip``."""
from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                        "libsaga_probe.so")
EXPORTED_SYMBOLS = ("saga_probe_read", "saga_probe_read_tiles", "saga_probe_rows")

_lib = None


def library():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run "
                               "`python -m sparse_decode_attention_atop_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        vp, sz, i32, i64, u32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32,
                                 ctypes.c_int64, ctypes.c_uint32)
        lib.saga_probe_read.argtypes = [vp, sz, i32, i32, vp, vp]
        lib.saga_probe_read.restype = ctypes.c_int
        lib.saga_probe_read_tiles.argtypes = [vp, sz, i32, i32, i32, vp, vp]
        lib.saga_probe_read_tiles.restype = ctypes.c_int
        lib.saga_probe_rows.argtypes = [vp, sz, i32, i64, u32, i32, i32, vp, vp]
        lib.saga_probe_rows.restype = ctypes.c_int
        _lib = lib
    return _lib


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def probe_read(buf: torch.Tensor, nbytes: int, workgroups: int, depth: int,
               sink: torch.Tensor) -> None:
    """Sequential read of the first nbytes of buf (uint8 device tensor)."""
    assert buf.is_cuda and buf.dtype == torch.uint8 and buf.numel() >= nbytes
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= workgroups
    st = library().saga_probe_read(ctypes.c_void_p(buf.data_ptr()), nbytes, workgroups, depth,
                                   ctypes.c_void_p(sink.data_ptr()), _stream())
    if st != 0:
        raise RuntimeError(f"saga_probe_read: status {st}")


def probe_read_tiles(buf: torch.Tensor, nbytes: int, row_bytes: int, workgroups: int,
                     tiles: int, sink: torch.Tensor) -> None:
    """Sequential read of the first nbytes of buf in the K stream's lane mapping."""
    assert buf.is_cuda and buf.dtype == torch.uint8 and buf.numel() >= nbytes
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= workgroups
    st = library().saga_probe_read_tiles(ctypes.c_void_p(buf.data_ptr()), nbytes, row_bytes,
                                         workgroups, tiles, ctypes.c_void_p(sink.data_ptr()),
                                         _stream())
    if st != 0:
        raise RuntimeError(f"saga_probe_read_tiles: status {st}")


def probe_rows(buf: torch.Tensor, row_bytes: int, rows: int, seed: int, workgroups: int,
               depth: int, sink: torch.Tensor) -> None:
    """Read `rows` pseudo-random rows of row_bytes bytes from buf."""
    assert buf.is_cuda and buf.dtype == torch.uint8
    assert sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= workgroups
    st = library().saga_probe_rows(ctypes.c_void_p(buf.data_ptr()), buf.numel(), row_bytes, rows,
                                   seed & 0xFFFFFFFF, workgroups, depth,
                                   ctypes.c_void_p(sink.data_ptr()), _stream())
    if st != 0:
        raise RuntimeError(f"saga_probe_rows: status {st}")
