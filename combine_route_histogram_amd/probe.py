"""Binding of libmdc_probe.so: the memory-ceiling probes (include/mdc_probe.h).

The probes compute nothing of the method; the benchmark times them beside the
dispatch and combine kernels, on the same stream, to measure what the same
bytes cost in the plainest kernel of each access pattern.  Loading fails
loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (binds the probe library to torch's HIP runtime, as for libmdc)

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmdc_probe.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"libmdc_probe.so not found at {LIB_PATH}; build it with "
                      "`python combine_route_histogram_amd/build.py`")
_lib = ctypes.CDLL(LIB_PATH)

EXPORTS = ("mdc_probe_read", "mdc_probe_write", "mdc_probe_copy", "mdc_probe_rows_read", "mdc_probe_rows_write",
           "mdc_probe_rows_fanout", "mdc_probe_rows_reduce")

_P, _U64, _I32, _U32 = ctypes.c_void_p, ctypes.c_uint64, ctypes.c_int32, ctypes.c_uint32
_lib.mdc_probe_read.argtypes = [_P, _U64, _P, _P]
_lib.mdc_probe_write.argtypes = [_P, _U64, _U32, _P]
_lib.mdc_probe_copy.argtypes = [_P, _P, _U64, _P]
_lib.mdc_probe_rows_read.argtypes = [_P, _P, _I32, _I32, _P, _P]
_lib.mdc_probe_rows_write.argtypes = [_P, _P, _P, _I32, _I32, _P]
_lib.mdc_probe_rows_fanout.argtypes = [_P, _P, _P, _P, _P, _I32, _I32, _P]
_lib.mdc_probe_rows_reduce.argtypes = [_P, _P, _I32, _P, _P, _I32, _I32, _P]
for _n in EXPORTS:
    getattr(_lib, _n).restype = ctypes.c_int


def _ok(st: int, name: str) -> None:
    if st != 0:
        raise RuntimeError(f"{name} returned {st}")


def _bytes(t) -> int:
    return t.numel() * t.element_size()


def read(src, nbytes: int, sink, stream) -> None:
    assert nbytes <= _bytes(src) and _bytes(sink) >= 4096
    _ok(_lib.mdc_probe_read(src.data_ptr(), nbytes, sink.data_ptr(), stream), "mdc_probe_read")


def write(dst, nbytes: int, value: int, stream) -> None:
    assert nbytes <= _bytes(dst)
    _ok(_lib.mdc_probe_write(dst.data_ptr(), nbytes, value, stream), "mdc_probe_write")


def copy(src, dst, nbytes: int, stream) -> None:
    assert nbytes <= min(_bytes(src), _bytes(dst))
    _ok(_lib.mdc_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes, stream), "mdc_probe_copy")


def rows_read(src, rows, row_bytes: int, sink, stream) -> None:
    """rows: int32 device tensor of row indices into src."""
    assert rows.dtype == torch.int32 and _bytes(sink) >= 4096
    _ok(_lib.mdc_probe_rows_read(src.data_ptr(), rows.data_ptr(), rows.numel(), row_bytes, sink.data_ptr(), stream),
        "mdc_probe_rows_read")


def rows_write(dst, offsets, rows, row_bytes: int, stream) -> None:
    """offsets: int32 [n_src + 1] into rows (int32 row indices of dst)."""
    assert offsets.dtype == torch.int32 and rows.dtype == torch.int32
    _ok(_lib.mdc_probe_rows_write(dst.data_ptr(), offsets.data_ptr(), rows.data_ptr(), offsets.numel() - 1,
                                  row_bytes, stream), "mdc_probe_rows_write")


def rows_fanout(src, src_rows, offsets, dst_rows, dst, row_bytes: int, stream) -> None:
    """src_rows: int32 [n_src]; offsets: int32 [n_src + 1] into dst_rows (int32 row indices of dst)."""
    assert src_rows.dtype == offsets.dtype == dst_rows.dtype == torch.int32
    assert offsets.numel() == src_rows.numel() + 1
    _ok(_lib.mdc_probe_rows_fanout(src.data_ptr(), src_rows.data_ptr(), offsets.data_ptr(), dst_rows.data_ptr(),
                                   dst.data_ptr(), src_rows.numel(), row_bytes, stream), "mdc_probe_rows_fanout")


def rows_reduce(src, rows, k: int, own, dst, row_bytes: int, stream) -> None:
    """rows: int32 [n_out][k] row indices into src (negative = absent); own, dst: [n_out] rows."""
    assert rows.dtype == torch.int32 and rows.numel() % k == 0
    _ok(_lib.mdc_probe_rows_reduce(src.data_ptr(), rows.data_ptr(), k, own.data_ptr(), dst.data_ptr(),
                                   rows.numel() // k, row_bytes, stream), "mdc_probe_rows_reduce")
