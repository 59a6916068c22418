"""Python binding of libmdc (MoE dispatch/combine for MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmdc.so, declared in include/mdc.h.  torch tensors are passed as device
pointers; torch provides device memory and streams.  The functions carry the
names of the C entry points.  Importing this package fails loudly when
libmdc.so has not been built (python combine_route_histogram_amd/build.py).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, replace
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmdc.so")

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"libmdc.so not found at {LIB_PATH}; build it with "
        "`python combine_route_histogram_amd/build.py` (hipcc, gfx950)")

# torch provides device memory and streams.  Its wheel carries its own HIP
# runtime (same SONAME, libamdhip64.so.7): loading torch first makes libmdc
# bind to that runtime, so torch's streams and pointers are valid in libmdc.
import torch  # noqa: E402,F401

_lib = ctypes.CDLL(LIB_PATH)

MDC_OK = 0
MDC_ERR_NULLPTR = 1
MDC_ERR_INVALID = 2
MDC_ERR_WORKSPACE = 3
MDC_ERR_HIP = 4
MDC_MAX_TOPK = 16
MDC_MAX_LOCAL_EXPERTS = 2048
MDC_MAX_COMBINE_WORLD = 64

EXPORTS = (
    "mdc_status_string", "mdc_abi_version",
    "mdc_dispatch_workspace_size", "mdc_dispatch_layout", "mdc_dispatch_gather", "mdc_dispatch",
    "mdc_combine_workspace_size", "mdc_combine",
    "mdc_ffn_workspace_size", "mdc_ffn", "mdc_dispatch_quant", "mdc_dispatch_quant_gather",
    "mdc_ffn_quant_input",
)


class mdc_shape(ctypes.Structure):
    _fields_ = [("world", ctypes.c_int32), ("rank", ctypes.c_int32), ("bs", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("mask_per_route", ctypes.c_int32),
                ("zero_experts", ctypes.c_int32), ("copy_experts", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SHP = ctypes.POINTER(mdc_shape)

_lib.mdc_status_string.restype = ctypes.c_char_p
_lib.mdc_status_string.argtypes = [ctypes.c_int]
_lib.mdc_abi_version.restype = ctypes.c_int32
_lib.mdc_abi_version.argtypes = []
_lib.mdc_dispatch_workspace_size.restype = ctypes.c_int
_lib.mdc_dispatch_workspace_size.argtypes = [_SHP, ctypes.POINTER(_SZ)]
_lib.mdc_dispatch_layout.restype = ctypes.c_int
_lib.mdc_dispatch_layout.argtypes = [_SHP, _P, _P, _P, _SZ, _P]
_lib.mdc_dispatch_gather.restype = ctypes.c_int
_lib.mdc_dispatch_gather.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.mdc_dispatch.restype = ctypes.c_int
_lib.mdc_dispatch.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.mdc_combine_workspace_size.restype = ctypes.c_int
_lib.mdc_combine_workspace_size.argtypes = [_SHP, ctypes.POINTER(_SZ)]
_lib.mdc_combine.restype = ctypes.c_int
_lib.mdc_combine.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.mdc_ffn_workspace_size.restype = ctypes.c_int
_lib.mdc_ffn_workspace_size.argtypes = [_SHP, ctypes.c_int32, ctypes.POINTER(_SZ)]
_lib.mdc_ffn.restype = ctypes.c_int
_lib.mdc_ffn.argtypes = [_SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.mdc_dispatch_quant.restype = ctypes.c_int
_lib.mdc_dispatch_quant.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.mdc_dispatch_quant_gather.restype = ctypes.c_int
_lib.mdc_dispatch_quant_gather.argtypes = [_SHP, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]
_lib.mdc_ffn_quant_input.restype = ctypes.c_int
_lib.mdc_ffn_quant_input.argtypes = [_SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P]


class MdcError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mdc_status_string(status)}")


def mdc_status_string(status: int) -> str:
    return _lib.mdc_status_string(int(status)).decode()


def mdc_abi_version() -> int:
    return int(_lib.mdc_abi_version())


@dataclass
class Shape:
    world: int
    rank: int
    bs: int
    hidden: int
    topk: int
    num_experts: int
    capacity: int
    mask_per_route: int = 0
    zero_experts: int = 0
    copy_experts: int = 0

    @property
    def local_experts(self) -> int:
        return self.num_experts // self.world

    def c(self) -> mdc_shape:
        return mdc_shape(self.world, self.rank, self.bs, self.hidden, self.topk, self.num_experts, self.capacity,
                         self.mask_per_route, self.zero_experts, self.copy_experts, 0)

    def with_rank(self, rank: int) -> "Shape":
        return replace(self, rank=rank)


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("mdc: tensors must be contiguous")
    return t.data_ptr()


def _nbytes(t) -> int:
    """Size in bytes of a tensor argument; a raw integer pointer carries no size (0)."""
    if t is None or isinstance(t, int):
        return 0
    return t.numel() * t.element_size()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != MDC_OK:
        raise MdcError(status, where)


def mdc_dispatch_workspace_size(shape: Shape) -> int:
    out = _SZ(0)
    sh = shape.c()
    _check(_lib.mdc_dispatch_workspace_size(ctypes.byref(sh), ctypes.byref(out)), "mdc_dispatch_workspace_size")
    return int(out.value)


def mdc_combine_workspace_size(shape: Shape) -> int:
    out = _SZ(0)
    sh = shape.c()
    _check(_lib.mdc_combine_workspace_size(ctypes.byref(sh), ctypes.byref(out)), "mdc_combine_workspace_size")
    return int(out.value)


def mdc_dispatch_layout(shape: Shape, expert_ids, x_active_mask, workspace, stream=None, check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_dispatch_layout(ctypes.byref(sh), _ptr(expert_ids), _ptr(x_active_mask), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream))
    if check:
        _check(st, "mdc_dispatch_layout")
    return st


def mdc_dispatch_gather(shape: Shape, x, expand_x, assist_info, ep_recv_counts, expert_token_nums,
                        expanded_row_idx, workspace, stream=None, check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_dispatch_gather(ctypes.byref(sh), _ptr(x), _ptr(expand_x), _ptr(assist_info),
                                  _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream))
    if check:
        _check(st, "mdc_dispatch_gather")
    return st


def mdc_dispatch(shape: Shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                 expert_token_nums, expanded_row_idx, workspace, stream=None, check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_dispatch(ctypes.byref(sh), _ptr(x), _ptr(expert_ids), _ptr(x_active_mask), _ptr(expand_x),
                           _ptr(assist_info), _ptr(ep_recv_counts), _ptr(expert_token_nums),
                           _ptr(expanded_row_idx), _ptr(workspace), _nbytes(workspace), _stream(stream))
    if check:
        _check(st, "mdc_dispatch")
    return st


def _table(items: Sequence) -> ctypes.Array:
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = _ptr(t)
    return arr


def mdc_combine(shape: Shape, expand_x: Sequence, assist_info: Sequence, ep_recv_counts: Sequence,
                expanded_row_idx, expert_ids, expert_scales, x_active_mask, shared_expert_x, x_out,
                workspace=None, stream=None, check: bool = True, ori_x=None) -> int:
    sh = shape.c()
    ty, ta, tc = _table(expand_x), _table(assist_info), _table(ep_recv_counts)
    st = _lib.mdc_combine(ctypes.byref(sh), ctypes.cast(ty, _P), ctypes.cast(ta, _P), ctypes.cast(tc, _P),
                          _ptr(expanded_row_idx), _ptr(expert_ids), _ptr(expert_scales), _ptr(x_active_mask),
                          _ptr(shared_expert_x), _ptr(ori_x), _ptr(x_out), _ptr(workspace), _nbytes(workspace),
                          _stream(stream))
    if check:
        _check(st, "mdc_combine")
    return st


def mdc_ffn_workspace_size(shape: Shape, inter_n: int) -> int:
    out = _SZ(0)
    sh = shape.c()
    _check(_lib.mdc_ffn_workspace_size(ctypes.byref(sh), int(inter_n), ctypes.byref(out)), "mdc_ffn_workspace_size")
    return int(out.value)


def mdc_ffn(shape: Shape, inter_n: int, expand_x, expert_token_nums, w1, w1_scale, w2, w2_scale, y, workspace,
            stream=None, check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_ffn(ctypes.byref(sh), int(inter_n), _ptr(expand_x), _ptr(expert_token_nums), _ptr(w1),
                      _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(workspace), _nbytes(workspace),
                      _stream(stream))
    if check:
        _check(st, "mdc_ffn")
    return st


def mdc_dispatch_quant(shape: Shape, x, expert_ids, x_active_mask, expand_q, dynamic_scales, assist_info,
                       ep_recv_counts, expert_token_nums, expanded_row_idx, workspace, stream=None,
                       check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_dispatch_quant(ctypes.byref(sh), _ptr(x), _ptr(expert_ids), _ptr(x_active_mask), _ptr(expand_q),
                                 _ptr(dynamic_scales), _ptr(assist_info), _ptr(ep_recv_counts),
                                 _ptr(expert_token_nums), _ptr(expanded_row_idx), _ptr(workspace),
                                 _nbytes(workspace), _stream(stream))
    if check:
        _check(st, "mdc_dispatch_quant")
    return st


def mdc_dispatch_quant_gather(shape: Shape, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                              expert_token_nums, expanded_row_idx, workspace, stream=None, check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_dispatch_quant_gather(ctypes.byref(sh), _ptr(x), _ptr(expand_q), _ptr(dynamic_scales),
                                        _ptr(assist_info), _ptr(ep_recv_counts), _ptr(expert_token_nums),
                                        _ptr(expanded_row_idx), _ptr(workspace), _nbytes(workspace), _stream(stream))
    if check:
        _check(st, "mdc_dispatch_quant_gather")
    return st


def prepare_dispatch_quant_gather(shape: Shape, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                                  expert_token_nums, expanded_row_idx, workspace, stream=None) -> "Prepared":
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expand_q), _ptr(dynamic_scales), _ptr(assist_info),
            _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_dispatch_quant_gather, args, "mdc_dispatch_quant_gather", (sh,))


def mdc_ffn_quant_input(shape: Shape, inter_n: int, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale, w2,
                        w2_scale, y, workspace, stream=None, check: bool = True) -> int:
    sh = shape.c()
    st = _lib.mdc_ffn_quant_input(ctypes.byref(sh), int(inter_n), _ptr(expand_q), _ptr(dynamic_scales),
                                  _ptr(expert_token_nums), _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale),
                                  _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream))
    if check:
        _check(st, "mdc_ffn_quant_input")
    return st


def prepare_ffn_quant_input(shape: Shape, inter_n: int, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale,
                            w2, w2_scale, y, workspace, stream=None) -> "Prepared":
    sh = shape.c()
    args = (ctypes.byref(sh), int(inter_n), _ptr(expand_q), _ptr(dynamic_scales), _ptr(expert_token_nums), _ptr(w1),
            _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    return Prepared(_lib.mdc_ffn_quant_input, args, "mdc_ffn_quant_input", (sh,))


def prepare_ffn(shape: Shape, inter_n: int, expand_x, expert_token_nums, w1, w1_scale, w2, w2_scale, y,
                workspace, stream=None) -> "Prepared":
    sh = shape.c()
    args = (ctypes.byref(sh), int(inter_n), _ptr(expand_x), _ptr(expert_token_nums), _ptr(w1), _ptr(w1_scale),
            _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_ffn, args, "mdc_ffn", (sh,))


class Prepared:
    """A C entry point with its arguments marshalled once, for repeated launches.

    Calling it enqueues the same work again on the stream captured at
    preparation; the referenced tensors must stay alive.
    """
    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != MDC_OK:
            raise MdcError(st, self._name)


def prepare_dispatch(shape: Shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                     expert_token_nums, expanded_row_idx, workspace, stream=None) -> Prepared:
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expert_ids), _ptr(x_active_mask), _ptr(expand_x), _ptr(assist_info),
            _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_dispatch, args, "mdc_dispatch", (sh,))


def prepare_dispatch_layout(shape: Shape, expert_ids, x_active_mask, workspace, stream=None) -> Prepared:
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(expert_ids), _ptr(x_active_mask), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    return Prepared(_lib.mdc_dispatch_layout, args, "mdc_dispatch_layout", (sh,))


def prepare_dispatch_gather(shape: Shape, x, expand_x, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, workspace, stream=None) -> Prepared:
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expand_x), _ptr(assist_info), _ptr(ep_recv_counts),
            _ptr(expert_token_nums), _ptr(expanded_row_idx), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    return Prepared(_lib.mdc_dispatch_gather, args, "mdc_dispatch_gather", (sh,))


def prepare_combine(shape: Shape, expand_x: Sequence, assist_info: Sequence, ep_recv_counts: Sequence,
                    expanded_row_idx, expert_ids, expert_scales, x_active_mask, shared_expert_x, x_out,
                    workspace=None, stream=None, ori_x=None) -> Prepared:
    sh = shape.c()
    ty, ta, tc = _table(expand_x), _table(assist_info), _table(ep_recv_counts)
    args = (ctypes.byref(sh), ctypes.cast(ty, _P), ctypes.cast(ta, _P), ctypes.cast(tc, _P),
            _ptr(expanded_row_idx), _ptr(expert_ids), _ptr(expert_scales), _ptr(x_active_mask),
            _ptr(shared_expert_x), _ptr(ori_x), _ptr(x_out), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    return Prepared(_lib.mdc_combine, args, "mdc_combine", (sh, ty, ta, tc))


def alloc_dispatch_outputs(shape: Shape, device="cuda"):
    """Device buffers for one destination rank's dispatch outputs (plumbing for callers)."""
    import torch
    L, W, A = shape.local_experts, shape.world, shape.capacity
    return {
        "expand_x": torch.empty((A, shape.hidden), dtype=torch.bfloat16, device=device),
        "assist_info": torch.empty((A, 3), dtype=torch.int32, device=device),
        "ep_recv_counts": torch.empty((L * W,), dtype=torch.int32, device=device),
        "expert_token_nums": torch.empty((L,), dtype=torch.int64, device=device),
        "workspace": torch.empty((mdc_dispatch_workspace_size(shape),), dtype=torch.uint8, device=device),
    }
