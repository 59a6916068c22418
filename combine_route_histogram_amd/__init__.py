"""Python binding of libmdc (MoE dispatch/combine for MI355X).

Argument marshalling only: every step of the path runs in the HIP kernels of
libmdc.so, declared in include/mdc.h.  torch tensors are passed as device
pointers; torch provides device memory and streams.  The functions carry the
names of the C entry points.  Tensor arguments are checked for dtype and
size against the shape once, when they are marshalled (an undersized buffer
would otherwise be read or written out of bounds on the device).  Importing
this package fails loudly when libmdc.so has not been built
(python combine_route_histogram_amd/build.py).
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
import torch  # noqa: E402

_lib = ctypes.CDLL(LIB_PATH)

MDC_ABI_VERSION = 4
MDC_OK = 0
MDC_ERR_NULLPTR = 1
MDC_ERR_INVALID = 2
MDC_ERR_UNSUPPORTED = 3
MDC_ERR_WORKSPACE = 4
MDC_ERR_HIP = 5
MDC_MAX_TOPK = 16
MDC_MAX_LOCAL_EXPERTS = 2048
MDC_MAX_COMBINE_WORLD = 64
MDC_FLAG_FFN_PIPELINE = 0x1
MDC_FLAG_SPIN_SHIFT = 8
MDC_STATUS_BYTES = 256

EXPORTS = (
    "mdc_status_string", "mdc_abi_version",
    "mdc_dispatch_workspace", "mdc_dispatch_workspace_size", "mdc_dispatch_layout", "mdc_dispatch_gather",
    "mdc_dispatch", "mdc_combine_workspace", "mdc_combine_workspace_size", "mdc_combine",
    "mdc_ffn_workspace", "mdc_ffn_workspace_size", "mdc_ffn", "mdc_dispatch_quant", "mdc_dispatch_quant_gather",
    "mdc_ffn_quant_input", "mdc_dispatch_noalloc", "mdc_dispatch_ffn",
)


class mdc_shape(ctypes.Structure):
    _fields_ = [("world", ctypes.c_int32), ("rank", ctypes.c_int32), ("bs", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("topk", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("capacity", ctypes.c_int64), ("mask_per_route", ctypes.c_int32),
                ("zero_experts", ctypes.c_int32), ("copy_experts", ctypes.c_int32), ("flags", ctypes.c_int32)]


_P = ctypes.c_void_p
_SZ = ctypes.c_size_t
_SHP = ctypes.POINTER(mdc_shape)


def _sig(name, *args):
    fn = getattr(_lib, name, None)
    if fn is None:
        return
    fn.restype = ctypes.c_int
    fn.argtypes = list(args)


_lib.mdc_status_string.restype = ctypes.c_char_p
_lib.mdc_status_string.argtypes = [ctypes.c_int]
_lib.mdc_abi_version.restype = ctypes.c_int32
_lib.mdc_abi_version.argtypes = []
for _n in ("mdc_dispatch_workspace", "mdc_dispatch_workspace_size", "mdc_combine_workspace",
           "mdc_combine_workspace_size"):
    _sig(_n, _SHP, ctypes.POINTER(_SZ))
for _n in ("mdc_ffn_workspace", "mdc_ffn_workspace_size"):
    _sig(_n, _SHP, ctypes.c_int32, ctypes.POINTER(_SZ))
_sig("mdc_dispatch_layout", _SHP, _P, _P, _P, _SZ, _P)
_sig("mdc_dispatch_gather", _SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_dispatch", _SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_dispatch_quant_gather", _SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_dispatch_quant", _SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_combine", _SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_ffn", _SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_ffn_quant_input", _SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P)
_sig("mdc_dispatch_noalloc", _SHP, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P)
_sig("mdc_dispatch_ffn", _SHP, ctypes.c_int32, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _SZ, _P,
     _SZ, _P)
MDC_NOALLOC_SCRATCH_BYTES = 8 << 20


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
    flags: int = 0

    @property
    def local_experts(self) -> int:
        return self.num_experts // self.world

    def c(self) -> mdc_shape:
        return mdc_shape(self.world, self.rank, self.bs, self.hidden, self.topk, self.num_experts, self.capacity,
                         self.mask_per_route, self.zero_experts, self.copy_experts, self.flags)

    def with_rank(self, rank: int) -> "Shape":
        return replace(self, rank=rank)


# ----------------------------------------------------------------------------
# marshalling helpers
# ----------------------------------------------------------------------------

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
        if torch.cuda.is_available():
            return torch.cuda.current_stream().cuda_stream
        return None
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status: int, where: str) -> None:
    if status != MDC_OK:
        raise MdcError(status, where)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16) if hasattr(torch, "uint16") else (torch.bfloat16, torch.int16)


def _need(t, name: str, dtypes, numel: int) -> None:
    """Tensor argument `name` must have one of `dtypes` and hold at least `numel` elements.

    Raw integer pointers and None pass (the C library checks NULL; a raw
    pointer carries no size to check).
    """
    if t is None or isinstance(t, int):
        return
    if not isinstance(dtypes, tuple):
        dtypes = (dtypes,)
    if t.dtype not in dtypes:
        raise ValueError(f"mdc: {name} must be {'/'.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.numel() < numel:
        raise ValueError(f"mdc: {name} holds {t.numel()} elements, needs at least {numel}")


def _check_mask(shape: Shape, mask, ranks: int) -> None:
    per = shape.topk if shape.mask_per_route else 1
    _need(mask, "x_active_mask", (torch.uint8, torch.bool), ranks * shape.bs * per)


def _check_dispatch_inputs(shape: Shape, x, expert_ids, mask, expert_scales) -> None:
    W, BS, K, H = shape.world, shape.bs, shape.topk, shape.hidden
    _need(x, "x", _BF16, W * BS * H)
    _need(expert_ids, "expert_ids", torch.int32, W * BS * K)
    _check_mask(shape, mask, W)
    _need(expert_scales, "expert_scales", torch.float32, W * BS * K)


def _check_dispatch_outputs(shape: Shape, rows, rows_dtype, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales, dyn_scales=None) -> None:
    W, BS, K, H, A, L = shape.world, shape.bs, shape.topk, shape.hidden, shape.capacity, shape.local_experts
    _need(rows, "expand_x" if rows_dtype is _BF16 else "expand_q", rows_dtype, A * H)
    _need(dyn_scales, "dynamic_scales", torch.float32, A)
    _need(assist_info, "assist_info", torch.int32, A * 3)
    _need(ep_recv_counts, "ep_recv_counts", torch.int32, L * W)
    _need(expert_token_nums, "expert_token_nums", torch.int64, L)
    _need(expanded_row_idx, "expanded_row_idx", torch.int32, W * BS * K)
    _need(expand_scales, "expand_scales", torch.float32, A)


def _check_workspace(ws, need: int, name: str = "workspace") -> None:
    if ws is None or isinstance(ws, int):
        return
    if _nbytes(ws) < need:
        raise ValueError(f"mdc: {name} holds {_nbytes(ws)} bytes, needs {need}")


# ----------------------------------------------------------------------------
# size queries
# ----------------------------------------------------------------------------

def mdc_dispatch_workspace(shape: Shape) -> int:
    out = _SZ(0)
    sh = shape.c()
    _check(_lib.mdc_dispatch_workspace(ctypes.byref(sh), ctypes.byref(out)), "mdc_dispatch_workspace")
    return int(out.value)


def mdc_combine_workspace(shape: Shape) -> int:
    out = _SZ(0)
    sh = shape.c()
    _check(_lib.mdc_combine_workspace(ctypes.byref(sh), ctypes.byref(out)), "mdc_combine_workspace")
    return int(out.value)


def mdc_ffn_workspace(shape: Shape, inter_n: int) -> int:
    out = _SZ(0)
    sh = shape.c()
    _check(_lib.mdc_ffn_workspace(ctypes.byref(sh), int(inter_n), ctypes.byref(out)), "mdc_ffn_workspace")
    return int(out.value)


# the earlier names of the same queries
mdc_dispatch_workspace_size = mdc_dispatch_workspace
mdc_combine_workspace_size = mdc_combine_workspace
mdc_ffn_workspace_size = mdc_ffn_workspace


def read_status(workspace) -> dict:
    """The device status block at the start of a dispatch or FFN workspace (synchronises its stream)."""
    v = workspace[:16].view(torch.int32).cpu().tolist()
    return {"dropped_ids": v[0], "overflow_rows": v[1], "wait_timeouts": v[2]}


# ----------------------------------------------------------------------------
# Prepared calls: marshal once, launch many times
# ----------------------------------------------------------------------------

class Prepared:
    """A C entry point with its arguments marshalled once, for repeated launches.

    Calling it enqueues the same work again on the stream captured at
    preparation.  It holds references to the tensors it was prepared with, so
    their memory stays allocated while the object lives.
    """
    __slots__ = ("_fn", "_args", "_name", "_keep")

    def __init__(self, fn, args, name, keep):
        self._fn, self._args, self._name, self._keep = fn, args, name, keep

    def __call__(self) -> None:
        st = self._fn(*self._args)
        if st != MDC_OK:
            raise MdcError(st, self._name)


def _tensors(names: dict) -> tuple:
    """The tensor arguments among a prepare_* call's locals (and inside its pointer-table lists)."""
    out = []
    for v in names.values():
        if isinstance(v, torch.Tensor):
            out.append(v)
        elif isinstance(v, (list, tuple)):
            out.extend(t for t in v if isinstance(t, torch.Tensor))
    return tuple(out)


def _run(p: Prepared, check: bool) -> int:
    st = p._fn(*p._args)
    if check:
        _check(st, p._name)
    return st


def prepare_dispatch_layout(shape: Shape, expert_ids, x_active_mask, workspace, stream=None) -> Prepared:
    _need(expert_ids, "expert_ids", torch.int32, shape.world * shape.bs * shape.topk)
    _check_mask(shape, x_active_mask, shape.world)
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(expert_ids), _ptr(x_active_mask), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    return Prepared(_lib.mdc_dispatch_layout, args, "mdc_dispatch_layout", (sh, _tensors(locals())))


def prepare_dispatch_gather(shape: Shape, x, expand_x, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, workspace, stream=None, expert_scales=None,
                            expand_scales=None) -> Prepared:
    _check_dispatch_inputs(shape, x, None, None, expert_scales)
    _check_dispatch_outputs(shape, expand_x, _BF16, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales)
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expert_scales), _ptr(expand_x), _ptr(assist_info), _ptr(ep_recv_counts),
            _ptr(expert_token_nums), _ptr(expanded_row_idx), _ptr(expand_scales), _ptr(workspace),
            _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_dispatch_gather, args, "mdc_dispatch_gather", (sh, _tensors(locals())))


def prepare_dispatch(shape: Shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                     expert_token_nums, expanded_row_idx, workspace, stream=None, expert_scales=None,
                     expand_scales=None) -> Prepared:
    _check_dispatch_inputs(shape, x, expert_ids, x_active_mask, expert_scales)
    _check_dispatch_outputs(shape, expand_x, _BF16, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales)
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expert_ids), _ptr(x_active_mask), _ptr(expert_scales), _ptr(expand_x),
            _ptr(assist_info), _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx),
            _ptr(expand_scales), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_dispatch, args, "mdc_dispatch", (sh, _tensors(locals())))


def prepare_dispatch_quant_gather(shape: Shape, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                                  expert_token_nums, expanded_row_idx, workspace, stream=None, expert_scales=None,
                                  expand_scales=None) -> Prepared:
    _check_dispatch_inputs(shape, x, None, None, expert_scales)
    _check_dispatch_outputs(shape, expand_q, torch.int8, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales, dynamic_scales)
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expert_scales), _ptr(expand_q), _ptr(dynamic_scales), _ptr(assist_info),
            _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx), _ptr(expand_scales),
            _ptr(workspace), _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_dispatch_quant_gather, args, "mdc_dispatch_quant_gather", (sh, _tensors(locals())))


def prepare_dispatch_quant(shape: Shape, x, expert_ids, x_active_mask, expand_q, dynamic_scales, assist_info,
                           ep_recv_counts, expert_token_nums, expanded_row_idx, workspace, stream=None,
                           expert_scales=None, expand_scales=None) -> Prepared:
    _check_dispatch_inputs(shape, x, expert_ids, x_active_mask, expert_scales)
    _check_dispatch_outputs(shape, expand_q, torch.int8, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales, dynamic_scales)
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expert_ids), _ptr(x_active_mask), _ptr(expert_scales), _ptr(expand_q),
            _ptr(dynamic_scales), _ptr(assist_info), _ptr(ep_recv_counts), _ptr(expert_token_nums),
            _ptr(expanded_row_idx), _ptr(expand_scales), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_dispatch_quant, args, "mdc_dispatch_quant", (sh, _tensors(locals())))


def _table(items: Optional[Sequence]):
    if items is None:
        return None
    arr = (ctypes.c_void_p * max(1, len(items)))()
    for i, t in enumerate(items):
        arr[i] = _ptr(t)
    return arr


def prepare_combine(shape: Shape, expand_x: Sequence, assist_info: Sequence, ep_recv_counts: Sequence,
                    expanded_row_idx, expert_ids, expert_scales, x_active_mask, shared_expert_x, x_out,
                    workspace=None, stream=None, ori_x=None, expand_scales: Optional[Sequence] = None,
                    performance_info=None) -> Prepared:
    W, BS, K, H, A, L = shape.world, shape.bs, shape.topk, shape.hidden, shape.capacity, shape.local_experts
    for name, tab in (("expand_x", expand_x), ("assist_info", assist_info), ("ep_recv_counts", ep_recv_counts),
                      ("expand_scales", expand_scales)):
        if tab is not None and len(tab) < W:
            raise ValueError(f"mdc: {name} needs {W} entries, got {len(tab)}")
    for j in range(W):
        _need(expand_x[j], f"expand_x[{j}]", _BF16, A * H)
        _need(assist_info[j], f"assist_info[{j}]", torch.int32, A * 3)
        _need(ep_recv_counts[j], f"ep_recv_counts[{j}]", torch.int32, L * W)
        if expand_scales is not None:
            _need(expand_scales[j], f"expand_scales[{j}]", torch.float32, A)
    _need(expanded_row_idx, "expanded_row_idx", torch.int32, BS * K)
    _need(expert_ids, "expert_ids", torch.int32, BS * K)
    _need(expert_scales, "expert_scales", torch.float32, BS * K)
    _check_mask(shape, x_active_mask, 1)
    _need(shared_expert_x, "shared_expert_x", _BF16, BS * H)
    _need(ori_x, "ori_x", _BF16, BS * H)
    _need(x_out, "x_out", _BF16, BS * H)
    _need(performance_info, "performance_info", torch.int64, W)
    if performance_info is not None:
        _check_workspace(workspace, mdc_combine_workspace(shape))
    sh = shape.c()
    ty, ta, tc, te = _table(expand_x), _table(assist_info), _table(ep_recv_counts), _table(expand_scales)
    args = (ctypes.byref(sh), ctypes.cast(ty, _P), ctypes.cast(ta, _P), ctypes.cast(tc, _P),
            _ptr(expanded_row_idx), _ptr(expert_ids), _ptr(expert_scales), _ptr(x_active_mask),
            None if te is None else ctypes.cast(te, _P), _ptr(shared_expert_x), _ptr(ori_x),
            _ptr(performance_info), _ptr(x_out), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_combine, args, "mdc_combine", (sh, ty, ta, tc, te, _tensors(locals())))


def _check_ffn_weights(shape: Shape, inter_n: int, expert_token_nums, w1, w1_scale, w2, w2_scale, y) -> None:
    L, H, A, N = shape.local_experts, shape.hidden, shape.capacity, int(inter_n)
    _need(expert_token_nums, "expert_token_nums", torch.int64, L)
    _need(w1, "w1", torch.int8, L * N * H)
    _need(w1_scale, "w1_scale", torch.float32, L * N)
    _need(w2, "w2", torch.int8, L * H * (N // 2))
    _need(w2_scale, "w2_scale", torch.float32, L * H)
    _need(y, "y", _BF16, A * H)


def prepare_ffn(shape: Shape, inter_n: int, expand_x, expert_token_nums, w1, w1_scale, w2, w2_scale, y,
                workspace, stream=None) -> Prepared:
    _need(expand_x, "expand_x", _BF16, shape.capacity * shape.hidden)
    _check_ffn_weights(shape, inter_n, expert_token_nums, w1, w1_scale, w2, w2_scale, y)
    sh = shape.c()
    args = (ctypes.byref(sh), int(inter_n), _ptr(expand_x), _ptr(expert_token_nums), _ptr(w1), _ptr(w1_scale),
            _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(workspace), _nbytes(workspace), _stream(stream))
    return Prepared(_lib.mdc_ffn, args, "mdc_ffn", (sh, _tensors(locals())))


def prepare_ffn_quant_input(shape: Shape, inter_n: int, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale,
                            w2, w2_scale, y, workspace, stream=None) -> Prepared:
    _need(expand_q, "expand_q", torch.int8, shape.capacity * shape.hidden)
    _need(dynamic_scales, "dynamic_scales", torch.float32, shape.capacity)
    _check_ffn_weights(shape, inter_n, expert_token_nums, w1, w1_scale, w2, w2_scale, y)
    sh = shape.c()
    args = (ctypes.byref(sh), int(inter_n), _ptr(expand_q), _ptr(dynamic_scales), _ptr(expert_token_nums), _ptr(w1),
            _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(y), _ptr(workspace), _nbytes(workspace),
            _stream(stream))
    return Prepared(_lib.mdc_ffn_quant_input, args, "mdc_ffn_quant_input", (sh, _tensors(locals())))


def prepare_dispatch_noalloc(shape: Shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                             expert_token_nums, expanded_row_idx, stream=None, expert_scales=None,
                             expand_scales=None) -> Prepared:
    _check_dispatch_inputs(shape, x, expert_ids, x_active_mask, expert_scales)
    _check_dispatch_outputs(shape, expand_x, _BF16, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales)
    sh = shape.c()
    args = (ctypes.byref(sh), _ptr(x), _ptr(expert_ids), _ptr(x_active_mask), _ptr(expert_scales), _ptr(expand_x),
            _ptr(assist_info), _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx),
            _ptr(expand_scales), _stream(stream))
    return Prepared(_lib.mdc_dispatch_noalloc, args, "mdc_dispatch_noalloc", (sh, _tensors(locals())))


def prepare_dispatch_ffn(shape: Shape, inter_n: int, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                         expert_token_nums, expanded_row_idx, w1, w1_scale, w2, w2_scale, y, dispatch_workspace,
                         ffn_workspace, stream=None, expert_scales=None, expand_scales=None) -> Prepared:
    """Quantised dispatch + grouped FFN as one pipeline (after mdc_dispatch_layout on dispatch_workspace)."""
    _check_dispatch_inputs(shape, x, None, None, expert_scales)
    _check_dispatch_outputs(shape, expand_q, torch.int8, assist_info, ep_recv_counts, expert_token_nums,
                            expanded_row_idx, expand_scales, dynamic_scales)
    _check_ffn_weights(shape, inter_n, expert_token_nums, w1, w1_scale, w2, w2_scale, y)
    sh = shape.c()
    args = (ctypes.byref(sh), int(inter_n), _ptr(x), _ptr(expert_scales), _ptr(expand_q), _ptr(dynamic_scales),
            _ptr(assist_info), _ptr(ep_recv_counts), _ptr(expert_token_nums), _ptr(expanded_row_idx),
            _ptr(expand_scales), _ptr(w1), _ptr(w1_scale), _ptr(w2), _ptr(w2_scale), _ptr(y),
            _ptr(dispatch_workspace), _nbytes(dispatch_workspace), _ptr(ffn_workspace), _nbytes(ffn_workspace),
            _stream(stream))
    return Prepared(_lib.mdc_dispatch_ffn, args, "mdc_dispatch_ffn", (sh, _tensors(locals())))


# ----------------------------------------------------------------------------
# one-shot calls (marshal and launch)
# ----------------------------------------------------------------------------

def mdc_dispatch_layout(shape: Shape, expert_ids, x_active_mask, workspace, stream=None, check: bool = True) -> int:
    return _run(prepare_dispatch_layout(shape, expert_ids, x_active_mask, workspace, stream), check)


def mdc_dispatch_gather(shape: Shape, x, expand_x, assist_info, ep_recv_counts, expert_token_nums,
                        expanded_row_idx, workspace, stream=None, check: bool = True, expert_scales=None,
                        expand_scales=None) -> int:
    return _run(prepare_dispatch_gather(shape, x, expand_x, assist_info, ep_recv_counts, expert_token_nums,
                                        expanded_row_idx, workspace, stream, expert_scales, expand_scales), check)


def mdc_dispatch(shape: Shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                 expert_token_nums, expanded_row_idx, workspace, stream=None, check: bool = True, expert_scales=None,
                 expand_scales=None) -> int:
    return _run(prepare_dispatch(shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                                 expert_token_nums, expanded_row_idx, workspace, stream, expert_scales,
                                 expand_scales), check)


def mdc_dispatch_quant_gather(shape: Shape, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                              expert_token_nums, expanded_row_idx, workspace, stream=None, check: bool = True,
                              expert_scales=None, expand_scales=None) -> int:
    return _run(prepare_dispatch_quant_gather(shape, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                                              expert_token_nums, expanded_row_idx, workspace, stream, expert_scales,
                                              expand_scales), check)


def mdc_dispatch_quant(shape: Shape, x, expert_ids, x_active_mask, expand_q, dynamic_scales, assist_info,
                       ep_recv_counts, expert_token_nums, expanded_row_idx, workspace, stream=None,
                       check: bool = True, expert_scales=None, expand_scales=None) -> int:
    return _run(prepare_dispatch_quant(shape, x, expert_ids, x_active_mask, expand_q, dynamic_scales, assist_info,
                                       ep_recv_counts, expert_token_nums, expanded_row_idx, workspace, stream,
                                       expert_scales, expand_scales), check)


def mdc_combine(shape: Shape, expand_x: Sequence, assist_info: Sequence, ep_recv_counts: Sequence,
                expanded_row_idx, expert_ids, expert_scales, x_active_mask, shared_expert_x, x_out,
                workspace=None, stream=None, check: bool = True, ori_x=None, expand_scales=None,
                performance_info=None) -> int:
    return _run(prepare_combine(shape, expand_x, assist_info, ep_recv_counts, expanded_row_idx, expert_ids,
                                expert_scales, x_active_mask, shared_expert_x, x_out, workspace, stream, ori_x,
                                expand_scales, performance_info), check)


def mdc_ffn(shape: Shape, inter_n: int, expand_x, expert_token_nums, w1, w1_scale, w2, w2_scale, y, workspace,
            stream=None, check: bool = True) -> int:
    return _run(prepare_ffn(shape, inter_n, expand_x, expert_token_nums, w1, w1_scale, w2, w2_scale, y, workspace,
                            stream), check)


def mdc_ffn_quant_input(shape: Shape, inter_n: int, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale, w2,
                        w2_scale, y, workspace, stream=None, check: bool = True) -> int:
    return _run(prepare_ffn_quant_input(shape, inter_n, expand_q, dynamic_scales, expert_token_nums, w1, w1_scale,
                                        w2, w2_scale, y, workspace, stream), check)


def mdc_dispatch_noalloc(shape: Shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                         expert_token_nums, expanded_row_idx, stream=None, check: bool = True, expert_scales=None,
                         expand_scales=None) -> int:
    return _run(prepare_dispatch_noalloc(shape, x, expert_ids, x_active_mask, expand_x, assist_info, ep_recv_counts,
                                         expert_token_nums, expanded_row_idx, stream, expert_scales, expand_scales),
                check)


def mdc_dispatch_ffn(shape: Shape, inter_n: int, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                     expert_token_nums, expanded_row_idx, w1, w1_scale, w2, w2_scale, y, dispatch_workspace,
                     ffn_workspace, stream=None, check: bool = True, expert_scales=None, expand_scales=None) -> int:
    return _run(prepare_dispatch_ffn(shape, inter_n, x, expand_q, dynamic_scales, assist_info, ep_recv_counts,
                                     expert_token_nums, expanded_row_idx, w1, w1_scale, w2, w2_scale, y,
                                     dispatch_workspace, ffn_workspace, stream, expert_scales, expand_scales), check)


def alloc_dispatch_outputs(shape: Shape, device="cuda"):
    """Device buffers for one destination rank's dispatch outputs (plumbing for callers)."""
    L, W, A = shape.local_experts, shape.world, shape.capacity
    return {
        "expand_x": torch.empty((A, shape.hidden), dtype=torch.bfloat16, device=device),
        "assist_info": torch.empty((A, 3), dtype=torch.int32, device=device),
        "ep_recv_counts": torch.empty((L * W,), dtype=torch.int32, device=device),
        "expert_token_nums": torch.empty((L,), dtype=torch.int64, device=device),
        "workspace": torch.empty((mdc_dispatch_workspace(shape),), dtype=torch.uint8, device=device),
    }
