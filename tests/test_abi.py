"""The C-ABI library loads, exports every entry point include/mdc.h declares,
and reports argument errors synchronously (no GPU needed: every call below
returns before anything is enqueued)."""
import ctypes
import os
import re

import pytest

import combine_route_histogram_amd as mdc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mdc.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(mdc_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_expected_entry_points():
    names = _declared()
    for need in ("mdc_dispatch", "mdc_dispatch_layout", "mdc_dispatch_gather", "mdc_combine",
                 "mdc_dispatch_workspace_size", "mdc_combine_workspace_size", "mdc_status_string"):
        assert need in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mdc.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(mdc.EXPORTS)


def test_abi_version_and_status_strings():
    assert mdc.mdc_abi_version() == 2
    for code in range(5):
        assert mdc.mdc_status_string(code).startswith("MDC_")


SHARE = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)


def test_workspace_size_is_positive_and_grows():
    a = mdc.mdc_dispatch_workspace_size(SHARE)
    b = mdc.mdc_dispatch_workspace_size(mdc.Shape(8, 0, 4096, 7168, 8, 128, 131072))
    assert 0 < a < b
    assert mdc.mdc_combine_workspace_size(SHARE) >= 0


@pytest.mark.parametrize("field,value", [
    ("world", 0), ("rank", -1), ("rank", 8), ("bs", -1), ("hidden", 0), ("hidden", 100),
    ("topk", 0), ("topk", 17), ("num_experts", 0), ("num_experts", 100), ("capacity", -1),
    ("num_experts", 8 * 4096),
])
def test_invalid_shapes_rejected(field, value):
    d = dict(SHARE.__dict__)
    d[field] = value
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_dispatch_workspace_size(mdc.Shape(**d))
    assert ei.value.status == mdc.MDC_ERR_INVALID


def test_null_shape_and_pointers():
    lib = ctypes.CDLL(mdc.LIB_PATH)
    lib.mdc_dispatch_workspace_size.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    out = ctypes.c_size_t(0)
    assert lib.mdc_dispatch_workspace_size(None, ctypes.byref(out)) == mdc.MDC_ERR_NULLPTR
    sh = SHARE.c()
    assert lib.mdc_dispatch_workspace_size(ctypes.byref(sh), None) == mdc.MDC_ERR_NULLPTR
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace_size(SHARE)
    # missing ids / outputs / workspace -> NULLPTR, nothing enqueued
    for args in [
        (fake, None, None, fake, fake, fake, fake, fake, fake),
        (fake, fake, None, fake, fake, None, fake, fake, fake),
        (None, fake, None, fake, fake, fake, fake, fake, fake),
        (fake, fake, None, fake, fake, fake, fake, None, fake),
        (fake, fake, None, fake, fake, fake, fake, fake, None),
    ]:
        st = lib.mdc_dispatch(ctypes.byref(sh), *[ctypes.c_void_p(a) for a in args], ctypes.c_size_t(ws), None)
        assert st == mdc.MDC_ERR_NULLPTR


def test_small_workspace_rejected():
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace_size(SHARE)
    lib = ctypes.CDLL(mdc.LIB_PATH)
    sh = SHARE.c()
    st = lib.mdc_dispatch_layout(ctypes.byref(sh), ctypes.c_void_p(fake), None, ctypes.c_void_p(fake),
                                 ctypes.c_size_t(ws - 1), None)
    assert st == mdc.MDC_ERR_WORKSPACE
    st = lib.mdc_dispatch_gather(ctypes.byref(sh), *[ctypes.c_void_p(fake)] * 7, ctypes.c_size_t(ws - 1), None)
    assert st == mdc.MDC_ERR_WORKSPACE


def test_misaligned_rows_rejected():
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace_size(SHARE)
    lib = ctypes.CDLL(mdc.LIB_PATH)
    sh = SHARE.c()
    st = lib.mdc_dispatch_gather(ctypes.byref(sh), ctypes.c_void_p(fake + 2), *[ctypes.c_void_p(fake)] * 6,
                                 ctypes.c_size_t(ws), None)
    assert st == mdc.MDC_ERR_INVALID


def test_ffn_shape_checks():
    ok = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)
    assert mdc.mdc_ffn_workspace_size(ok, 4096) > 131072 * 7168
    for inter in (0, 100, 4096 + 128):
        with pytest.raises(mdc.MdcError) as ei:
            mdc.mdc_ffn_workspace_size(ok, inter)
        assert ei.value.status == mdc.MDC_ERR_INVALID
    bad_h = mdc.Shape(world=8, rank=0, bs=16, hidden=7176, topk=8, num_experts=128, capacity=1024)
    with pytest.raises(mdc.MdcError):
        mdc.mdc_ffn_workspace_size(bad_h, 4096)
    fake = 1 << 20
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_ffn(ok, 4096, fake, None, fake, fake, fake, fake, fake, fake)
    assert ei.value.status == mdc.MDC_ERR_NULLPTR
    # the GEMM tile count (A / 256 + L + 2) * (N / 256 + ceil(H / 256)) must stay below 2^31:
    # at the largest capacity, N = 2^23 with H = 128 passes the N * H bound but not this one
    big_a = mdc.Shape(world=8, rank=0, bs=16, hidden=128, topk=8, num_experts=128, capacity=2**31 - 1)
    assert mdc.mdc_ffn_workspace_size(big_a, 256) > 0
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_ffn_workspace_size(big_a, 2**23)
    assert ei.value.status == mdc.MDC_ERR_INVALID


def test_combine_world_limit_and_nulls():
    big = mdc.Shape(world=65, rank=0, bs=4, hidden=64, topk=2, num_experts=65, capacity=16)
    fake = 1 << 20
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(big, [fake] * 65, [fake] * 65, [fake] * 65, fake, fake, fake, None, None, fake)
    assert ei.value.status == mdc.MDC_ERR_INVALID
    small = mdc.Shape(world=2, rank=0, bs=4, hidden=64, topk=2, num_experts=4, capacity=16)
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(small, [fake, fake], [fake, fake], [fake, None], fake, fake, fake, None, None, fake)
    assert ei.value.status == mdc.MDC_ERR_NULLPTR
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(small, [fake, fake], [fake, fake], [fake, fake], fake, None, fake, None, None, fake)
    assert ei.value.status == mdc.MDC_ERR_NULLPTR
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(small, [fake, fake + 8], [fake, fake], [fake, fake], fake, fake, fake, None, None, fake)
    assert ei.value.status == mdc.MDC_ERR_INVALID
