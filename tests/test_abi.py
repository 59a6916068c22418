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
    for need in ("mdc_dispatch", "mdc_dispatch_layout", "mdc_dispatch_gather", "mdc_combine", "mdc_ffn",
                 "mdc_dispatch_workspace", "mdc_combine_workspace", "mdc_ffn_workspace",
                 "mdc_dispatch_workspace_size", "mdc_combine_workspace_size", "mdc_ffn_workspace_size",
                 "mdc_status_string"):
        assert need in names


def _header_int(name):
    src = open(HEADER).read()
    m = re.search(r"\b" + name + r"\s*=\s*(\d+)", src) or re.search(r"#define\s+" + name + r"\s+(\w+)", src)
    return int(m.group(1).rstrip("uU"), 0)


def test_status_codes_match_the_header_and_the_boundary():
    """MDC_OK .. MDC_ERR_HIP as the boundary lists them: 0 ok, 1 null, 2 invalid, 3 unsupported, 4 workspace, 5 HIP."""
    want = {"MDC_OK": 0, "MDC_ERR_NULLPTR": 1, "MDC_ERR_INVALID": 2, "MDC_ERR_UNSUPPORTED": 3,
            "MDC_ERR_WORKSPACE": 4, "MDC_ERR_HIP": 5}
    for name, code in want.items():
        assert _header_int(name) == code, name
        assert getattr(mdc, name) == code, name
        assert mdc.mdc_status_string(code).startswith(name)
    assert _header_int("MDC_STATUS_BYTES") == mdc.MDC_STATUS_BYTES == 256
    assert _header_int("MDC_FLAG_FFN_PIPELINE") == mdc.MDC_FLAG_FFN_PIPELINE
    assert _header_int("MDC_ABI_VERSION") == mdc.MDC_ABI_VERSION == mdc.mdc_abi_version()


def test_status_block_layout():
    """mdc_device_status: four int32 fields (dropped_ids, overflow_rows, wait_timeouts, reserved) at offset 0."""
    src = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    body = re.search(r"typedef struct \{([^}]*)\} mdc_device_status;", src).group(1)
    fields = re.findall(r"int32_t\s+(\w+);", body)
    assert fields == ["dropped_ids", "overflow_rows", "wait_timeouts", "reserved"]


def test_workspace_queries_and_their_earlier_names_agree():
    for sh in (SHARE, mdc.Shape(8, 3, 32, 7168, 8, 256, 2048), mdc.Shape(1, 0, 16, 128, 2, 8, 32)):
        a = mdc.mdc_dispatch_workspace(sh)
        assert a == mdc.mdc_dispatch_workspace_size(sh) >= mdc.MDC_STATUS_BYTES
        assert mdc.mdc_combine_workspace(sh) == mdc.mdc_combine_workspace_size(sh)
        lib = ctypes.CDLL(mdc.LIB_PATH)
        c = sh.c()
        for name in ("mdc_dispatch_workspace", "mdc_dispatch_workspace_size"):
            out = ctypes.c_size_t(0)
            fn = getattr(lib, name)
            fn.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            assert fn(ctypes.byref(c), ctypes.byref(out)) == mdc.MDC_OK and out.value == a
    ok = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)
    assert mdc.mdc_ffn_workspace(ok, 4096) == mdc.mdc_ffn_workspace_size(ok, 4096)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(mdc.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name
    assert set(_declared()) == set(mdc.EXPORTS)


def test_abi_version_and_status_strings():
    assert mdc.mdc_abi_version() == 4
    for code in range(6):
        assert mdc.mdc_status_string(code).startswith("MDC_")


SHARE = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)


def test_workspace_size_is_positive_and_grows():
    a = mdc.mdc_dispatch_workspace_size(SHARE)
    b = mdc.mdc_dispatch_workspace_size(mdc.Shape(8, 0, 4096, 7168, 8, 128, 131072))
    assert 0 < a < b
    assert mdc.mdc_combine_workspace_size(SHARE) >= 0


@pytest.mark.parametrize("field,value,code", [
    ("world", 0, mdc.MDC_ERR_INVALID), ("rank", -1, mdc.MDC_ERR_INVALID), ("rank", 8, mdc.MDC_ERR_INVALID),
    ("bs", -1, mdc.MDC_ERR_INVALID), ("hidden", 0, mdc.MDC_ERR_INVALID), ("hidden", 100, mdc.MDC_ERR_INVALID),
    ("topk", 0, mdc.MDC_ERR_INVALID), ("num_experts", 0, mdc.MDC_ERR_INVALID),
    ("num_experts", 100, mdc.MDC_ERR_INVALID), ("capacity", -1, mdc.MDC_ERR_INVALID),
    ("mask_per_route", 2, mdc.MDC_ERR_INVALID), ("zero_experts", -1, mdc.MDC_ERR_INVALID),
    ("flags", 0x4, mdc.MDC_ERR_INVALID), ("flags", 1 << 20, mdc.MDC_ERR_INVALID),
    # well formed, but outside what the library supports
    ("topk", 17, mdc.MDC_ERR_UNSUPPORTED), ("num_experts", 8 * 4096, mdc.MDC_ERR_UNSUPPORTED),
    ("capacity", 2 ** 31, mdc.MDC_ERR_UNSUPPORTED), ("bs", 2 ** 28, mdc.MDC_ERR_UNSUPPORTED),
])
def test_invalid_shapes_rejected(field, value, code):
    d = dict(SHARE.__dict__)
    d[field] = value
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_dispatch_workspace(mdc.Shape(**d))
    assert ei.value.status == code


def test_known_flags_accepted():
    d = dict(SHARE.__dict__)
    d["flags"] = mdc.MDC_FLAG_FFN_PIPELINE | (3 << mdc.MDC_FLAG_SPIN_SHIFT)
    assert mdc.mdc_dispatch_workspace(mdc.Shape(**d)) > 0


def test_null_shape_and_pointers():
    lib = ctypes.CDLL(mdc.LIB_PATH)
    lib.mdc_dispatch_workspace.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
    out = ctypes.c_size_t(0)
    assert lib.mdc_dispatch_workspace(None, ctypes.byref(out)) == mdc.MDC_ERR_NULLPTR
    sh = SHARE.c()
    assert lib.mdc_dispatch_workspace(ctypes.byref(sh), None) == mdc.MDC_ERR_NULLPTR
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace(SHARE)
    # mdc_dispatch(x, ids, mask, scales, expand_x, assist, ep_recv, etn, row_idx, expand_scales, ws):
    # missing ids / outputs / workspace, or expand_scales without scales -> NULLPTR, nothing enqueued
    for args in [
        (fake, None, None, None, fake, fake, fake, fake, fake, None, fake),
        (fake, fake, None, None, fake, fake, None, fake, fake, None, fake),
        (None, fake, None, None, fake, fake, fake, fake, fake, None, fake),
        (fake, fake, None, None, fake, fake, fake, fake, None, None, fake),
        (fake, fake, None, None, fake, fake, fake, fake, fake, None, None),
        (fake, fake, None, None, fake, fake, fake, fake, fake, fake, fake),
    ]:
        st = lib.mdc_dispatch(ctypes.byref(sh), *[ctypes.c_void_p(a) for a in args], ctypes.c_size_t(ws), None)
        assert st == mdc.MDC_ERR_NULLPTR


def test_small_workspace_rejected():
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace(SHARE)
    lib = ctypes.CDLL(mdc.LIB_PATH)
    sh = SHARE.c()
    st = lib.mdc_dispatch_layout(ctypes.byref(sh), ctypes.c_void_p(fake), None, ctypes.c_void_p(fake),
                                 ctypes.c_size_t(ws - 1), None)
    assert st == mdc.MDC_ERR_WORKSPACE
    st = lib.mdc_dispatch_gather(ctypes.byref(sh), ctypes.c_void_p(fake), None, *[ctypes.c_void_p(fake)] * 5, None,
                                 ctypes.c_void_p(fake), ctypes.c_size_t(ws - 1), None)
    assert st == mdc.MDC_ERR_WORKSPACE


def test_misaligned_rows_rejected():
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace(SHARE)
    lib = ctypes.CDLL(mdc.LIB_PATH)
    sh = SHARE.c()
    st = lib.mdc_dispatch_gather(ctypes.byref(sh), ctypes.c_void_p(fake + 2), None, *[ctypes.c_void_p(fake)] * 5,
                                 None, ctypes.c_void_p(fake), ctypes.c_size_t(ws), None)
    assert st == mdc.MDC_ERR_INVALID


def test_quantised_dispatch_past_row_limit_is_unsupported():
    """A whole quantised row lives in one wavefront's registers: H > 8192 is outside the supported range."""
    big = mdc.Shape(world=2, rank=0, bs=4, hidden=8200, topk=2, num_experts=4, capacity=16)
    fake = 1 << 20
    ws = mdc.mdc_dispatch_workspace(big)
    lib = ctypes.CDLL(mdc.LIB_PATH)
    sh = big.c()
    st = lib.mdc_dispatch_quant_gather(ctypes.byref(sh), ctypes.c_void_p(fake), None,
                                       *[ctypes.c_void_p(fake)] * 6, None, ctypes.c_void_p(fake),
                                       ctypes.c_size_t(ws), None)
    assert st == mdc.MDC_ERR_UNSUPPORTED


def test_ffn_shape_checks():
    ok = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)
    assert mdc.mdc_ffn_workspace(ok, 4096) > 131072 * 7168
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_ffn_workspace(ok, 0)
    assert ei.value.status == mdc.MDC_ERR_INVALID
    for inter in (100, 4096 + 128):
        with pytest.raises(mdc.MdcError) as ei:
            mdc.mdc_ffn_workspace(ok, inter)
        assert ei.value.status == mdc.MDC_ERR_UNSUPPORTED
    bad_h = mdc.Shape(world=8, rank=0, bs=16, hidden=7176, topk=8, num_experts=128, capacity=1024)
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_ffn_workspace(bad_h, 4096)
    assert ei.value.status == mdc.MDC_ERR_UNSUPPORTED
    fake = 1 << 20
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_ffn(ok, 4096, fake, None, fake, fake, fake, fake, fake, fake)
    assert ei.value.status == mdc.MDC_ERR_NULLPTR
    # the GEMM tile count (A / 256 + L + 2) * (N / 256 + ceil(H / 256)) must stay below 2^31:
    # at the largest capacity, N = 2^23 with H = 128 passes the N * H bound but not this one
    big_a = mdc.Shape(world=8, rank=0, bs=16, hidden=128, topk=8, num_experts=128, capacity=2**31 - 1)
    assert mdc.mdc_ffn_workspace(big_a, 256) > 0
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_ffn_workspace(big_a, 2**23)
    assert ei.value.status == mdc.MDC_ERR_UNSUPPORTED


def test_dispatch_ffn_argument_checks():
    """mdc_dispatch_ffn checks the quantised gather's arguments, the FFN's, and both workspaces."""
    sh_py = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=131072)
    lib = ctypes.CDLL(mdc.LIB_PATH)
    fake = 1 << 20
    dws, fws = mdc.mdc_dispatch_workspace(sh_py), mdc.mdc_ffn_workspace(sh_py, 4096)
    sh = sh_py.c()
    P = ctypes.c_void_p

    def call(shape=sh, inter=4096, x=fake, scales=None, q=fake, dyn=fake, assist=fake, recv=fake, etn=fake,
             ridx=fake, esc=None, w1=fake, w1s=fake, w2=fake, w2s=fake, y=fake, dw=fake, dwb=dws, fw=fake, fwb=fws):
        return lib.mdc_dispatch_ffn(ctypes.byref(shape), ctypes.c_int32(inter), P(x), P(scales), P(q), P(dyn),
                                    P(assist), P(recv), P(etn), P(ridx), P(esc), P(w1), P(w1s), P(w2), P(w2s), P(y),
                                    P(dw), ctypes.c_size_t(dwb), P(fw), ctypes.c_size_t(fwb), None)

    for kw in (dict(x=None), dict(q=None), dict(dyn=None), dict(assist=None), dict(recv=None), dict(etn=None),
               dict(ridx=None), dict(esc=fake), dict(w1=None), dict(w1s=None), dict(w2=None), dict(w2s=None),
               dict(y=None), dict(dw=None), dict(fw=None)):
        assert call(**kw) == mdc.MDC_ERR_NULLPTR, kw
    assert call(dwb=dws - 1) == mdc.MDC_ERR_WORKSPACE
    assert call(fwb=fws - 1) == mdc.MDC_ERR_WORKSPACE
    assert call(x=fake + 2) == mdc.MDC_ERR_INVALID
    assert call(y=fake + 2) == mdc.MDC_ERR_INVALID
    assert call(inter=0) == mdc.MDC_ERR_INVALID
    assert call(inter=4096 + 128) == mdc.MDC_ERR_UNSUPPORTED
    wide = mdc.Shape(world=2, rank=0, bs=4, hidden=8320, topk=2, num_experts=4, capacity=16).c()
    assert call(shape=wide, inter=256, dwb=1 << 30, fwb=1 << 30) == mdc.MDC_ERR_UNSUPPORTED
    # nothing to receive (A = 0): the weights and y may be NULL; the FFN workspace may not
    empty_py = mdc.Shape(world=8, rank=0, bs=2048, hidden=7168, topk=8, num_experts=128, capacity=0)
    empty = empty_py.c()
    assert call(shape=empty, fw=None, fwb=mdc.mdc_ffn_workspace(empty_py, 4096)) == mdc.MDC_ERR_NULLPTR


def test_combine_world_limit_and_nulls():
    big = mdc.Shape(world=65, rank=0, bs=4, hidden=64, topk=2, num_experts=65, capacity=16)
    fake = 1 << 20
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(big, [fake] * 65, [fake] * 65, [fake] * 65, fake, fake, fake, None, None, fake)
    assert ei.value.status == mdc.MDC_ERR_UNSUPPORTED
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
    # an expand_scales table with a missing entry, and performance_info without a workspace
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(small, [fake, fake], [fake, fake], [fake, fake], fake, fake, fake, None, None, fake,
                        expand_scales=[fake, None])
    assert ei.value.status == mdc.MDC_ERR_NULLPTR
    with pytest.raises(mdc.MdcError) as ei:
        mdc.mdc_combine(small, [fake, fake], [fake, fake], [fake, fake], fake, fake, fake, None, None, fake,
                        performance_info=fake)
    assert ei.value.status == mdc.MDC_ERR_NULLPTR
    lib = ctypes.CDLL(mdc.LIB_PATH)
    sh = small.c()
    tab = (ctypes.c_void_p * 2)(fake, fake)
    need = mdc.mdc_combine_workspace(small)
    assert need > 0
    st = lib.mdc_combine(ctypes.byref(sh), tab, tab, tab, ctypes.c_void_p(fake), ctypes.c_void_p(fake),
                         ctypes.c_void_p(fake), None, None, None, None, ctypes.c_void_p(fake), ctypes.c_void_p(fake),
                         ctypes.c_void_p(fake), ctypes.c_size_t(need - 1), None)
    assert st == mdc.MDC_ERR_WORKSPACE


# ---- the binding checks dtypes and sizes before it marshals (CPU tensors: nothing is launched) ----

TINY = mdc.Shape(world=2, rank=0, bs=8, hidden=64, topk=2, num_experts=4, capacity=32)


def _tiny_dispatch_args(**over):
    import torch
    W, BS, K, H, A, L = 2, 8, 2, 64, 32, 2
    a = dict(x=torch.zeros((W, BS, H), dtype=torch.bfloat16), expert_ids=torch.zeros((W, BS, K), dtype=torch.int32),
             x_active_mask=None, expand_x=torch.zeros((A, H), dtype=torch.bfloat16),
             assist_info=torch.zeros((A, 3), dtype=torch.int32), ep_recv_counts=torch.zeros(L * W, dtype=torch.int32),
             expert_token_nums=torch.zeros(L, dtype=torch.int64),
             expanded_row_idx=torch.zeros((W, BS, K), dtype=torch.int32),
             workspace=torch.zeros(mdc.mdc_dispatch_workspace(TINY), dtype=torch.uint8))
    a.update(over)
    return a


@pytest.mark.parametrize("name,bad", [
    ("x", ("shape", (2, 8, 63))), ("x", ("dtype", "float32")), ("expert_ids", ("dtype", "int64")),
    ("expert_ids", ("shape", (2, 8, 1))), ("expand_x", ("shape", (31, 64))), ("assist_info", ("shape", (32, 2))),
    ("ep_recv_counts", ("shape", (3,))), ("expert_token_nums", ("dtype", "int32")),
    ("expanded_row_idx", ("shape", (2, 8, 1))), ("x_active_mask", ("shape", (2, 7))),
])
def test_binding_rejects_wrong_dtype_or_size(name, bad):
    import torch
    kind, v = bad
    a = _tiny_dispatch_args()
    ref = a[name] if a[name] is not None else torch.zeros((2, 8), dtype=torch.uint8)
    if kind == "shape":
        t = torch.zeros(v, dtype=ref.dtype)
    else:
        t = torch.zeros(ref.shape, dtype=getattr(torch, v))
    a[name] = t
    with pytest.raises(ValueError):
        mdc.prepare_dispatch(TINY, **a)


def test_binding_rejects_undersized_combine_and_ffn_tensors():
    import torch
    W, BS, K, H, A, L = 2, 8, 2, 64, 32, 2
    ys = [torch.zeros((A, H), dtype=torch.bfloat16) for _ in range(W)]
    ai = [torch.zeros((A, 3), dtype=torch.int32) for _ in range(W)]
    ep = [torch.zeros(L * W, dtype=torch.int32) for _ in range(W)]
    row = torch.zeros((BS, K), dtype=torch.int32)
    ids = torch.zeros((BS, K), dtype=torch.int32)
    sc = torch.zeros((BS, K), dtype=torch.float32)
    out = torch.zeros((BS, H), dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        mdc.prepare_combine(TINY, ys, ai, ep, row, ids, sc.double(), None, None, out)
    with pytest.raises(ValueError):
        mdc.prepare_combine(TINY, ys, ai, ep, row, ids, sc, None, None, out[:-1])
    with pytest.raises(ValueError):
        mdc.prepare_combine(TINY, ys[:1], ai, ep, row, ids, sc, None, None, out)
    with pytest.raises(ValueError):
        mdc.prepare_combine(TINY, ys, ai, ep, row, ids, sc, None, None, out,
                            performance_info=torch.zeros(W, dtype=torch.int32))
    fs = mdc.Shape(world=2, rank=0, bs=8, hidden=128, topk=2, num_experts=4, capacity=32)
    N = 256
    w1 = torch.zeros((L, N, 128), dtype=torch.int8)
    with pytest.raises(ValueError):
        mdc.prepare_ffn(fs, N, torch.zeros((32, 128), dtype=torch.bfloat16), torch.zeros(L, dtype=torch.int64),
                        w1[:, :-1], torch.zeros((L, N)), torch.zeros((L, 128, N // 2), dtype=torch.int8),
                        torch.zeros((L, 128)), torch.zeros((32, 128), dtype=torch.bfloat16), 0)


def test_probe_library_exports_every_declared_symbol():
    """libmdc_probe.so (the benchmark's memory-ceiling probes) exports what include/mdc_probe.h declares."""
    from combine_route_histogram_amd import probe
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "mdc_probe.h")).read(), flags=re.S)
    declared = set(re.findall(r"\b(mdc_probe_[a-z_0-9]+)\s*\(", src))
    assert declared == set(probe.EXPORTS)
    lib = ctypes.CDLL(probe.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_probe_argument_errors():
    """Probe calls reject NULL pointers and sizes that are not multiples of 16 without launching."""
    from combine_route_histogram_amd import probe
    lib = probe._lib
    fake = 1 << 20
    assert lib.mdc_probe_read(None, 16, fake, None) == 2
    assert lib.mdc_probe_write(fake, 17, 0, None) == 2
    assert lib.mdc_probe_copy(fake, None, 16, None) == 2
    assert lib.mdc_probe_rows_reduce(fake, fake, 17, fake, fake, 4, 64, None) == 2
    assert lib.mdc_probe_rows_read(fake, fake, 4, 12, fake, None) == 2


def test_every_header_is_covered_by_an_export_test():
    headers = sorted(f for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h"))
    assert headers == ["mdc.h", "mdc_probe.h"]
