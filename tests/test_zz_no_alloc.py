"""mdc_dispatch_noalloc (the dispatch whose workspace is the library's static
device array, for callers that cannot allocate) against mdc_dispatch with a
caller workspace: every output bit-exact, on two calls in a row, the second
with a smaller input than the first; and the size limit.
"""
import ctypes
import sys

import numpy as np
import pytest
import torch

from workloads import gen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_route_histogram_amd as mdc  # noqa: E402
from tests import gpu_harness as G  # noqa: E402


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _outputs(shape, dev):
    o = mdc.alloc_dispatch_outputs(shape, dev)
    for k in ("expand_x", "assist_info", "ep_recv_counts", "expert_token_nums"):
        o[k].zero_()
    o["expand_scales"] = torch.zeros((shape.capacity,), dtype=torch.float32, device=dev)
    return o


def _run_pair(w, d, lib_call_noalloc):
    """Dispatch for destination d twice, with a caller workspace and without; compare everything."""
    wi = gen.world_inputs(w)
    shape = mdc.Shape(w.world, d, w.bs, w.hidden, w.topk, w.experts, w.capacity,
                      mask_per_route=1 if w.route_mask_frac > 0 else 0)
    x = G.to_dev_bf16(wi.x)
    ids = torch.from_numpy(wi.ids).to(G.DEV)
    mask = None if wi.mask is None else torch.from_numpy(wi.mask).to(G.DEV)
    sc = torch.from_numpy(wi.scales).to(G.DEV)
    ref, got = _outputs(shape, G.DEV), _outputs(shape, G.DEV)
    row_ref = torch.full((w.world, w.bs, w.topk), -2, dtype=torch.int32, device=G.DEV)
    row_got = row_ref.clone()
    mdc.mdc_dispatch(shape, x, ids, mask, ref["expand_x"], ref["assist_info"], ref["ep_recv_counts"],
                     ref["expert_token_nums"], row_ref, ref["workspace"], expert_scales=sc,
                     expand_scales=ref["expand_scales"])
    lib_call_noalloc(shape, x, ids, mask, sc, got, row_got)
    torch.cuda.synchronize()
    n = min(int(ref["ep_recv_counts"][-1].item()), w.capacity)
    assert n > 0
    for k in ("ep_recv_counts", "expert_token_nums"):
        assert torch.equal(ref[k], got[k]), k
    assert torch.equal(ref["assist_info"][:n], got["assist_info"][:n])
    assert torch.equal(ref["expand_x"][:n].view(torch.int16), got["expand_x"][:n].view(torch.int16))
    assert torch.equal(ref["expand_scales"][:n].view(torch.int32), got["expand_scales"][:n].view(torch.int32))
    assert torch.equal(row_ref, row_got)
    say(f"  W={w.world} BS={w.bs} d={d}: {n} rows identical to mdc_dispatch")


def _via_c_abi(shape, x, ids, mask, sc, o, row_idx):
    """The no-alloc entry point called through ctypes with plain pointers (no workspace argument)."""
    lib = ctypes.CDLL(mdc.LIB_PATH)
    fn = lib.mdc_dispatch_noalloc
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 12
    sh = shape.c()
    P = lambda t: None if t is None else t.data_ptr()  # noqa: E731
    st = fn(ctypes.byref(sh), P(x), P(ids), P(mask), P(sc), P(o["expand_x"]), P(o["assist_info"]),
            P(o["ep_recv_counts"]), P(o["expert_token_nums"]), P(row_idx), P(o["expand_scales"]),
            torch.cuda.current_stream().cuda_stream)
    assert st == mdc.MDC_OK, mdc.mdc_status_string(st)


def test_noalloc_matches_dispatch_two_calls_second_smaller():
    # first call: the share shape (rank kernel + gather kernel, 0.53 MB of scratch);
    # second: a decode-size batch (the one-launch path), smaller in every dimension
    say("no-alloc dispatch: share shape, then decode shape")
    _run_pair(gen.workload("share"), 0, _via_c_abi)
    _run_pair(gen.workload("decode"), 3, _via_c_abi)


def test_noalloc_second_call_smaller_after_skewed_and_masked():
    say("no-alloc dispatch: skewed (masked) share shape, then a small ragged world")
    _run_pair(gen.workload("skewed"), 0, _via_c_abi)
    _run_pair(gen.workload("tiny", world=3, bs=101, hidden=136, experts=9, topk=3, inactive_frac=0.2, index=99), 2,
              lambda sh, x, ids, mask, sc, o, row: mdc.mdc_dispatch_noalloc(
                  sh, x, ids, mask, o["expand_x"], o["assist_info"], o["ep_recv_counts"], o["expert_token_nums"],
                  row, expert_scales=sc, expand_scales=o["expand_scales"]))


def test_noalloc_rejects_shapes_past_its_scratch():
    # 8 x 16384 tokens x top-16: 2M routes, 8 MiB of route ranks alone
    big = mdc.Shape(world=8, rank=0, bs=16384, hidden=128, topk=16, num_experts=128, capacity=1)
    assert mdc.mdc_dispatch_workspace(big) > mdc.MDC_NOALLOC_SCRATCH_BYTES
    fake = 1 << 20
    lib = ctypes.CDLL(mdc.LIB_PATH)
    fn = lib.mdc_dispatch_noalloc
    fn.restype = ctypes.c_int
    fn.argtypes = [ctypes.c_void_p] * 12
    sh = big.c()
    st = fn(ctypes.byref(sh), fake, fake, None, None, fake, fake, fake, fake, fake, None, None)
    assert st == mdc.MDC_ERR_UNSUPPORTED
