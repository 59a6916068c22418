"""GPU parity of the grouped int8 expert FFN (mdc_ffn) against the CPU oracle.

The FFN is not bit-exact (fp32 epilogues on the GPU, float64 in the oracle;
bf16 intermediate g): the bar is relative L2 error <= 2e-2 over all rows.
"""
import os
import sys

import numpy as np
import pytest
import torch

from oracle import mdc_oracle as O
from workloads import gen

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import combine_route_histogram_amd as mdc  # noqa: E402
from tests import gpu_harness as G  # noqa: E402

REL_L2 = 2e-2


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_l2(got_bits, want_bits):
    a = O.bf16_to_f32(got_bits).astype(np.float64)
    b = O.bf16_to_f32(want_bits).astype(np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def _weights_dev(fw):
    d = G.DEV
    return (torch.from_numpy(fw.w1).to(d), torch.from_numpy(fw.w1_scale).to(d),
            torch.from_numpy(fw.w2).to(d), torch.from_numpy(fw.w2_scale).to(d))


def _run_ffn(w, inter, capacity=None, mask=None, rank=0):
    cap = w.capacity if capacity is None else capacity
    wi = gen.world_inputs(w)
    if mask is not None:
        wi.mask = mask
    fw = gen.ffn_weights(w, rank=rank, inter=inter)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, cap)
    gw = G.dispatch_world(shape, wi.x, wi.ids, wi.mask)
    o = gw.outs[rank]
    y = torch.empty_like(o["expand_x"])
    ws = torch.empty(mdc.mdc_ffn_workspace_size(shape.with_rank(rank), inter), dtype=torch.uint8, device=G.DEV)
    w1, s1, w2, s2 = _weights_dev(fw)
    mdc.mdc_ffn(shape.with_rank(rank), inter, o["expand_x"], o["expert_token_nums"], w1, s1, w2, s2, y, ws)
    torch.cuda.synchronize()
    ref = O.dispatch(wi.x, wi.ids, wi.mask, rank, w.experts, cap)
    n = ref.assist_info.shape[0]
    row_expert = np.repeat(np.arange(w.local_experts), ref.expert_token_nums)[:n]
    want = O.ffn(ref.expand_x, row_expert, fw.w1, fw.w1_scale, fw.w2, fw.w2_scale)
    got = G.bits(y[:n])
    return got, want, gw, wi, fw, y


@pytest.mark.parametrize("variant", [
    dict(world=2, bs=64, hidden=256, experts=4, topk=2, inter=512),
    dict(world=1, bs=300, hidden=384, experts=3, topk=2, inter=256),      # ragged tiles, 3 experts
    dict(world=4, bs=96, hidden=128, experts=16, topk=3, inter=768),
    dict(world=1, bs=700, hidden=256, experts=37, topk=3, inter=512),     # 37 experts, one partial tile each
    dict(world=1, bs=128, hidden=128, experts=2048, topk=16, inter=256),  # max L: 2048 experts of ~1 row
    dict(world=8, bs=256, hidden=256, experts=128, topk=8, inter=512, routing="zipf"),  # skewed expert loads
])
def test_ffn_small(variant):
    inter = variant.pop("inter")
    w = gen.workload("tiny", index=80 + inter // 256, **variant)
    say(f"ffn case W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N={inter}")
    got, want, *_ = _run_ffn(w, inter)
    err = rel_l2(got, want)
    say(f"  rel L2 {err:.3e}")
    assert err <= REL_L2


@pytest.mark.parametrize("bs", [2500, 4700])
def test_ffn_experts_with_several_tile_chunks(bs):
    """Both experts receive every token: bs rows each, 10 or 19 m-tiles, cut
    into chunks of 5 + 5 or 7 + 6 + 6 m-tiles.  H = N = 2048 give both GEMMs
    8 n-tiles, more than one n-group of a chunk holds (6, 4 or 5), so the walk
    crosses chunk and n-group boundaries.  Every row is checked on its own:
    a tile the walk skipped or sent to the wrong rows shows there."""
    w = gen.workload("tiny", world=1, bs=bs, hidden=2048, experts=2, topk=2, index=95)
    say(f"ffn case W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N=2048")
    got, want, *_ = _run_ffn(w, 2048)
    assert got.shape[0] == 2 * bs
    err = rel_l2(got, want)
    a = O.bf16_to_f32(got).astype(np.float64)
    b = O.bf16_to_f32(want).astype(np.float64)
    row_err = np.linalg.norm(a - b, axis=1) / np.maximum(np.linalg.norm(b, axis=1), 1e-30)
    say(f"  rel L2 {err:.3e}, worst row {row_err.max():.3e}")
    assert err <= REL_L2
    assert row_err.max() <= 3 * REL_L2


def test_ffn_hidden_past_the_quantiser_row_cache():
    """H = 8320: 1040 vectors per row, more than the x quantiser keeps in
    registers (1024), so it streams each row twice; 65 k stages per GMM1 tile."""
    w = gen.workload("tiny", world=1, bs=96, hidden=8320, experts=2, topk=2, index=97)
    say(f"ffn case W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N=256")
    got, want, *_ = _run_ffn(w, 256)
    err = rel_l2(got, want)
    say(f"  rel L2 {err:.3e}")
    assert err <= REL_L2


def test_ffn_empty_expert_and_overflow():
    """Every route goes to experts 0..K-1 (A2 sample routing): other experts are empty; capacity cuts the tail."""
    w = gen.workload("tiny", world=2, bs=200, hidden=256, experts=8, topk=2, routing="first_k", index=85)
    got, want, gw, *_ = _run_ffn(w, 256, capacity=300)
    assert got.shape[0] == 300
    err = rel_l2(got, want)
    say(f"  rel L2 {err:.3e}")
    assert err <= REL_L2


def test_ffn_full_size_then_combine():
    """The FFN workload: one GPU's share routing, int8 GMM1 7168 -> 4096, SwiGLU, GMM2 2048 -> 7168, then combine."""
    w = gen.workload("ffn")
    say("ffn full size: generating inputs and weights")
    got, want, gw, wi, fw, y = _run_ffn(w, w.inter)
    err = rel_l2(got, want)
    say(f"  FFN rel L2 {err:.3e} over {got.shape[0]} rows")
    assert err <= REL_L2
    # combine rank 0 with the FFN outputs of destination 0 and the identity elsewhere
    ys = [y] + [o["expand_x"] for o in gw.outs[1:]]
    out = G.bits(G.run_combine(gw, ys, 0, wi.scales[0], wi.shared[0]))
    segs = [O.dispatch(wi.x, wi.ids, None, d, w.experts, w.capacity) for d in range(w.world)]
    oys = [want] + [s.expand_x for s in segs[1:]]
    ref = O.combine(oys, [s.assist_info for s in segs], 0, wi.ids[0], None, wi.scales[0], wi.shared[0], w.hidden)
    err2 = rel_l2(out, ref)
    say(f"  combine after FFN rel L2 {err2:.3e}")
    assert err2 <= REL_L2


@pytest.mark.parametrize("pipeline", ["0", "1"])
def test_ffn_tile_table_in_global_memory(pipeline):
    """A capacity of 400000 rows bounds the m-tile table above the 1536 entries
    the persistent GEMMs cache in LDS: they read it from global memory."""
    w = gen.workload("tiny", world=2, bs=64, hidden=128, experts=4, topk=2, index=90)
    old = os.environ.get("MDC_FFN_PIPELINE")
    try:
        os.environ["MDC_FFN_PIPELINE"] = pipeline
        got, want, *_ = _run_ffn(w, 256, capacity=400_000)
    finally:
        if old is None:
            os.environ.pop("MDC_FFN_PIPELINE", None)
        else:
            os.environ["MDC_FFN_PIPELINE"] = old
    err = rel_l2(got, want)
    say(f"  pipeline={pipeline} rel L2 {err:.3e} over {got.shape[0]} rows")
    assert err <= REL_L2


@pytest.mark.parametrize("variant", [
    dict(world=4, bs=96, hidden=128, experts=16, topk=3, inter=768),
    dict(world=1, bs=128, hidden=128, experts=2048, topk=16, inter=256),
    dict(world=8, bs=2048, hidden=7168, experts=128, topk=8, inter=4096),
])
def test_ffn_pipeline_equals_stream_ordered_kernels(variant):
    """The persistent GMM1 -> quantise -> GMM2 kernel (ready flags between the
    GEMMs) gives y bit-identical to the three stream-ordered kernels."""
    v = dict(variant)
    inter = v.pop("inter")
    name = "share" if v.get("bs") == 2048 else "tiny"
    w = gen.workload(name, **({} if name == "share" else dict(index=80 + inter // 256, **v)))
    say(f"ffn pipeline vs kernels W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N={inter}")
    wi = gen.world_inputs(w)
    fw = gen.ffn_weights(w, rank=0, inter=inter)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity)
    gw = G.dispatch_world(shape, wi.x, wi.ids, wi.mask)
    o = gw.outs[0]
    w1, s1, w2, s2 = _weights_dev(fw)
    ws = torch.empty(mdc.mdc_ffn_workspace_size(shape, inter), dtype=torch.uint8, device=G.DEV)
    ys = []
    old = os.environ.get("MDC_FFN_PIPELINE")
    try:
        for flag in ("1", "0", "1"):
            os.environ["MDC_FFN_PIPELINE"] = flag
            y = torch.zeros_like(o["expand_x"])
            mdc.mdc_ffn(shape, inter, o["expand_x"], o["expert_token_nums"], w1, s1, w2, s2, y, ws)
            torch.cuda.synchronize()
            ys.append(y)
    finally:
        if old is None:
            os.environ.pop("MDC_FFN_PIPELINE", None)
        else:
            os.environ["MDC_FFN_PIPELINE"] = old
    n = int(o["ep_recv_counts"][-1].item())
    n = min(n, w.capacity)
    assert n > 0
    a, b, c = (t[:n].view(torch.int16) for t in ys)
    assert torch.equal(a, b), f"pipeline vs kernels: {(a != b).sum().item()} values differ"
    assert torch.equal(a, c), "pipeline not repeatable"
    say(f"  y bit-identical over {n} rows")
