"""GPU parity of the grouped int8 expert FFN (mdc_ffn) against the CPU oracle.

The FFN is not bit-exact (fp32 epilogues on the GPU, float64 in the oracle;
bf16 intermediate g): the bar is relative L2 error <= 2e-2 over all rows.
"""
import sys
from dataclasses import replace

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


def _run_ffn(w, inter, capacity=None, mask=None, rank=0, flags=0):
    cap = w.capacity if capacity is None else capacity
    wi = gen.world_inputs(w)
    if mask is not None:
        wi.mask = mask
    fw = gen.ffn_weights(w, rank=rank, inter=inter)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, cap, flags=flags)
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


@pytest.mark.parametrize("hidden", [384, 256])
def test_ffn_tail_rows_ride_along(hidden):
    """Expert loads chosen around the tail rule of the stream-ordered GEMMs:
    an expert with n rows whose tail n % 256 is at most 32 per full 256-row
    m-tile spreads it over its first full m-tiles, 32 rows each; a longer
    tail keeps an m-tile of its own.  Counts: 0, 1, 33 (no full m-tile),
    256 (no tail), 288 (tail 32 on one m-tile), 289 (tail 33: own m-tile),
    544 (tail 32 on two m-tiles), 576 (tail 64: 32 + 32), 577 (tail 65: own
    m-tile).  H = 384 leaves GMM2's last n-tile half full (the extra rows'
    column check) and gives GMM1 an odd number of k stages.  The fused
    pipeline keeps every tail in an m-tile of its own, so its y must be
    bit-identical; both are checked against the oracle row by row."""
    counts = [0, 1, 33, 256, 288, 289, 544, 576, 577]
    L, inter = len(counts), 512
    w = gen.workload("tiny", world=1, bs=64, hidden=hidden, experts=L, topk=2, index=98)
    n = sum(counts)
    cap = n + 64
    say(f"ffn tail rows H={hidden} N={inter} counts={counts}")
    x = gen.normal_bf16(gen.rng(w.index, 0, "x"), (cap, hidden))
    fw = gen.ffn_weights(w, rank=0, inter=inter)
    w1, s1, w2, s2 = _weights_dev(fw)
    shape = mdc.Shape(1, 0, w.bs, hidden, 2, L, cap)
    xd = torch.from_numpy(x.view(np.int16)).to(G.DEV).view(torch.bfloat16)
    nums = torch.tensor(counts, dtype=torch.int64, device=G.DEV)
    ws = torch.empty(mdc.mdc_ffn_workspace(shape, inter), dtype=torch.uint8, device=G.DEV)
    ys = []
    for flag in (0, mdc.MDC_FLAG_FFN_PIPELINE):
        y = torch.zeros((cap, hidden), dtype=torch.bfloat16, device=G.DEV)
        mdc.mdc_ffn(replace(shape, flags=flag), inter, xd, nums, w1, s1, w2, s2, y, ws)
        torch.cuda.synchronize()
        assert mdc.read_status(ws)["wait_timeouts"] == 0
        ys.append(y)
    a, b = (t[:n].view(torch.int16) for t in ys)
    assert torch.equal(a, b), f"stream-ordered vs pipeline: {(a != b).sum().item()} values differ"
    assert not torch.any(ys[0][n:].view(torch.int16) != 0), "rows past the experts' rows were written"
    row_expert = np.repeat(np.arange(L), counts)
    want = O.ffn(x[:n], row_expert, fw.w1, fw.w1_scale, fw.w2, fw.w2_scale)
    got = G.bits(ys[0][:n])
    af = O.bf16_to_f32(got).astype(np.float64)
    bf = O.bf16_to_f32(want).astype(np.float64)
    row_err = np.linalg.norm(af - bf, axis=1) / np.maximum(np.linalg.norm(bf, axis=1), 1e-30)
    err = rel_l2(got, want)
    say(f"  bit-identical to the pipeline; rel L2 {err:.3e}, worst row {row_err.max():.3e}")
    assert err <= REL_L2
    assert row_err.max() <= 3 * REL_L2


@pytest.mark.parametrize("capacity", [300_000, 400_000])
@pytest.mark.parametrize("pipeline", [0, 1])
def test_ffn_tile_table_in_global_memory(pipeline, capacity):
    """A capacity of 400000 rows bounds the m-tile table above the 1536
    entries the fused kernel caches in LDS and the 1024 the stream-ordered
    GEMMs cache: both read it from global memory.  At 300000 rows (a bound of
    1177 entries) the GEMMs read it from global memory and the fused kernel
    from LDS."""
    w = gen.workload("tiny", world=2, bs=64, hidden=128, experts=4, topk=2, index=90)
    got, want, *_ = _run_ffn(w, 256, capacity=capacity, flags=mdc.MDC_FLAG_FFN_PIPELINE if pipeline else 0)
    err = rel_l2(got, want)
    say(f"  pipeline={pipeline} capacity={capacity} rel L2 {err:.3e} over {got.shape[0]} rows")
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
    ws = torch.empty(mdc.mdc_ffn_workspace(shape, inter), dtype=torch.uint8, device=G.DEV)
    ys = []
    for flag in (mdc.MDC_FLAG_FFN_PIPELINE, 0, mdc.MDC_FLAG_FFN_PIPELINE):
        y = torch.zeros_like(o["expand_x"])
        ws[:16].fill_(0x7F)   # the call must rewrite its status block
        mdc.mdc_ffn(replace(shape, flags=flag), inter, o["expand_x"], o["expert_token_nums"], w1, s1, w2, s2, y, ws)
        torch.cuda.synchronize()
        st = mdc.read_status(ws)
        assert st["wait_timeouts"] == 0, st      # no pipeline wait ran out of its bound
        assert st["dropped_ids"] == 0 and st["overflow_rows"] == 0, st
        ys.append(y)
    n = int(o["ep_recv_counts"][-1].item())
    n = min(n, w.capacity)
    assert n > 0
    a, b, c = (t[:n].view(torch.int16) for t in ys)
    assert torch.equal(a, b), f"pipeline vs kernels: {(a != b).sum().item()} values differ"
    assert torch.equal(a, c), "pipeline not repeatable"
    say(f"  y bit-identical over {n} rows")


def test_ffn_pipeline_wait_timeout_is_reported():
    """A bounded wait that runs out is reported, never silent.  The spin field
    of the flags lets each GMM2 tile poll its ready flag at most twice
    (2^1 polls): tiles whose rows of g are not quantised by then give up,
    count themselves in the status block's wait_timeouts and write NaN rows.
    Every kernel still exits; the tiles whose flag was set in time match the
    stream-ordered result bit for bit."""
    w = gen.workload("tiny", world=2, bs=512, hidden=1024, experts=4, topk=2, index=98)
    inter = 2048
    say(f"ffn pipeline forced time-out W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N={inter}")
    wi = gen.world_inputs(w)
    fw = gen.ffn_weights(w, rank=0, inter=inter)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity)
    gw = G.dispatch_world(shape, wi.x, wi.ids, wi.mask)
    o = gw.outs[0]
    w1, s1, w2, s2 = _weights_dev(fw)
    ws = torch.empty(mdc.mdc_ffn_workspace(shape, inter), dtype=torch.uint8, device=G.DEV)
    n = min(int(o["ep_recv_counts"][-1].item()), w.capacity)
    y_ref = torch.zeros_like(o["expand_x"])
    mdc.mdc_ffn(shape, inter, o["expand_x"], o["expert_token_nums"], w1, s1, w2, s2, y_ref, ws)
    y = torch.zeros_like(o["expand_x"])
    quick = mdc.MDC_FLAG_FFN_PIPELINE | (1 << mdc.MDC_FLAG_SPIN_SHIFT)
    mdc.mdc_ffn(replace(shape, flags=quick), inter, o["expand_x"], o["expert_token_nums"], w1, s1, w2, s2, y, ws)
    torch.cuda.synchronize()
    st = mdc.read_status(ws)
    a = y[:n].view(torch.int16)
    nan_rows = torch.isnan(y[:n].float()).any(dim=1)
    say(f"  wait_timeouts {st['wait_timeouts']}, rows with NaN {int(nan_rows.sum())} of {n}")
    assert st["wait_timeouts"] > 0
    assert int(nan_rows.sum()) > 0
    # a poisoned tile is NaN in all its values; every other value equals the stream-ordered result
    fine = ~torch.isnan(y[:n].float())
    assert torch.equal(a[fine], y_ref[:n].view(torch.int16)[fine])
    # the default wait bound: nothing runs out, and the status block is rewritten by the next call
    mdc.mdc_ffn(replace(shape, flags=mdc.MDC_FLAG_FFN_PIPELINE), inter, o["expand_x"], o["expert_token_nums"],
                w1, s1, w2, s2, y, ws)
    torch.cuda.synchronize()
    assert mdc.read_status(ws)["wait_timeouts"] == 0
    assert torch.equal(y[:n].view(torch.int16), y_ref[:n].view(torch.int16))


def test_ffn_bench_composition_full_size():
    """The ffn step as timed: quantised dispatch (mdc_dispatch_layout +
    mdc_dispatch_quant_gather) -> mdc_ffn_quant_input -> mdc_combine, at the
    full ffn shape, against the oracle (dispatch -> ffn -> combine) on y and
    on xOut."""
    w = gen.workload("ffn")
    say("ffn bench composition, full size: generating inputs and weights")
    wi = gen.world_inputs(w)
    fw = gen.ffn_weights(w, rank=0)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity)
    gw = G.dispatch_world(shape, wi.x, wi.ids, wi.mask)       # every destination's bf16 rows (identity elsewhere)
    o = gw.outs[0]
    q = torch.empty((w.capacity, w.hidden), dtype=torch.int8, device=G.DEV)
    qs = torch.empty((w.capacity,), dtype=torch.float32, device=G.DEV)
    ws = torch.empty(mdc.mdc_dispatch_workspace(shape), dtype=torch.uint8, device=G.DEV)
    ai = torch.empty_like(o["assist_info"])
    ep = torch.empty_like(o["ep_recv_counts"])
    etn = torch.empty_like(o["expert_token_nums"])
    row_idx = gw.row_idx.clone()
    mdc.mdc_dispatch_layout(shape, gw.ids, gw.mask, ws)
    mdc.mdc_dispatch_quant_gather(shape, gw.x, q, qs, ai, ep, etn, row_idx, ws)
    w1, s1, w2, s2 = _weights_dev(fw)
    fws = torch.empty(mdc.mdc_ffn_workspace(shape, w.inter), dtype=torch.uint8, device=G.DEV)
    y = torch.empty((w.capacity, w.hidden), dtype=torch.bfloat16, device=G.DEV)
    mdc.mdc_ffn_quant_input(shape, w.inter, q, qs, etn, w1, s1, w2, s2, y, fws)
    torch.cuda.synchronize()
    ref = O.dispatch(wi.x, wi.ids, wi.mask, 0, w.experts, w.capacity)
    n = ref.assist_info.shape[0]
    assert np.array_equal(ai[:n].cpu().numpy(), ref.assist_info)
    assert np.array_equal(row_idx.cpu().numpy(), gw.row_idx.cpu().numpy())
    row_expert = np.repeat(np.arange(w.local_experts), ref.expert_token_nums)[:n]
    want = O.ffn(ref.expand_x, row_expert, fw.w1, fw.w1_scale, fw.w2, fw.w2_scale)
    err = rel_l2(G.bits(y[:n]), want)
    say(f"  y rel L2 {err:.3e} over {n} rows")
    assert err <= REL_L2
    ys = [y] + [oo["expand_x"] for oo in gw.outs[1:]]
    aid = [ai] + [oo["assist_info"] for oo in gw.outs[1:]]
    epd = [ep] + [oo["ep_recv_counts"] for oo in gw.outs[1:]]
    out = torch.empty((w.bs, w.hidden), dtype=torch.bfloat16, device=G.DEV)
    mdc.mdc_combine(shape, ys, aid, epd, row_idx[0].contiguous(), gw.ids[0].contiguous(),
                    torch.from_numpy(wi.scales[0]).to(G.DEV), None, G.to_dev_bf16(wi.shared[0]), out)
    torch.cuda.synchronize()
    segs = [O.dispatch(wi.x, wi.ids, None, d, w.experts, w.capacity) for d in range(w.world)]
    oys = [want] + [sg.expand_x for sg in segs[1:]]
    xo = O.combine(oys, [sg.assist_info for sg in segs], 0, wi.ids[0], None, wi.scales[0], wi.shared[0], w.hidden)
    err2 = rel_l2(G.bits(out), xo)
    say(f"  xOut rel L2 {err2:.3e}")
    assert err2 <= REL_L2
