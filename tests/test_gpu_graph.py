"""HIP graph capture of the decode-size step (one-shot mdc_dispatch, then
mdc_combine) and of the pipelined dispatch + FFN: each captured graph is
replayed several times, with eager work between the replays, and every
replay's outputs must equal the eager run's bit for bit (and the oracle's).
The kernels issue no memset, so the graphs hold kernel nodes only.
"""
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _outputs(o, x_out, row_idx, n):
    return (o["ep_recv_counts"].cpu(), o["expert_token_nums"].cpu(), o["assist_info"][:n].cpu(),
            o["expand_x"][:n].view(torch.int16).cpu(), row_idx.cpu(), x_out.view(torch.int16).cpu())


@pytest.mark.parametrize("name", ["decode", "tiny"])
def test_graph_replays_equal_eager(name):
    w = gen.workload(name)
    say(f"case graph {name} W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk}")
    wi = gen.world_inputs(w)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity)
    gw = G.dispatch_world(shape, wi.x, wi.ids, wi.mask)          # every destination, eager
    ys = [o["expand_x"] for o in gw.outs]                        # identity expert
    sc = torch.from_numpy(wi.scales[0]).to(G.DEV)
    shd = None if wi.shared is None else G.to_dev_bf16(wi.shared[0])
    ids0 = gw.ids[0].contiguous()

    # eager reference: dispatch for destination 0 again into fresh buffers, then combine for source 0
    ref = mdc.alloc_dispatch_outputs(shape, G.DEV)
    ref_row = gw.row_idx.clone()
    mdc.mdc_dispatch(shape, gw.x, gw.ids, gw.mask, ref["expand_x"], ref["assist_info"], ref["ep_recv_counts"],
                     ref["expert_token_nums"], ref_row, ref["workspace"])
    ref_out = torch.empty((w.bs, w.hidden), dtype=torch.bfloat16, device=G.DEV)
    mdc.mdc_combine(shape, [ref["expand_x"]] + ys[1:], [ref["assist_info"]] + [o["assist_info"] for o in gw.outs[1:]],
                    [ref["ep_recv_counts"]] + [o["ep_recv_counts"] for o in gw.outs[1:]], ref_row[0].contiguous(),
                    ids0, sc, None, shd, ref_out)
    torch.cuda.synchronize()
    n = int(ref["ep_recv_counts"][-1].item())
    want = _outputs(ref, ref_out, ref_row, n)

    # the oracle agrees with the eager reference
    seg = O.dispatch(wi.x, wi.ids, wi.mask, 0, w.experts, w.capacity)
    assert np.array_equal(want[2].numpy(), seg.assist_info)
    segs = [O.dispatch(wi.x, wi.ids, wi.mask, d, w.experts, w.capacity) for d in range(w.world)]
    oc = O.combine([s.expand_x for s in segs], [s.assist_info for s in segs], 0, wi.ids[0], None, wi.scales[0],
                   None if wi.shared is None else wi.shared[0], w.hidden)
    assert np.array_equal(want[5].numpy().view(np.uint16), oc)

    # captured: the same two calls on the capture stream, into their own buffers
    cs = torch.cuda.Stream()
    o = mdc.alloc_dispatch_outputs(shape, G.DEV)
    row = gw.row_idx.clone()
    out = torch.empty_like(ref_out)
    dsp = mdc.prepare_dispatch(shape, gw.x, gw.ids, gw.mask, o["expand_x"], o["assist_info"], o["ep_recv_counts"],
                               o["expert_token_nums"], row, o["workspace"], cs)
    row0 = row[0]   # a view: the combine reads what the captured dispatch writes
    cmb = mdc.prepare_combine(shape, [o["expand_x"]] + ys[1:], [o["assist_info"]] + [p["assist_info"] for p in gw.outs[1:]],
                              [o["ep_recv_counts"]] + [p["ep_recv_counts"] for p in gw.outs[1:]], row0, ids0, sc, None,
                              shd, out, stream=cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        dsp()
        cmb()
    torch.cuda.synchronize()
    # inverse-index entries that dispatch 0 writes: every source's routes to a local expert of rank 0
    L = w.experts // w.world
    sent0 = torch.from_numpy((wi.ids >= 0) & (wi.ids < w.experts) & (wi.ids // L == 0)).to(G.DEV)
    for rep in range(3):
        # eager work between the replays: scramble every output the graph writes
        o["expand_x"].view(torch.int16).fill_(-1)
        o["assist_info"].fill_(-7)
        o["ep_recv_counts"].fill_(-3)
        o["expert_token_nums"].fill_(-5)
        row.masked_fill_(sent0, -9)
        out.view(torch.int16).fill_(0x7F00)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = _outputs(o, out, row, n)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager run"
        say(f"  replay {rep}: bit-exact")


def test_graph_replays_of_the_dispatch_ffn_pipeline():
    """The pipelined dispatch + FFN (mdc_dispatch_layout, then mdc_dispatch_ffn:
    plan, route placement and the persistent kernel, whose synchronisation
    words the plan kernel clears without a memset) captured once and replayed
    three times, every output scrambled in between: each replay equals the
    eager stream-ordered calls bit for bit."""
    w = gen.workload("tiny", world=4, bs=128, hidden=256, experts=16, topk=4, index=77)
    inter = 512
    say(f"case graph dispatch_ffn W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N={inter}")
    wi = gen.world_inputs(w)
    fw = gen.ffn_weights(w, rank=0, inter=inter)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity)
    d = G.DEV
    x = G.to_dev_bf16(wi.x)
    ids = torch.from_numpy(np.ascontiguousarray(wi.ids)).to(d)
    wts = [torch.from_numpy(a).to(d) for a in (fw.w1, fw.w1_scale, fw.w2, fw.w2_scale)]
    A, H, L, W = shape.capacity, shape.hidden, shape.local_experts, shape.world

    def bufs():
        return dict(q=torch.zeros((A, H), dtype=torch.int8, device=d),
                    qs=torch.zeros((A,), dtype=torch.float32, device=d),
                    assist=torch.zeros((A, 3), dtype=torch.int32, device=d),
                    recv=torch.zeros((L * W,), dtype=torch.int32, device=d),
                    etn=torch.zeros((L,), dtype=torch.int64, device=d),
                    row=torch.full((W, w.bs, w.topk), -1, dtype=torch.int32, device=d),
                    y=torch.zeros((A, H), dtype=torch.bfloat16, device=d),
                    dws=torch.empty(mdc.mdc_dispatch_workspace(shape), dtype=torch.uint8, device=d),
                    fws=torch.empty(mdc.mdc_ffn_workspace(shape, inter), dtype=torch.uint8, device=d))

    ref = bufs()
    mdc.mdc_dispatch_layout(shape, ids, None, ref["dws"])
    mdc.mdc_dispatch_quant_gather(shape, x, ref["q"], ref["qs"], ref["assist"], ref["recv"], ref["etn"], ref["row"],
                                  ref["dws"])
    mdc.mdc_ffn_quant_input(shape, inter, ref["q"], ref["qs"], ref["etn"], *wts, ref["y"], ref["fws"])
    torch.cuda.synchronize()
    n = min(int(ref["etn"].sum().item()), A)
    assert n > 0

    def outputs(b):
        return (b["q"][:n].cpu(), b["qs"][:n].view(torch.int32).cpu(), b["assist"][:n].cpu(), b["recv"].cpu(),
                b["etn"].cpu(), b["row"].cpu(), b["y"][:n].view(torch.int16).cpu())

    want = outputs(ref)
    cs = torch.cuda.Stream()
    o = bufs()
    lay = mdc.prepare_dispatch_layout(shape, ids, None, o["dws"], cs)
    dfn = mdc.prepare_dispatch_ffn(shape, inter, x, o["q"], o["qs"], o["assist"], o["recv"], o["etn"], o["row"],
                                   *wts, o["y"], o["dws"], o["fws"], cs)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        lay()
        dfn()
    torch.cuda.synchronize()
    L0 = w.experts // w.world
    sent0 = torch.from_numpy((wi.ids >= 0) & (wi.ids < w.experts) & (wi.ids // L0 == 0)).to(d)
    for rep in range(3):
        o["q"].fill_(-1)
        o["qs"].fill_(float("nan"))
        o["assist"].fill_(-7)
        o["recv"].fill_(-3)
        o["etn"].fill_(-5)
        o["row"].masked_fill_(sent0, -9)
        o["y"].view(torch.int16).fill_(0x7F00)
        o["fws"][:64].fill_(0x5A)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = outputs(o)
        for i, (a, b) in enumerate(zip(got, want)):
            assert torch.equal(a, b), f"replay {rep}: output {i} differs from the eager stream-ordered calls"
        assert mdc.read_status(o["fws"])["wait_timeouts"] == 0
        say(f"  replay {rep}: bit-exact")
