"""HIP graph capture of the decode-size step (one-shot mdc_dispatch, then
mdc_combine): the captured graph is replayed several times, with eager work
between the replays, and every replay's outputs must equal the eager run's
bit for bit (and the oracle's).  The kernels issue no memset, so the graph
holds kernel nodes only.
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
