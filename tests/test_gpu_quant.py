"""GPU parity of the quantised dispatch (int8 rows + per-row scales) and of the
FFN fed with them.

Codes and scales are decided in fp32 by the same rule on both sides, so they
are compared bit-exactly, as are triplets, counts and the inverse index.
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


def _quant_world(w, capacity=None, split=False):
    cap = w.capacity if capacity is None else capacity
    wi = gen.world_inputs(w)
    shape = mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, cap,
                      mask_per_route=1 if w.route_mask_frac > 0 else 0)
    xd = G.to_dev_bf16(wi.x)
    idd = torch.from_numpy(wi.ids).to(G.DEV)
    md = None if wi.mask is None else torch.from_numpy(wi.mask).to(G.DEV)
    row_idx = torch.full((w.world, w.bs, w.topk), -2, dtype=torch.int32, device=G.DEV)
    outs = []
    for d in range(w.world):
        sh = shape.with_rank(d)
        o = mdc.alloc_dispatch_outputs(sh, G.DEV)
        o["expand_q"] = torch.empty((cap, w.hidden), dtype=torch.int8, device=G.DEV)
        o["scales"] = torch.empty((cap,), dtype=torch.float32, device=G.DEV)
        if split:
            mdc.mdc_dispatch_layout(sh, idd, md, o["workspace"])
            mdc.mdc_dispatch_quant_gather(sh, xd, o["expand_q"], o["scales"], o["assist_info"],
                                          o["ep_recv_counts"], o["expert_token_nums"], row_idx, o["workspace"])
        else:
            mdc.mdc_dispatch_quant(sh, xd, idd, md, o["expand_q"], o["scales"], o["assist_info"],
                                   o["ep_recv_counts"], o["expert_token_nums"], row_idx, o["workspace"])
        outs.append(o)
    torch.cuda.synchronize()
    return wi, shape, outs, row_idx


@pytest.mark.parametrize("variant", [
    dict(name="tiny"),
    dict(name="decode"),
    dict(name="tiny", world=3, bs=70, hidden=136, experts=9, topk=3, route_mask_frac=0.2, index=93),
    dict(name="tiny", world=2, bs=40, hidden=8192, experts=4, topk=2, index=94),
    dict(name="share"),
])
@pytest.mark.parametrize("split", [False, True], ids=["one_shot", "split_stages"])
def test_dispatch_quant_matches_oracle(variant, split):
    v = dict(variant)
    w = gen.workload(v.pop("name"), **v)
    say(f"quant dispatch W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} split={split}")
    wi, shape, outs, row_idx = _quant_world(w, split=split)
    ridx = row_idx.cpu().numpy()
    for d in range(w.world):
        ref, q, sc = O.dispatch_quant(wi.x, wi.ids, wi.mask, d, w.experts, w.capacity)
        n = ref.assist_info.shape[0]
        o = outs[d]
        assert np.array_equal(o["ep_recv_counts"].cpu().numpy(), ref.ep_recv_counts)
        assert np.array_equal(o["expert_token_nums"].cpu().numpy(), ref.expert_token_nums)
        assert np.array_equal(o["assist_info"][:n].cpu().numpy(), ref.assist_info)
        assert np.array_equal(o["expand_q"][:n].cpu().numpy(), q), f"codes d={d}"
        assert np.array_equal(o["scales"][:n].cpu().numpy().view(np.uint32), sc.view(np.uint32)), f"scales d={d}"
        for (s, t, k), row in ref.expanded_row_idx.items():
            assert ridx[s, t, k] == row


def test_ffn_on_quantised_rows_equals_bf16_path():
    """Codes from the quantised dispatch equal mdc_ffn's own quantiser, so y is identical."""
    w = gen.workload("tiny", world=2, bs=96, hidden=256, experts=4, topk=2, index=95)
    inter = 512
    wi, shape, outs, _ = _quant_world(w)
    gw = G.dispatch_world(mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity), wi.x, wi.ids, None)
    fw = gen.ffn_weights(w, rank=0, inter=inter)
    dev = G.DEV
    w1, s1, w2, s2 = (torch.from_numpy(a).to(dev) for a in (fw.w1, fw.w1_scale, fw.w2, fw.w2_scale))
    ws = torch.empty(mdc.mdc_ffn_workspace_size(shape, inter), dtype=torch.uint8, device=dev)
    y_a = torch.zeros((w.capacity, w.hidden), dtype=torch.bfloat16, device=dev)
    y_b = torch.zeros_like(y_a)
    mdc.mdc_ffn(shape, inter, gw.outs[0]["expand_x"], gw.outs[0]["expert_token_nums"], w1, s1, w2, s2, y_a, ws)
    mdc.mdc_ffn_quant_input(shape, inter, outs[0]["expand_q"], outs[0]["scales"], outs[0]["expert_token_nums"],
                            w1, s1, w2, s2, y_b, ws)
    torch.cuda.synchronize()
    n = int(outs[0]["ep_recv_counts"][-1].item())
    assert n > 0
    assert torch.equal(y_a[:n].view(torch.int16), y_b[:n].view(torch.int16))
