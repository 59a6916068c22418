"""GPU parity of the pipelined dispatch + FFN (mdc_dispatch_ffn).

Every output must equal, bit for bit, what the stream-ordered calls give on
the same inputs (mdc_dispatch_layout -> mdc_dispatch_quant_gather ->
mdc_ffn_quant_input): the quantised rows and scales, triplets, inverse
index, counts, expand_scales, both status blocks and y.  The dispatch part is
also checked against the oracle's dispatch (bit-exact), and y against the
oracle's FFN (relative L2 <= 2e-2), at small sizes and at the full ffn size.
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


class Inputs:
    """Device copies of one world's inputs and the destination's weights."""

    def __init__(self, w, inter, capacity=None, ids=None, mask_per_route=0, rank=0):
        self.w, self.inter, self.rank = w, inter, rank
        self.wi = gen.world_inputs(w)
        if ids is not None:
            self.wi.ids = ids
        self.cap = w.capacity if capacity is None else capacity
        self.shape = mdc.Shape(w.world, rank, w.bs, w.hidden, w.topk, w.experts, self.cap,
                               mask_per_route=mask_per_route, zero_experts=w.zero_experts,
                               copy_experts=w.copy_experts)
        self.fw = gen.ffn_weights(w, rank=rank, inter=inter)
        d = G.DEV
        W, BS, H = w.world, w.bs, w.hidden
        self.x = G.to_dev_bf16(self.wi.x) if self.wi.x.size else torch.empty((W, BS, H), dtype=torch.bfloat16,
                                                                              device=d)
        self.ids = torch.from_numpy(np.ascontiguousarray(self.wi.ids)).to(d)
        self.mask = None if self.wi.mask is None else torch.from_numpy(
            np.ascontiguousarray(self.wi.mask.astype(np.uint8))).to(d)
        self.scales = torch.from_numpy(np.ascontiguousarray(self.wi.scales, dtype=np.float32)).to(d)
        self.weights = tuple(torch.from_numpy(a).to(d) for a in (self.fw.w1, self.fw.w1_scale, self.fw.w2,
                                                                  self.fw.w2_scale))

    def outputs(self, fill):
        """Fresh output buffers filled with garbage (fill byte), so that unwritten values show."""
        sh, d = self.shape, G.DEV
        A, H, L, W = sh.capacity, sh.hidden, sh.local_experts, sh.world
        o = dict(q=torch.full((A, H), fill, dtype=torch.int8, device=d),
                 qs=torch.full((A,), float(fill), dtype=torch.float32, device=d),
                 assist=torch.full((A, 3), fill, dtype=torch.int32, device=d),
                 recv=torch.full((L * W,), fill, dtype=torch.int32, device=d),
                 etn=torch.full((L,), fill, dtype=torch.int64, device=d),
                 row_idx=torch.full((W, sh.bs, sh.topk), -1, dtype=torch.int32, device=d),
                 esc=torch.full((A,), float(fill), dtype=torch.float32, device=d),
                 y=torch.full((A, H), fill, dtype=torch.int16, device=d).view(torch.bfloat16),
                 dws=torch.empty(mdc.mdc_dispatch_workspace(sh), dtype=torch.uint8, device=d),
                 fws=torch.empty(mdc.mdc_ffn_workspace(sh, self.inter), dtype=torch.uint8, device=d))
        o["dws"][:mdc.MDC_STATUS_BYTES].fill_(0x5A)
        o["fws"][:mdc.MDC_STATUS_BYTES].fill_(0x5A)
        return o

    def run_stream_ordered(self):
        o = self.outputs(0x33)
        sh = self.shape
        mdc.mdc_dispatch_layout(sh, self.ids, self.mask, o["dws"])
        mdc.mdc_dispatch_quant_gather(sh, self.x, o["q"], o["qs"], o["assist"], o["recv"], o["etn"], o["row_idx"],
                                      o["dws"], expert_scales=self.scales, expand_scales=o["esc"])
        mdc.mdc_ffn_quant_input(sh, self.inter, o["q"], o["qs"], o["etn"], *self.weights, o["y"], o["fws"])
        torch.cuda.synchronize()
        return o

    def run_pipelined(self, flags=0, o=None):
        o = self.outputs(0x33) if o is None else o
        sh = replace(self.shape, flags=flags)
        mdc.mdc_dispatch_layout(sh, self.ids, self.mask, o["dws"])
        mdc.mdc_dispatch_ffn(sh, self.inter, self.x, o["q"], o["qs"], o["assist"], o["recv"], o["etn"],
                             o["row_idx"], *self.weights, o["y"], o["dws"], o["fws"], expert_scales=self.scales,
                             expand_scales=o["esc"])
        torch.cuda.synchronize()
        return o


def rows_received(o, cap):
    return min(int(o["etn"].sum().item()), cap)


def assert_same_dispatch(a, b, n):
    for k in ("q", "assist"):
        assert torch.equal(a[k][:n], b[k][:n]), k
    for k in ("qs", "esc"):
        assert torch.equal(a[k][:n].view(torch.int32), b[k][:n].view(torch.int32)), k
    for k in ("recv", "etn", "row_idx"):
        assert torch.equal(a[k], b[k]), k
    sa, sb = mdc.read_status(a["dws"]), mdc.read_status(b["dws"])
    assert sa == sb, (sa, sb)


def check_against_oracle(inp, o, n, check_y=True):
    w, wi = inp.w, inp.wi
    mask = wi.mask
    ref = O.dispatch(wi.x, wi.ids, mask, inp.rank, w.experts, inp.cap, w.zero_experts, w.copy_experts,
                     scales=wi.scales)
    assert n == ref.assist_info.shape[0]
    assert np.array_equal(o["assist"][:n].cpu().numpy(), ref.assist_info)
    assert np.array_equal(o["recv"].cpu().numpy(), ref.ep_recv_counts)
    assert np.array_equal(o["etn"].cpu().numpy(), ref.expert_token_nums)
    assert np.array_equal(o["esc"][:n].cpu().numpy().view(np.uint32), ref.expand_scales.view(np.uint32))
    st = mdc.read_status(o["dws"])
    assert st["dropped_ids"] == ref.dropped_ids and st["overflow_rows"] == ref.overflow_rows, st
    if check_y and n > 0:
        row_expert = np.repeat(np.arange(w.local_experts), ref.expert_token_nums)[:n]
        want = O.ffn(ref.expand_x, row_expert, inp.fw.w1, inp.fw.w1_scale, inp.fw.w2, inp.fw.w2_scale)
        err = rel_l2(G.bits(o["y"][:n]), want)
        say(f"  y rel L2 vs oracle {err:.3e} over {n} rows")
        assert err <= REL_L2


@pytest.mark.parametrize("variant", [
    dict(world=2, bs=64, hidden=256, experts=4, topk=2, inter=512),
    dict(world=1, bs=300, hidden=384, experts=3, topk=2, inter=256),       # ragged m-tiles
    dict(world=4, bs=96, hidden=128, experts=16, topk=3, inter=768),
    dict(world=1, bs=700, hidden=256, experts=37, topk=3, inter=512),      # 37 experts, one partial m-tile each
    dict(world=8, bs=512, hidden=512, experts=32, topk=4, inter=512),      # several m-tiles per expert
    dict(world=8, bs=256, hidden=256, experts=128, topk=8, inter=512, routing="zipf"),   # skewed expert loads
    dict(world=4, bs=128, hidden=256, experts=32, topk=4, inter=256, inactive_frac=0.25),  # 1D mask
    dict(world=4, bs=128, hidden=256, experts=32, topk=4, inter=256, route_mask_frac=0.2),  # 2D mask
    dict(world=2, bs=1024, hidden=8192, experts=4, topk=2, inter=256),     # the widest quantised row
    dict(world=4, bs=128, hidden=256, experts=32, topk=4, inter=256, zero_experts=4, copy_experts=4),
    dict(world=1, bs=128, hidden=128, experts=2048, topk=16, inter=256),   # max L: 2048 experts of ~1 row
])
def test_dispatch_ffn_equals_stream_ordered(variant):
    v = dict(variant)
    inter = v.pop("inter")
    w = gen.workload("tiny", index=60 + v["bs"] % 13 + v["experts"] % 7, **v)
    say(f"dispatch_ffn W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} N={inter} "
        f"routing={w.routing} mask1d={w.inactive_frac} mask2d={w.route_mask_frac} "
        f"Z={w.zero_experts} C={w.copy_experts}")
    inp = Inputs(w, inter, mask_per_route=1 if w.route_mask_frac > 0 else 0)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined()
    n = rows_received(a, inp.cap)
    assert n > 0
    assert_same_dispatch(a, b, n)
    assert mdc.read_status(b["fws"])["wait_timeouts"] == 0
    assert torch.equal(a["y"][:n].view(torch.int16), b["y"][:n].view(torch.int16))
    say(f"  bit-identical over {n} rows")
    check_against_oracle(inp, b, n)


def test_dispatch_ffn_invalid_ids_and_overflow():
    """Ids outside [0, E) are counted as dropped; rows past a small capacity are
    dropped and counted; both paths agree and match the oracle."""
    w = gen.workload("tiny", world=4, bs=256, hidden=256, experts=16, topk=4, index=71)
    wi = gen.world_inputs(w)
    ids = wi.ids.copy()
    g = np.random.default_rng(5)
    bad = g.random(ids.shape) < 0.05
    ids[bad] = g.choice([-1, -7, w.experts, w.experts + 3], size=int(bad.sum()))
    cap = 700   # below the ~1024 rows this rank receives
    inp = Inputs(w, 256, capacity=cap, ids=ids)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined()
    n = rows_received(a, cap)
    st = mdc.read_status(b["dws"])
    say(f"  status {st}, rows {n}")
    assert st["dropped_ids"] > 0 and st["overflow_rows"] > 0
    assert n == cap
    assert_same_dispatch(a, b, n)
    assert torch.equal(a["y"][:n].view(torch.int16), b["y"][:n].view(torch.int16))
    check_against_oracle(inp, b, n)


def test_dispatch_ffn_tile_table_in_global_memory():
    """A capacity of 400000 rows bounds the m-tile table above the 1536 entries
    the persistent kernel caches in LDS: it reads the table from global memory."""
    w = gen.workload("tiny", world=2, bs=256, hidden=256, experts=4, topk=2, index=79)
    inp = Inputs(w, 256, capacity=400_000)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined()
    n = rows_received(a, inp.cap)
    assert n > 0
    assert_same_dispatch(a, b, n)
    assert torch.equal(a["y"][:n].view(torch.int16), b["y"][:n].view(torch.int16))
    assert mdc.read_status(b["fws"])["wait_timeouts"] == 0
    check_against_oracle(inp, b, n)


@pytest.mark.parametrize("case", ["no_tokens", "no_capacity", "empty_experts"])
def test_dispatch_ffn_degenerate(case):
    if case == "no_tokens":
        w = gen.workload("tiny", world=2, bs=0, hidden=128, experts=4, topk=2, index=72)
        inp = Inputs(w, 256, capacity=64)
    elif case == "no_capacity":
        w = gen.workload("tiny", world=2, bs=32, hidden=128, experts=4, topk=2, index=73)
        inp = Inputs(w, 256, capacity=0)
    else:
        # every route goes to experts of rank 1: rank 0's experts receive nothing
        w = gen.workload("tiny", world=2, bs=64, hidden=128, experts=8, topk=2, index=74)
        wi = gen.world_inputs(w)
        ids = 4 + (wi.ids % 4)
        inp = Inputs(w, 256, ids=ids)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined()
    n = rows_received(b, inp.cap)
    say(f"  {case}: rows {n}, status {mdc.read_status(b['dws'])}")
    assert n == 0
    assert_same_dispatch(a, b, 0)
    check_against_oracle(inp, b, 0, check_y=False)
    assert mdc.read_status(b["fws"])["wait_timeouts"] == 0


def test_dispatch_ffn_full_size():
    """The ffn workload's shapes (8 x 2048 tokens, H = 7168, 128 experts, top-8,
    N = 4096): bit-identical to the stream-ordered calls, repeatable, and y
    within the FFN tolerance of the oracle."""
    w = gen.workload("ffn")
    say("dispatch_ffn full size: generating inputs and weights")
    inp = Inputs(w, w.inter)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined()
    n = rows_received(a, inp.cap)
    assert_same_dispatch(a, b, n)
    assert mdc.read_status(b["fws"])["wait_timeouts"] == 0
    assert torch.equal(a["y"][:n].view(torch.int16), b["y"][:n].view(torch.int16))
    c = inp.run_pipelined(o=b)   # again on the same buffers and workspaces
    assert torch.equal(a["y"][:n].view(torch.int16), c["y"][:n].view(torch.int16))
    say(f"  bit-identical over {n} rows, twice")
    check_against_oracle(inp, b, n)


def test_dispatch_ffn_wait_timeout_is_reported():
    """With the spin field at 1 every wait polls at most twice: tiles whose rows
    are not ready by then give up, count themselves in the FFN status block's
    wait_timeouts and leave NaN in their y rows.  Every kernel still exits; the
    dispatched rows are unaffected, and every value that is not NaN equals the
    stream-ordered result."""
    w = gen.workload("tiny", world=4, bs=512, hidden=1024, experts=8, topk=2, index=75)
    inp = Inputs(w, 2048)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined(flags=1 << mdc.MDC_FLAG_SPIN_SHIFT)
    n = rows_received(a, inp.cap)
    st = mdc.read_status(b["fws"])
    nan_vals = torch.isnan(b["y"][:n].float())
    say(f"  wait_timeouts {st['wait_timeouts']}, rows with NaN {int(nan_vals.any(dim=1).sum())} of {n}")
    assert st["wait_timeouts"] > 0 and bool(nan_vals.any())
    assert_same_dispatch(a, b, n)
    fine = ~nan_vals
    assert torch.equal(b["y"][:n].view(torch.int16)[fine], a["y"][:n].view(torch.int16)[fine])
    c = inp.run_pipelined(o=b)
    assert mdc.read_status(c["fws"])["wait_timeouts"] == 0
    assert torch.equal(c["y"][:n].view(torch.int16), a["y"][:n].view(torch.int16))


def _random_worlds(n=16, seed=20261203):
    """Seeded random small worlds for the pipelined path: ragged W/BS/E/K, H a
    multiple of 128 up to 2048, FFN widths up to 1024, uniform, Zipf, first-K
    or round-robin routing, 1D or 2D masks, zero/copy experts, full or
    overflowing capacity."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        W = int(rng.integers(1, 9))
        L = int(rng.integers(1, 33))
        Z = int(rng.choice([0, 0, 2]))
        C = int(rng.choice([0, 0, 2]))
        E = W * L
        K = int(rng.integers(1, min(8, E + Z + C) + 1))
        routing = str(rng.choice(["uniform", "uniform", "zipf", "first_k", "round_robin"]))
        if Z or C or (routing == "zipf" and K > E):
            routing = "uniform"   # the other generators draw routed experts only
        c = dict(world=W, bs=int(rng.integers(1, 513)), hidden=int(rng.choice([128, 256, 384, 1024, 2048])),
                 experts=E, topk=K, zero_experts=Z, copy_experts=C, routing=routing,
                 inactive_frac=float(rng.choice([0.0, 0.2])), route_mask_frac=float(rng.choice([0.0, 0.0, 0.3])))
        inter = int(rng.choice([256, 512, 1024]))
        cap_scale = float(rng.choice([1.0, 1.0, 0.4]))
        cases.append(pytest.param(i, c, inter, cap_scale, id=f"world{i}"))
    return cases


@pytest.mark.parametrize("i,cfg,inter,cap_scale", _random_worlds())
def test_dispatch_ffn_random_worlds(i, cfg, inter, cap_scale):
    w = gen.workload("tiny", index=300 + i, **cfg)
    cap = max(1, int(round(w.capacity * cap_scale)))
    say(f"dispatch_ffn random world {i}: {cfg} N={inter} A={cap}")
    inp = Inputs(w, inter, capacity=cap, mask_per_route=1 if w.route_mask_frac > 0 else 0)
    a = inp.run_stream_ordered()
    b = inp.run_pipelined()
    n = rows_received(a, inp.cap)
    assert_same_dispatch(a, b, n)
    assert mdc.read_status(b["fws"])["wait_timeouts"] == 0
    assert torch.equal(a["y"][:n].view(torch.int16), b["y"][:n].view(torch.int16))
    check_against_oracle(inp, b, n)
