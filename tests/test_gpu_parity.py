"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Dispatch is compared bit-exactly (every integer output and every copied bf16
row); combine within 1 bf16 ulp of the oracle (the contract), and bit-exactly
as well (the kernels round every fp32 product and sum in the oracle's order).
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


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _shape(w: gen.Workload, capacity=None):
    return mdc.Shape(w.world, 0, w.bs, w.hidden, w.topk, w.experts, w.capacity if capacity is None else capacity,
                     mask_per_route=1 if w.route_mask_frac > 0 else 0, zero_experts=w.zero_experts,
                     copy_experts=w.copy_experts)


def _end_to_end(w: gen.Workload, expert="identity", capacity=None, ranks=None, split=False, expand_scales=None):
    """Dispatch every rank, apply the test expert, combine the given ranks; compare all with the oracle.

    The dispatches also carry the routes' weights to expand_scales (checked
    bit-exactly).  The combine takes its weights from those expand_scales on
    odd ranks (or on every rank with expand_scales=True, none with False) and
    from expert_scales otherwise; the result must be the same.
    """
    say(f"case {w.name} W={w.world} BS={w.bs} H={w.hidden} E={w.experts} K={w.topk} routing={w.routing} "
        f"inactive={w.inactive_frac} route_mask={w.route_mask_frac} Z={w.zero_experts} C={w.copy_experts} "
        f"shared={w.shared} expert={expert} cap={capacity}")
    wi = gen.world_inputs(w)
    cap = w.capacity if capacity is None else capacity
    gw = G.dispatch_world(_shape(w, cap), wi.x, wi.ids, wi.mask, split=split, scales=wi.scales)
    segs, oys = G.oracle_segments(wi.x, wi.ids, wi.mask, w.experts, cap, expert, w.zero_experts, w.copy_experts,
                                  wi.scales)
    G.check_dispatch(gw, wi.x, wi.ids, wi.mask, w.experts, cap, refs=segs)
    say("  dispatch bit-exact on every rank (rows, triplets, counts, expand_scales, status)")
    ys = G.apply_expert(gw, expert, w.experts)
    for r in (range(w.world) if ranks is None else ranks):
        sh = None if wi.shared is None else wi.shared[r]
        m = None if wi.mask is None else wi.mask[r]
        ori = wi.x[r] if w.copy_experts else None
        use_esc = (r % 2 == 1) if expand_scales is None else expand_scales
        got = G.bits(G.run_combine(gw, ys, r, wi.scales[r], sh, ori, use_expand_scales=use_esc))
        want = O.combine(oys, [s.assist_info for s in segs], r, wi.ids[r], m, wi.scales[r], sh, w.hidden,
                         experts=w.experts, zero_experts=w.zero_experts, copy_experts=w.copy_experts, ori_r=ori)
        assert G.ulp_diff(got, want) <= 1, f"combine r={r} beyond 1 ulp"
        assert np.array_equal(got, want), f"combine r={r} not bit-exact ({int((got != want).sum())} differ)"
    say("  combine bit-exact")
    return gw, wi


def test_tiny_identity():
    _end_to_end(gen.workload("tiny"))


def test_tiny_split_stages():
    _end_to_end(gen.workload("tiny"), split=True)


def test_decode_shared():
    _end_to_end(gen.workload("decode"), expert="pow2")


def test_share_full_size():
    """One GPU's real share (8 x 2048 x 7168, 128 experts, topK 8, shared expert), every rank."""
    _end_to_end(gen.workload("share"))


def test_skewed_full_size():
    """Zipf(1.2) routing with 10% inactive tokens at the full share shape, power-of-two expert, every rank."""
    _end_to_end(gen.workload("skewed"), expert="pow2")


@pytest.mark.parametrize("variant", [
    dict(world=3, bs=101, hidden=136, experts=9, topk=3),           # ragged chunks and column tile
    dict(world=2, bs=300, hidden=2056, experts=6, topk=5, inactive_frac=0.3),
    dict(world=1, bs=257, hidden=8, experts=2048, topk=16),          # max K, max L, H = one vector
    dict(world=4, bs=64, hidden=64, experts=4, topk=1),              # K = 1, L = 1
    dict(world=5, bs=33, hidden=4104, experts=40, topk=8, shared=True),
    dict(world=8, bs=17, hidden=7168, experts=256, topk=9, shared=True),
    dict(world=64, bs=6, hidden=136, experts=128, topk=4, shared=True),   # max combine world (W = 64)
])
@pytest.mark.parametrize("split", [False, True], ids=["one_shot", "split_stages"])
def test_ragged_shapes(variant, split):
    # one-shot mdc_dispatch takes the one-launch path at these sizes where it
    # applies; the split stages always take the rank + gather kernels
    w = gen.workload("tiny", index=60 + len(str(variant)), **variant)
    _end_to_end(w, expert="pow2", split=split)


@pytest.mark.parametrize("hidden,split", [(8192, False), (8200, False), (12296, False), (12296, True)])
def test_large_hidden(hidden, split):
    """H = 8192 is the one-launch dispatch's longest row (1024 vectors, one
    per thread); 8200 falls back to the rank and gather kernels; 12296 spreads
    a row over three gather tiles and 13 combine tiles, the last ones ragged."""
    w = gen.workload("tiny", world=2, bs=40, hidden=hidden, experts=8, topk=3, shared=True, index=96)
    _end_to_end(w, expert="pow2", split=split)


def test_capacity_overflow_drops_rows():
    w = gen.workload("tiny", world=2, bs=64, hidden=64, experts=4, topk=2, index=70)
    _end_to_end(w, capacity=37)


def test_zero_capacity():
    w = gen.workload("tiny", world=2, bs=16, hidden=64, experts=4, topk=2, index=71)
    _end_to_end(w, capacity=0)


def test_all_to_first_experts_fills_capacity():
    """The A2 sample routing: every route lands on rank 0 and A is filled exactly."""
    w = gen.workload("tiny", world=8, bs=32, hidden=256, experts=256, topk=8, routing="first_k",
                     shared=True, index=72)
    gw, wi = _end_to_end(w, ranks=[0, 5])
    assert int(gw.outs[0]["ep_recv_counts"][-1].item()) == w.capacity == 2048
    for d in range(1, 8):
        assert int(gw.outs[d]["ep_recv_counts"][-1].item()) == 0


def test_round_robin_routing():
    w = gen.workload("tiny", world=4, bs=100, hidden=128, experts=16, topk=4, routing="round_robin", index=73)
    _end_to_end(w)


def test_all_inactive():
    w = gen.workload("tiny", world=2, bs=40, hidden=64, experts=8, topk=2, inactive_frac=1.0, index=74,
                     shared=True)
    gw, wi = _end_to_end(w)
    for o in gw.outs:
        assert int(o["ep_recv_counts"][-1].item()) == 0


def test_empty_batch():
    w = gen.workload("tiny", world=2, bs=0, hidden=64, experts=8, topk=2, index=75)
    sh = _shape(w)
    ids = np.zeros((2, 0, 2), np.int32)
    gw = G.dispatch_world(sh, np.zeros((2, 0, 64), np.uint16), ids, None)
    for o in gw.outs:
        assert not o["ep_recv_counts"].any() and not o["expert_token_nums"].any()


@pytest.mark.parametrize("split", [False, True], ids=["one_shot", "split_stages"])
def test_invalid_and_duplicate_ids(split):
    """Out-of-range ids are dropped and counted in the status block, as many as the oracle counts."""
    g = np.random.default_rng(5)
    W, BS, K, E, H = 2, 50, 4, 8, 64
    ids = g.integers(-3, E + 3, size=(W, BS, K)).astype(np.int32)   # duplicates and out-of-range ids
    x = gen.bf16_from_f32(g.standard_normal((W, BS, H), dtype=np.float32))
    sh = mdc.Shape(W, 0, BS, H, K, E, W * BS * K)
    gw = G.dispatch_world(sh, x, ids, None, split=split)
    G.check_dispatch(gw, x, ids, None, E, W * BS * K)
    want = O.dispatch(None, ids, None, 0, E, W * BS * K).dropped_ids
    assert want == int(((ids < 0) | (ids >= E)).sum()) > 0
    for o in gw.outs:
        assert mdc.read_status(o["workspace"])["dropped_ids"] == want
    ys = G.apply_expert(gw, "identity", E)
    segs, oys = G.oracle_segments(x, ids, None, E, W * BS * K, "identity")
    sc = g.standard_normal((BS, K)).astype(np.float32)
    for r in range(W):
        got = G.bits(G.run_combine(gw, ys, r, sc, None))
        want = O.combine(oys, [s.assist_info for s in segs], r, ids[r], None, sc, None, H)
        assert np.array_equal(got, want)


def test_identity_round_trip_returns_x():
    """dispatch -> identity -> combine with unit-sum scales and no shared expert returns x by value."""
    w = gen.workload("share", bs=512, shared=False, index=76)
    wi = gen.world_inputs(w)
    gw = G.dispatch_world(_shape(w), wi.x, wi.ids, None)
    ys = G.apply_expert(gw, "identity", w.experts)
    for r in (0, 6):
        got = G.bits(G.run_combine(gw, ys, r, wi.scales[r], None))
        assert np.array_equal(O.bf16_to_f32(got), O.bf16_to_f32(wi.x[r]))


def test_deterministic_repeat():
    w = gen.workload("decode")
    wi = gen.world_inputs(w)
    a = G.dispatch_world(_shape(w), wi.x, wi.ids, wi.mask)
    b = G.dispatch_world(_shape(w), wi.x, wi.ids, wi.mask)
    for oa, ob in zip(a.outs, b.outs):
        n = int(oa["ep_recv_counts"][-1].item())
        assert torch.equal(oa["assist_info"][:n], ob["assist_info"][:n])
        assert torch.equal(oa["expand_x"][:n].view(torch.int16), ob["expand_x"][:n].view(torch.int16))
    ya = G.apply_expert(a, "identity", w.experts)
    ca = G.run_combine(a, ya, 0, wi.scales[0], wi.shared[0])
    cb = G.run_combine(a, ya, 0, wi.scales[0], wi.shared[0])
    assert torch.equal(ca.view(torch.int16), cb.view(torch.int16))


def test_combine_stale_row_index_is_rejected():
    """Garbage in the inverse index (a dispatch that never ran) is caught by the triplet check."""
    w = gen.workload("tiny", world=2, bs=32, hidden=64, experts=4, topk=2, index=77)
    wi = gen.world_inputs(w)
    gw = G.dispatch_world(_shape(w), wi.x, wi.ids, None)
    ys = G.apply_expert(gw, "identity", w.experts)
    gw.row_idx[0].fill_(0)          # every entry of rank 0 now points at row 0 of its destination
    got = G.bits(G.run_combine(gw, ys, 0, wi.scales[0], None))
    segs, oys = G.oracle_segments(wi.x, wi.ids, None, w.experts, w.capacity, "identity")
    # only a route whose true row is 0 survives: give the oracle just row 0 of each segment
    first = [s.assist_info[:1] if s.assist_info.shape[0] and s.assist_info[0, 0] == 0 else s.assist_info[:0]
             for s in segs]
    want = O.combine(oys, first, 0, wi.ids[0], None, wi.scales[0], None, w.hidden)
    assert np.array_equal(got, want)


def test_route_mask_2d():
    """Route-level mask [BS][K]: single routes off, some whole tokens off."""
    w = gen.workload("tiny", world=2, bs=100, hidden=264, experts=8, topk=3, route_mask_frac=0.3,
                     inactive_frac=0.1, shared=True, index=90)
    _end_to_end(w, expert="pow2")


def test_zero_and_copy_experts():
    """Zero experts contribute 0, copy experts the token's own row; neither is dispatched."""
    w = gen.workload("tiny", world=2, bs=64, hidden=136, experts=8, topk=4, zero_experts=2, copy_experts=3,
                     inactive_frac=0.2, shared=True, index=91)
    gw, wi = _end_to_end(w, expert="pow2")
    n_special = int(((wi.ids >= w.experts) & (wi.ids < w.experts + 5)).sum())
    assert n_special > 0


def test_special_experts_and_route_mask_full_size():
    """Share shapes with 8 zero and 8 copy experts and a 2D route mask."""
    w = gen.workload("share", zero_experts=8, copy_experts=8, route_mask_frac=0.05, index=92)
    _end_to_end(w, ranks=[0, 4])


def _random_cases(n=40, seed=20261202):
    """Seeded random small worlds: ragged W/BS/H/E/K (BS up to 700, H up to
    7168), uniform, Zipf, first-K or round-robin routing, 1D or 2D masks,
    zero/copy experts, shared expert on or off, full or overflowing capacity,
    both dispatch paths and both test experts."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        W = int(rng.integers(1, 9))
        L = int(rng.integers(1, 41))
        Z = int(rng.choice([0, 0, 1, 3]))
        C = int(rng.choice([0, 0, 2]))
        E = W * L
        K = int(rng.integers(1, min(16, E + Z + C) + 1))
        routing = str(rng.choice(["uniform", "uniform", "zipf", "first_k", "round_robin"]))
        if Z or C or (routing == "zipf" and K > E):
            routing = "uniform"   # the other generators draw routed experts only
        c = dict(world=W, bs=int(rng.integers(1, 701)),
                 hidden=int(rng.choice([8, 64, 136, 520, 1032, 2056, 2056, 7168])),
                 experts=E, topk=K, zero_experts=Z, copy_experts=C, shared=bool(rng.integers(0, 2)), routing=routing,
                 inactive_frac=float(rng.choice([0.0, 0.2])), route_mask_frac=float(rng.choice([0.0, 0.0, 0.3])))
        cap_scale = float(rng.choice([1.0, 1.0, 0.3]))
        split = bool(rng.integers(0, 2))
        expert = str(rng.choice(["identity", "pow2"]))
        cases.append(pytest.param(i, c, cap_scale, split, expert, id=f"case{i}"))
    return cases


@pytest.mark.parametrize("i,cfg,cap_scale,split,expert", _random_cases())
def test_random_shapes(i, cfg, cap_scale, split, expert):
    w = gen.workload("tiny", index=200 + i, **cfg)
    cap = max(0, int(round(w.capacity * cap_scale)))
    _end_to_end(w, expert=expert, capacity=cap, split=split)


@pytest.mark.parametrize("split", [False, True], ids=["one_shot", "split_stages"])
def test_dropped_ids_beside_zero_and_copy_experts_and_masks(split):
    """Ids in [E, E+Z+C) are zero/copy experts, not dropped; ids outside [0, E+Z+C) on active routes are
    dropped; masked-off routes never count.  Share-size ranks so the split path uses several rank groups."""
    g = np.random.default_rng(11)
    W, BS, K, E, Z, C, H = 4, 700, 6, 32, 3, 2, 136
    ids = g.integers(-4, E + Z + C + 4, size=(W, BS, K)).astype(np.int32)
    mask = (g.random((W, BS, K)) >= 0.25).astype(np.uint8)
    x = gen.bf16_from_f32(g.standard_normal((W, BS, H), dtype=np.float32))
    sc = g.random((W, BS, K)).astype(np.float32)
    sh = mdc.Shape(W, 0, BS, H, K, E, W * BS * K, mask_per_route=1, zero_experts=Z, copy_experts=C)
    gw = G.dispatch_world(sh, x, ids, mask, split=split, scales=sc)
    G.check_dispatch(gw, x, ids, mask, E, W * BS * K, scales=sc)
    want = O.dispatch(None, ids, mask, 0, E, 1, Z, C).dropped_ids
    assert want == int((((ids < 0) | (ids >= E + Z + C)) & (mask != 0)).sum()) > 0


def test_overflow_rows_reported():
    w = gen.workload("tiny", world=2, bs=64, hidden=64, experts=4, topk=2, index=70)
    wi = gen.world_inputs(w)
    gw = G.dispatch_world(_shape(w, 37), wi.x, wi.ids, None)
    G.check_dispatch(gw, wi.x, wi.ids, None, w.experts, 37)
    for d, o in enumerate(gw.outs):
        total = int(o["ep_recv_counts"][-1].item())
        assert mdc.read_status(o["workspace"])["overflow_rows"] == max(0, total - 37) > 0


@pytest.mark.parametrize("name", ["share", "decode"])
def test_performance_info_per_rank_waits(name):
    """performance_info[j] accumulates the wait for rank j's rows: nonzero for every rank the combine reads
    rows from, untouched for ranks it reads nothing from; a second call adds to it.  The output is the
    same as without timing."""
    w = gen.workload(name)
    if name == "share":
        # ranks 5..7 hold no expert any token of rank 0 routes to: draw ids from ranks 0..4 only
        w = gen.workload(name, bs=512, index=120)
    wi = gen.world_inputs(w)
    L = w.experts // w.world
    ids = wi.ids.copy()
    if name == "share":
        ids[0] = ids[0] % (5 * L)
        g = np.random.default_rng(3)
        for t in range(w.bs):   # keep each token's experts distinct
            ids[0, t] = g.permutation(5 * L)[:w.topk]
    gw = G.dispatch_world(_shape(w), wi.x, ids, wi.mask)
    ys = G.apply_expert(gw, "identity", w.experts)
    sh0 = None if wi.shared is None else wi.shared[0]
    plain = G.run_combine(gw, ys, 0, wi.scales[0], sh0)
    perf = torch.full((w.world,), 7, dtype=torch.int64, device=G.DEV)
    timed = G.run_combine(gw, ys, 0, wi.scales[0], sh0, perf=perf)
    assert torch.equal(plain.view(torch.int16), timed.view(torch.int16))
    p1 = perf.cpu().numpy().copy()
    read = np.zeros(w.world, bool)
    read[np.unique(ids[0] // L)] = True
    say(f"  waits (us, +7): {p1.tolist()}; ranks read {np.nonzero(read)[0].tolist()}")
    assert np.all(p1[read] > 7) and np.all(p1[~read] == 7)
    G.run_combine(gw, ys, 0, wi.scales[0], sh0, perf=perf)
    p2 = perf.cpu().numpy()
    assert np.all(p2[read] > p1[read]) and np.all(p2[~read] == 7)
