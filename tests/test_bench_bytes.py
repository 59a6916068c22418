"""The roofline's algorithmic bytes (bench.algorithmic_bytes) against a
route-by-route count written out from the definition of each call.

Per step, dispatch share d then combine share r:
  layout  reads every id (4 B) and mask byte, writes L*W int32 prefixes and L int64 counts;
  gather  reads every id again, each source row with a route to d once (2H), and writes
          per received row the row (2H, or H int8 + a 4 B scale), its triplet (12 B) and
          its inverse-index entry (4 B);
  combine reads per token and k an id, a scale and an inverse-index entry (12 B), the
          token's mask byte(s), one expert row per dispatched route (2H), the token's
          original row once if it has a present copy-expert route, its shared-expert row
          once if it has any present route, and writes the output row (2H).
Zero-expert routes read no row.
"""
import numpy as np
import pytest

import bench
from workloads import gen


def brute(w, ids, mask, d=0, r=0):
    W, BS, K = ids.shape
    E, Z, C, H = w.experts, w.zero_experts, w.copy_experts, w.hidden
    L = E // W
    row_out = (H + 4) if w.inter else 2 * H

    def active(s, t, k):
        if mask is None:
            return True
        return bool(mask[s, t, k]) if mask.ndim == 3 else bool(mask[s, t])

    layout = ids.size * 4 + (0 if mask is None else mask.size) + L * W * 4 + L * 8
    gather = ids.size * 4
    for s in range(W):
        for t in range(BS):
            n_local = 0
            for k in range(K):
                e = int(ids[s, t, k])
                if active(s, t, k) and 0 <= e < E and e // L == d:
                    n_local += 1
            if n_local:
                gather += 2 * H + n_local * (row_out + 12 + 4)
    combine = BS * K * 12 + (0 if mask is None else mask.size // W)
    for t in range(BS):
        any_present = has_copy = False
        for k in range(K):
            e = int(ids[r, t, k])
            if not active(r, t, k) or not (0 <= e < E + Z + C):
                continue
            any_present = True
            if e < E:
                combine += 2 * H
            elif e >= E + Z:
                has_copy = True
        combine += (2 * H if has_copy else 0) + (2 * H if (w.shared and any_present) else 0) + 2 * H
    return layout, gather, combine


@pytest.mark.parametrize("over", [
    dict(),
    dict(inactive_frac=0.2),
    dict(route_mask_frac=0.3, zero_experts=3, copy_experts=2),
    dict(zero_experts=4, copy_experts=4, shared=True),
    dict(routing="zipf", inactive_frac=0.1, shared=True),
    dict(inter=512),
])
def test_algorithmic_bytes_match_route_count(over):
    w = gen.workload("tiny", world=4, bs=37, hidden=64, experts=16, topk=3, index=70, **over)
    wi = gen.world_inputs(w)
    for d, r in ((0, 0), (2, 3)):
        got = bench.algorithmic_bytes(w, wi.ids, wi.mask, d=d, r=r)
        assert (got["layout"], got["gather"], got["combine"]) == brute(w, wi.ids, wi.mask, d=d, r=r), (d, r)


def test_share_step_bytes():
    """The share workload's figures quoted with the roofline (390.4 + 293.8 + 0.5 MB)."""
    w = gen.workload("share")
    wi = gen.world_inputs(w)
    by = bench.algorithmic_bytes(w, wi.ids, wi.mask)
    assert (by["R"], by["U"]) == (16307, 10871)
    assert (by["gather"], by["combine"], by["layout"]) == (390409008, 293797888, 524928)
