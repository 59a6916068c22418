"""Helpers shared by the GPU tests: upload seeded inputs, run the W virtual
dispatches and the combine through the C ABI, compare with the oracle.

Only marshalling and test-side experts live here (torch on the GPU); every
step of the path runs in libmdc's kernels.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
import torch

import combine_route_histogram_amd as mdc
from oracle import mdc_oracle as O

DEV = "cuda"


def to_dev_bf16(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)


def bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@dataclass
class GpuWorld:
    shape: mdc.Shape
    x: torch.Tensor
    ids: torch.Tensor
    mask: Optional[torch.Tensor]
    row_idx: torch.Tensor
    outs: List[dict]


def dispatch_world(shape: mdc.Shape, x: np.ndarray, ids: np.ndarray, mask: Optional[np.ndarray],
                   split: bool = False, sentinel: int = -2, scales: Optional[np.ndarray] = None) -> GpuWorld:
    """Run the dispatch of every destination rank d = 0..W-1 on the GPU.

    With scales ([W][BS][K] fp32) every dispatch also writes expand_scales.
    The status block of every workspace is filled with garbage first, so a
    dispatch that did not rewrite it shows.
    """
    W, BS, K = ids.shape
    xd = to_dev_bf16(x) if x.size else torch.empty((W, BS, shape.hidden), dtype=torch.bfloat16, device=DEV)
    idd = torch.from_numpy(np.ascontiguousarray(ids)).to(DEV)
    md = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask.astype(np.uint8))).to(DEV)
    scd = None if scales is None else torch.from_numpy(np.ascontiguousarray(scales, dtype=np.float32)).to(DEV)
    row_idx = torch.full((W, BS, K), sentinel, dtype=torch.int32, device=DEV)
    outs = []
    for d in range(W):
        sh = shape.with_rank(d)
        o = mdc.alloc_dispatch_outputs(sh, DEV)
        o["workspace"][:mdc.MDC_STATUS_BYTES].fill_(0x5A)
        esc = None
        if scd is not None:
            esc = torch.full((shape.capacity,), float("nan"), dtype=torch.float32, device=DEV)
            o["expand_scales"] = esc
        if split:
            mdc.mdc_dispatch_layout(sh, idd, md, o["workspace"])
            mdc.mdc_dispatch_gather(sh, xd, o["expand_x"], o["assist_info"], o["ep_recv_counts"],
                                    o["expert_token_nums"], row_idx, o["workspace"], expert_scales=scd,
                                    expand_scales=esc)
        else:
            mdc.mdc_dispatch(sh, xd, idd, md, o["expand_x"], o["assist_info"], o["ep_recv_counts"],
                             o["expert_token_nums"], row_idx, o["workspace"], expert_scales=scd, expand_scales=esc)
        outs.append(o)
    torch.cuda.synchronize()
    return GpuWorld(shape, xd, idd, md, row_idx, outs)


def check_dispatch(gw: GpuWorld, x, ids, mask, experts: int, capacity: int, refs=None, scales=None):
    """Bit-exact comparison of every integer output, every copied row, the
    expand_scales rows and the status block with the oracle."""
    W, BS, K = ids.shape
    Z, C = gw.shape.zero_experts, gw.shape.copy_experts
    row_idx = gw.row_idx.cpu().numpy()
    seen = np.zeros((W, BS, K), bool)
    for d in range(W):
        o = gw.outs[d]
        ref = O.dispatch(x, ids, mask, d, experts, capacity, Z, C, scales) if refs is None else refs[d]
        ep = o["ep_recv_counts"].cpu().numpy()
        etn = o["expert_token_nums"].cpu().numpy()
        assert ep.dtype == np.int32 and etn.dtype == np.int64
        assert np.array_equal(ep, ref.ep_recv_counts), f"epRecvCounts d={d}"
        assert np.array_equal(etn, ref.expert_token_nums), f"expertTokenNums d={d}"
        st = mdc.read_status(o["workspace"])
        assert st["dropped_ids"] == ref.dropped_ids, f"dropped_ids d={d}: {st}"
        assert st["overflow_rows"] == ref.overflow_rows, f"overflow_rows d={d}: {st}"
        assert st["wait_timeouts"] == 0, f"status d={d}: {st}"
        n = ref.assist_info.shape[0]
        assist = o["assist_info"][:n].cpu().numpy()
        assert np.array_equal(assist, ref.assist_info), f"assistInfo d={d}"
        if "expand_scales" in o:
            got_s = o["expand_scales"][:n].cpu().numpy()
            assert np.array_equal(got_s.view(np.uint32), ref.expand_scales.view(np.uint32)), f"expandScales d={d}"
        if x is not None and x.size:
            got = bits(o["expand_x"][:n])
            assert np.array_equal(got, ref.expand_x), f"expandX d={d}"
        # inverse index: row of every route sent to d, -1 past the capacity
        for (le, s, t, k) in O.local_routes(ids, mask, d, experts):
            want = ref.expanded_row_idx.get((s, t, k), -1)
            assert row_idx[s, t, k] == want, (d, s, t, k)
            seen[s, t, k] = True
    # routes sent nowhere keep the caller's value
    assert np.all(row_idx[~seen] == -2)
    return True


def apply_expert(gw: GpuWorld, kind: str, experts: int) -> List[torch.Tensor]:
    """Test-side expert on the GPU: identity, or y = x * 2^((e mod 4) - 2) on valid rows."""
    ys = []
    W, BS, K = gw.ids.shape
    ids_flat = gw.ids.reshape(-1).long()
    for d, o in enumerate(gw.outs):
        if kind == "identity":
            ys.append(o["expand_x"])
            continue
        n = int(min(int(o["ep_recv_counts"][-1].item()), gw.shape.capacity))
        y = o["expand_x"].clone()
        if n:
            a = o["assist_info"][:n].long()
            e = ids_flat[(a[:, 0] * BS + a[:, 1]) * K + a[:, 2]]
            f = torch.exp2(((e % 4) - 2).to(torch.float32))
            y[:n] = (o["expand_x"][:n].float() * f[:, None]).to(torch.bfloat16)
        ys.append(y)
    torch.cuda.synchronize()
    return ys


def oracle_segments(x, ids, mask, experts, capacity, kind, zero_experts=0, copy_experts=0, scales=None):
    W = ids.shape[0]
    L = experts // W
    segs = [O.dispatch(x, ids, mask, d, experts, capacity, zero_experts, copy_experts, scales) for d in range(W)]
    fn = O.expert_identity if kind == "identity" else O.expert_pow2
    ys = [fn(s.expand_x, s.assist_info, ids, L) for s in segs]
    return segs, ys


def run_combine(gw: GpuWorld, ys: List[torch.Tensor], r: int, scales: np.ndarray,
                shared: Optional[np.ndarray], ori: Optional[np.ndarray] = None, use_expand_scales: bool = False,
                perf: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mdc_combine for source rank r.  With use_expand_scales the weights of
    dispatched routes come from the dispatches' expand_scales; with perf the
    call adds its per-rank waits to that [W] int64 tensor."""
    sh = gw.shape.with_rank(r)
    BS, K = scales.shape
    out = torch.empty((BS, sh.hidden), dtype=torch.bfloat16, device=DEV)
    sc = torch.from_numpy(np.ascontiguousarray(scales)).to(DEV)
    shd = None if shared is None else to_dev_bf16(shared)
    orid = None if ori is None else to_dev_bf16(ori)
    m = None if gw.mask is None else gw.mask[r].contiguous()
    esc = [o["expand_scales"] for o in gw.outs] if use_expand_scales else None
    ws = None
    if perf is not None:
        ws = torch.empty(mdc.mdc_combine_workspace(sh), dtype=torch.uint8, device=DEV)
    mdc.mdc_combine(sh, ys, [o["assist_info"] for o in gw.outs], [o["ep_recv_counts"] for o in gw.outs],
                    gw.row_idx[r].contiguous(), gw.ids[r].contiguous(), sc, m, shd, out, workspace=ws, ori_x=orid,
                    expand_scales=esc, performance_info=perf)
    torch.cuda.synchronize()
    return out


def ulp_diff(a: np.ndarray, b: np.ndarray) -> int:
    def ordered(u):
        u = u.astype(np.int32)
        mag = u & 0x7FFF
        return np.where(u & 0x8000, -mag, mag)
    if a.size == 0:
        return 0
    return int(np.max(np.abs(ordered(a) - ordered(b))))
