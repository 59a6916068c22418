"""Plain, slow CPU oracle for the MoE dispatch/combine hot path.

TEST INFRASTRUCTURE ONLY: only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import or call this module. It shares no
code with the HIP library (combine_route_histogram_amd) and never imports it.

Sources (web pages; cited by title and section):
  [TL]  "dispatch_combine_shmem.py" (TileLang-Ascend example), the dispatch
        kernel (send loop, SetStatus, GetCumSum, local data copy,
        UpdateTokenNumsOut) and the combine kernel (weighted sum).
  [CV4] "aclnnMoeDistributeCombineV4" (CANN API page), Function/Formula,
        parameter table, shape-variable table, A2 sample.
  [PTO] "PTO MegaMoE Dispatch + Combine Fusion Example", FrontReorder,
        Dispatch, GMM1/SwiGLU/GMM2 and Combine/Unpermute stages.

Conventions.  bf16 tensors are carried as uint16 bit patterns.  W virtual EP
ranks each own L = E / W contiguous experts; expert e lives on rank e // L as
local expert e % L ([TL] send loop; [CV4] shape-variable table, localExpertNum).
A route is (s, t, k): source rank s, token t, top-k slot k.

Readings of points the pages leave open (each is also listed in the design
notes):
  * row order inside the expert-major layout is (local expert, source rank,
    token, k), stable  ([TL] rank-within-expert counts earlier equal ids, the
    local copy walks status rows le*W + src in order; [PTO] Dispatch orders a
    local expert's rows by source rank);
  * epRecvCounts is the inclusive prefix of the per-(le, src) counts in
    (le-major, src-minor) order ([TL] receive count = begin + count);
  * expertTokenNums are per-local-expert counts, int64 ([TL] UpdateTokenNumsOut);
  * assistInfo rows are (src, token, k) int32 triplets ([TL] send loop);
  * a 1D mask in any order is accepted; inactive tokens send nothing and
    combine to +0.0 (the empty sum of the [CV4] formula); a 2D mask [BS][K]
    switches single routes off ([CV4] A3 notes: a token whose K entries are all
    false does not take part);
  * zero experts (ids in [E, E+Z)) and copy experts (ids in [E+Z, E+Z+C)) are
    never dispatched; in combine such a route is present with output 0 (zero)
    or the token's own unprocessed row oriX[t] (copy) ([CV4] parameter notes on
    zeroExpertNum, copyExpertNum and oriXOptional);
  * ids outside [0, E) are not dispatched; of them, those outside
    [0, E+Z+C) (no routed, zero or copy expert) on active routes are counted
    as dropped ids;
  * expandScales, the dispatch output the combine may take back, holds each
    received row's route weight;
  * rows whose index would reach the capacity A are not written; counts still
    include them, so overflow is visible from epRecvCounts;
  * the shared-expert term is weighted per k, literally as the [CV4] formula
    reads: acc += s_k * y_k + s_k * sharedX;
  * fp32 accumulation from +0.0 in ascending k, each multiply and add rounded
    separately to fp32, then fp32 -> bf16 round-to-nearest-even ([TL] combine
    weighted sum, CAST_RINT);
  * FFN: silu on columns [0, N/2) times columns [N/2, N); dynamic per-row
    symmetric int8 quantisation amax/127 with round-half-even and clip to
    +-127, decided in fp32; integer GEMMs exact; dequant/SwiGLU in float64.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional, Sequence

import numpy as np

# ----------------------------------------------------------------------------
# bf16 <-> fp32 (bit-level definitions)
# ----------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> float32: the bf16 bits are the top half of the fp32 word."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_rne(values: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even ([TL] combine, CAST_RINT).

    Adding 0x7FFF plus the lowest kept bit and truncating rounds the dropped
    16 bits to nearest with ties going to the even result.  NaN maps to the
    quiet NaN 0x7FC0 (sign kept).
    """
    u = np.ascontiguousarray(values, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = ((u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)).astype(np.uint32)
    nan = np.isnan(np.asarray(values, dtype=np.float32))
    if nan.any():
        sign = ((u >> np.uint64(16)) & np.uint64(0x8000)).astype(np.uint32)
        r = np.where(nan, sign | np.uint32(0x7FC0), r)
    return r.astype(np.uint16)


# ----------------------------------------------------------------------------
# Dispatch
# ----------------------------------------------------------------------------


@dataclass
class DispatchResult:
    """One destination rank's dispatch outputs (valid rows only)."""
    expand_x: np.ndarray          # [n_rows][H] uint16, n_rows = min(total, capacity)
    assist_info: np.ndarray       # [n_rows][3] int32 = (src, token, k)
    ep_recv_counts: np.ndarray    # [L*W] int32, inclusive, index le*W + src
    expert_token_nums: np.ndarray  # [L] int64
    counts: np.ndarray            # [L][W] int32 (per (le, src) histogram)
    total: int                    # number of routes received (may exceed capacity)
    expanded_row_idx: dict        # (src, token, k) -> row, for written rows
    dropped_ids: int = 0          # active routes (all sources) whose id is outside [0, E+Z+C)
    overflow_rows: int = 0        # max(0, total - capacity)
    expand_scales: Optional[np.ndarray] = None   # [n_rows] fp32 route weights, when scales were given


def route_active(mask: Optional[np.ndarray], t: int, k: int) -> bool:
    """Mask of one rank: None (all active), 1D [BS] per token, or 2D [BS][K] per route."""
    if mask is None:
        return True
    if mask.ndim == 1:
        return bool(mask[t])
    return bool(mask[t][k])


def local_routes(ids: np.ndarray, mask: Optional[np.ndarray], d: int, experts: int):
    """Active routes whose expert lives on rank d, as (le, s, t, k), enumerated in (s, t, k) order.

    Routing rule: expert e goes to rank e // L as local expert e % L
    ([TL] send loop).  Inactive tokens or routes send nothing ([CV4]
    xActiveMask: whether the token takes part in communication; 2D per
    route).  Ids outside [0, E) are not dispatched.
    """
    W, BS, K = ids.shape
    L = experts // W
    out = []
    for s in range(W):
        for t in range(BS):
            for k in range(K):
                if mask is not None and not route_active(mask[s], t, k):
                    continue
                e = int(ids[s][t][k])
                if 0 <= e < experts and e // L == d:
                    out.append((e % L, s, t, k))
    return out


def dropped_ids(ids: np.ndarray, mask: Optional[np.ndarray], n_ids: int) -> int:
    """Active routes of every source rank whose expert id lies outside [0, n_ids), n_ids = E + Z + C.

    Such an id names no routed, zero or copy expert ([CV4] parameter notes:
    the valid id ranges of routed, zero and copy experts), so the route is
    sent nowhere and takes no part in combine; the dispatch reports how many
    there were.  Inactive routes are not counted (they are not sent anyway).
    """
    W, BS, K = ids.shape
    n = 0
    for s in range(W):
        for t in range(BS):
            for k in range(K):
                if mask is not None and not route_active(mask[s], t, k):
                    continue
                e = int(ids[s][t][k])
                if e < 0 or e >= n_ids:
                    n += 1
    return n


def dispatch(x: Optional[np.ndarray], ids: np.ndarray, mask: Optional[np.ndarray],
             d: int, experts: int, capacity: int, zero_experts: int = 0, copy_experts: int = 0,
             scales: Optional[np.ndarray] = None) -> DispatchResult:
    """Expert-major dispatch for destination rank d.

    Rows are laid out by local expert, then source rank, then (token, k):
    bucket the (s, t, k)-ordered local routes stably by local expert
    ([TL] rank-within-expert = number of earlier routes with the same id,
    window slot per (src, expert), local copy in status-row order le*W + src;
    [PTO] Dispatch: a group's rows ordered by source rank).
    x may be None to compute the layout only.  With scales ([W][BS][K] fp32
    route weights) the result also carries expand_scales: each row's route
    weight, the weight that travels with the row ([CV4] expandScalesOptional,
    the dispatch's expandScales of shape (A,)).
    """
    W, BS, K = ids.shape
    L = experts // W
    routes = local_routes(ids, mask, d, experts)
    buckets: List[list] = [[] for _ in range(L)]
    for r in routes:
        buckets[r[0]].append(r)
    ordered = [r for b in buckets for r in b]

    counts = np.zeros((L, W), dtype=np.int32)
    for le, s, _, _ in ordered:
        counts[le, s] += 1
    ep_recv_counts = np.cumsum(counts.reshape(L * W), dtype=np.int64).astype(np.int32)
    expert_token_nums = counts.sum(axis=1).astype(np.int64)

    total = len(ordered)
    n_rows = min(total, capacity)
    assist = np.zeros((n_rows, 3), dtype=np.int32)
    rowmap = {}
    for row, (le, s, t, k) in enumerate(ordered[:n_rows]):
        assist[row] = (s, t, k)
        rowmap[(s, t, k)] = row
    if x is not None:
        H = x.shape[-1]
        ex = np.zeros((n_rows, H), dtype=np.uint16)
        for row, (le, s, t, k) in enumerate(ordered[:n_rows]):
            ex[row] = x[s][t]          # bitwise row copy ([TL] send loop row put)
    else:
        ex = np.zeros((n_rows, 0), dtype=np.uint16)
    esc = None
    if scales is not None:
        esc = np.zeros(n_rows, dtype=np.float32)
        for row, (le, s, t, k) in enumerate(ordered[:n_rows]):
            esc[row] = scales[s][t][k]
    return DispatchResult(ex, assist, ep_recv_counts, expert_token_nums, counts, total, rowmap,
                          dropped_ids(ids, mask, experts + zero_experts + copy_experts),
                          max(0, total - capacity), esc)


def dispatch_quant(x: np.ndarray, ids: np.ndarray, mask: Optional[np.ndarray], d: int, experts: int,
                   capacity: int, zero_experts: int = 0, copy_experts: int = 0, scales: Optional[np.ndarray] = None):
    """Quantised dispatch: the rows of dispatch(), each the per-row int8 quantisation of its token.

    [CV4] parameter notes: commQuantMode 2 quantises communicated rows to int8
    with a dynamic per-row scale; [PTO] FrontReorder Stage writes quantised
    token rows.  The quantiser is quant_rows (fp32 decisions).  Returns the
    DispatchResult and (codes [n][H] int8, scales [n] fp32).
    """
    res = dispatch(x, ids, mask, d, experts, capacity, zero_experts, copy_experts, scales)
    q, sc = quant_rows(bf16_to_f32(res.expand_x)) if res.expand_x.shape[0] else (
        np.zeros((0, x.shape[-1]), np.int8), np.zeros(0, np.float32))
    return res, q, sc


# ----------------------------------------------------------------------------
# Experts used by the tests in place of the FFN
# ----------------------------------------------------------------------------


def expert_identity(expand_x: np.ndarray, assist: np.ndarray, ids: np.ndarray, L: int) -> np.ndarray:
    return expand_x.copy()


def pow2_exponent(e: int) -> int:
    """Tag exponent of global expert e for the power-of-two test expert: (e mod 4) - 2."""
    return (e % 4) - 2


def expert_pow2(expand_x: np.ndarray, assist: np.ndarray, ids: np.ndarray, L: int) -> np.ndarray:
    """y = x * 2^((e mod 4) - 2), e the row's global expert (exact in bf16 for normal values).

    Makes a row landing on the wrong expert, or a swapped k, visible in the
    combined output.
    """
    if expand_x.shape[0] == 0:
        return expand_x.copy()
    e = ids[assist[:, 0], assist[:, 1], assist[:, 2]].astype(np.int64)
    f = 2.0 ** np.array([pow2_exponent(int(v)) for v in e], dtype=np.float64)
    prod = bf16_to_f32(expand_x).astype(np.float64) * f[:, None]
    return f32_to_bf16_rne(prod.astype(np.float32))


# ----------------------------------------------------------------------------
# Combine
# ----------------------------------------------------------------------------


def combine(segments_y: Sequence[np.ndarray], segments_assist: Sequence[np.ndarray], r: int,
            ids_r: np.ndarray, mask_r: Optional[np.ndarray], scales_r: np.ndarray,
            shared_r: Optional[np.ndarray], hidden: int, experts: Optional[int] = None,
            zero_experts: int = 0, copy_experts: int = 0, ori_r: Optional[np.ndarray] = None) -> np.ndarray:
    """Combine for source rank r: xOut[t] = sum_k ( s[t,k]*y[t,k] + s[t,k]*sharedX[t] ).

    segments_y[j] / segments_assist[j] are destination rank j's expert outputs
    and (src, token, k) triplets (valid rows only).  The expert output of route
    (r, t, k) is the row of some segment whose triplet is (r, t, k): data is
    returned along the dispatch path ([CV4] Function note; [TL] combine sends
    each row back to slot token*K + k of its source).  A route whose id is a
    zero expert (E <= e < E+Z) has output 0; a copy expert (E+Z <= e < E+Z+C)
    has output oriX[t] ([CV4] zeroExpertNum / copyExpertNum / oriXOptional).
    Any other route with no such row (inactive, dropped id, past capacity)
    contributes nothing; a masked-off route contributes nothing.

    Arithmetic ([TL] combine weighted sum; [CV4] formula): fp32 accumulator
    from +0.0, k ascending, a = s*y and b = s*sharedX each rounded to fp32,
    acc = acc + (a + b), then round-to-nearest-even to bf16.
    """
    BS, K = ids_r.shape
    where = {}
    for j, assist in enumerate(segments_assist):
        for row in range(assist.shape[0]):
            s, t, k = (int(v) for v in assist[row])
            if s == r:
                where[(t, k)] = (j, row)
    zero_row = np.zeros(hidden, dtype=np.uint16)
    out = np.zeros((BS, hidden), dtype=np.uint16)
    for t in range(BS):
        acc = np.zeros(hidden, dtype=np.float32)
        for k in range(K):
            if mask_r is not None and not route_active(mask_r, t, k):
                continue
            hit = where.get((t, k))
            if hit is not None:
                j, row = hit
                y = segments_y[j][row]
            else:
                e = int(ids_r[t][k])
                if experts is not None and experts <= e < experts + zero_experts:
                    y = zero_row
                elif experts is not None and experts + zero_experts <= e < experts + zero_experts + copy_experts:
                    y = ori_r[t]
                else:
                    continue
            sc = np.float32(scales_r[t][k])
            a = sc * bf16_to_f32(y)
            if shared_r is not None:
                b = sc * bf16_to_f32(shared_r[t])
                acc = acc + (a + b)
            else:
                acc = acc + a
        out[t] = f32_to_bf16_rne(acc)
    return out


# ----------------------------------------------------------------------------
# Grouped int8 expert FFN (PTO MegaMoE GMM1 -> SwiGLU -> GMM2)
# ----------------------------------------------------------------------------


def quant_rows(v: np.ndarray):
    """Dynamic per-row symmetric int8 quantisation, decided in fp32.

    amax = max |v| over the row; q = clip(rint(v * (127 / amax)), -127, 127)
    with round-half-even; the dequant scale is amax / 127.  A zero row gives
    q = 0 and scale 0.  ([PTO] SwiGLU: dynamic quantisation to int8 plus a
    per-token scale; the pages name the step but not its formula, so this is
    the plain symmetric reading.)
    """
    v = np.asarray(v, dtype=np.float32)
    amax = np.max(np.abs(v), axis=1).astype(np.float32)
    q = np.zeros(v.shape, dtype=np.int8)
    scale = np.zeros(v.shape[0], dtype=np.float32)
    nz = amax > 0
    inv = np.float32(127.0) / amax[nz]
    q[nz] = np.clip(np.rint(v[nz] * inv[:, None]), -127, 127).astype(np.int8)
    scale[nz] = amax[nz] / np.float32(127.0)
    return q, scale


def silu(a: np.ndarray) -> np.ndarray:
    return a / (1.0 + np.exp(-a))


def ffn(expand_x: np.ndarray, row_expert: np.ndarray, w1: np.ndarray, w1_scale: np.ndarray,
        w2: np.ndarray, w2_scale: np.ndarray) -> np.ndarray:
    """Per local expert: quant -> GMM1 (int) -> dequant -> SwiGLU -> quant -> GMM2 (int) -> bf16.

    [PTO] GMM1: int8 x int8 -> int32 -> scale1; SwiGLU: dequant by the
    per-token scale, silu(up)*gate, dynamic quant; GMM2: int8 x int8 -> int32
    -> scale2.  Integer products are summed exactly (float64 holds every
    partial sum: |sum| <= H * 127^2 < 2^53).
    """
    R, H = expand_x.shape
    N = w1.shape[1]
    y = np.zeros((R, H), dtype=np.uint16)
    xf = bf16_to_f32(expand_x)
    for le in np.unique(row_expert):
        rows = np.nonzero(row_expert == le)[0]
        q1, sc1 = quant_rows(xf[rows])
        acc1 = q1.astype(np.float64) @ w1[le].astype(np.float64).T
        h = acc1 * sc1.astype(np.float64)[:, None] * w1_scale[le].astype(np.float64)[None, :]
        g = silu(h[:, : N // 2]) * h[:, N // 2:]
        q2, sc2 = quant_rows(g.astype(np.float32))
        acc2 = q2.astype(np.float64) @ w2[le].astype(np.float64).T
        out = acc2 * sc2.astype(np.float64)[:, None] * w2_scale[le].astype(np.float64)[None, :]
        y[rows] = f32_to_bf16_rne(out.astype(np.float32))
    return y
