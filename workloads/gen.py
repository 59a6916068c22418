"""Seeded synthetic inputs for the MoE dispatch/combine path.

This module only draws random inputs. It holds none of the method's arithmetic
(no routing, ranking, scanning or combining), so both the CPU oracle and the
GPU path may take their inputs from it without sharing any of the method.

Workloads (sizes follow the shapes used on the PTO MegaMoE page, "Specification"
and "Supported Cases": worldSize=8, M=2048, hidden 7168, N=4096, topK=8,
expertPerRank=16; and the aclnnMoeDistributeCombineV4 page, "Function Prototype"
parameter table, for the tensor roles):

  tiny    1 virtual rank, 8 experts, BS=16, H=128, topK=2, identity expert,
          no shared expert
  share   one GPU's real share: 8 virtual source ranks x 2048 tokens, H=7168,
          128 experts (16 per rank), topK=8, shared expert present
  skewed  as share, experts drawn Zipf(s=1.2) without replacement in natural
          id order, 10% of tokens inactive (Bernoulli)
  decode  8 x 32 tokens, H=7168, 256 experts (32 per rank), topK=8, shared
  ffn     share routing plus int8 expert weights for GMM1 7168->4096 and
          GMM2 2048->7168 with per-channel fp32 scales U(1e-3, 1e-2)

Random streams come from numpy PCG64 seeded with
SeedSequence([20261202, workload_index, virtual_rank, stream]).
bf16 values are float32 N(0,1) draws rounded to bf16 by torch's CPU cast
(a library conversion, used only to make input data).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional

import numpy as np

SEED_ROOT = 20261202
STREAM = {"x": 0, "routes": 1, "scale_logits": 2, "mask": 3, "shared": 4,
          "weights": 5, "weight_scales": 6}


@dataclass(frozen=True)
class Workload:
    name: str
    index: int            # seed slot of this workload
    world: int            # W virtual EP ranks
    bs: int               # tokens per rank
    hidden: int           # H (bf16 elements per row)
    experts: int          # E routed experts (L = E / W per rank)
    topk: int             # K
    routing: str = "uniform"      # "uniform" | "zipf" | "first_k" | "tagged_shuffle"
    zipf_s: float = 1.2
    inactive_frac: float = 0.0    # Bernoulli fraction of inactive tokens (1D mask)
    shared: bool = False          # sharedExpertX present in combine
    inter: int = 0                # FFN intermediate N (0 = no FFN weights)
    zero_experts: int = 0         # Z: ids [E, E+Z) are zero experts (drawn like routed experts)
    copy_experts: int = 0         # C: ids [E+Z, E+Z+C) are copy experts
    route_mask_frac: float = 0.0  # >0: 2D mask [BS][K], each route off with this probability

    @property
    def local_experts(self) -> int:
        return self.experts // self.world

    @property
    def capacity(self) -> int:
        """Row capacity per rank, A = W * BS * min(L, K) (CombineV4 page, shape-variable table)."""
        return self.world * self.bs * min(self.local_experts, self.topk)


WORKLOADS = {
    "tiny": Workload("tiny", 0, 1, 16, 128, 8, 2),
    "share": Workload("share", 1, 8, 2048, 7168, 128, 8, shared=True),
    "skewed": Workload("skewed", 2, 8, 2048, 7168, 128, 8, routing="zipf",
                       inactive_frac=0.1, shared=True),
    "decode": Workload("decode", 3, 8, 32, 7168, 256, 8, shared=True),
    "ffn": Workload("ffn", 4, 8, 2048, 7168, 128, 8, shared=True, inter=4096),
    # share shapes with 8 zero and 8 copy experts drawn beside the 128 routed
    # ones and a per-route [BS][K] mask with 5% of the routes off
    "special": Workload("special", 5, 8, 2048, 7168, 128, 8, shared=True, zero_experts=8, copy_experts=8,
                        route_mask_frac=0.05),
}


def workload(name: str, **over) -> Workload:
    w = WORKLOADS[name]
    return replace(w, **over) if over else w


def rng(index: int, vrank: int, stream: str) -> np.random.Generator:
    ss = np.random.SeedSequence([SEED_ROOT, index, vrank, STREAM[stream]])
    return np.random.Generator(np.random.PCG64(ss))


def bf16_from_f32(a: np.ndarray) -> np.ndarray:
    """float32 array -> bf16 bit patterns (uint16) via torch's CPU cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def normal_bf16(g: np.random.Generator, shape) -> np.ndarray:
    return bf16_from_f32(g.standard_normal(shape, dtype=np.float32))


def draw_routes(w: Workload, vrank: int) -> np.ndarray:
    """expertIds [BS][K] int32 for one virtual rank."""
    g = rng(w.index, vrank, "routes")
    n_ids = w.experts + w.zero_experts + w.copy_experts
    if w.routing == "uniform":
        # first K of a uniform random permutation = K distinct ids, uniform over
        # routed and special experts
        keys = g.random((w.bs, n_ids))
        return np.argsort(keys, axis=1, kind="stable")[:, :w.topk].astype(np.int32)
    if w.routing == "zipf":
        # successive sampling without replacement with p(e) ~ (e+1)^-s,
        # drawn as Gumbel-top-K (the same distribution as drawing one at a time
        # and renormalising)
        logp = -w.zipf_s * np.log(np.arange(1, w.experts + 1, dtype=np.float64))
        keys = logp[None, :] + g.gumbel(size=(w.bs, w.experts))
        return np.argsort(-keys, axis=1, kind="stable")[:, :w.topk].astype(np.int32)
    if w.routing == "first_k":
        # every token routes to experts 0..K-1 (the A2 sample on the CombineV4 page)
        return np.tile(np.arange(w.topk, dtype=np.int32), (w.bs, 1))
    if w.routing == "round_robin":
        # global token round robin over experts (the PTO MegaMoE page's synthetic note)
        base = (vrank * w.bs + np.arange(w.bs, dtype=np.int64))[:, None] * w.topk
        return ((base + np.arange(w.topk)[None, :]) % w.experts).astype(np.int32)
    raise ValueError(w.routing)


def draw_scales(w: Workload, vrank: int) -> np.ndarray:
    """expertScales [BS][K] float32 = softmax over K of N(0,1) logits, in float64."""
    g = rng(w.index, vrank, "scale_logits")
    z = g.standard_normal((w.bs, w.topk))
    z = np.exp(z - z.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


def draw_mask(w: Workload, vrank: int) -> Optional[np.ndarray]:
    """xActiveMask: 2D [BS][K] per route when route_mask_frac > 0, else 1D [BS]
    per token when inactive_frac > 0 (uint8 0/1), else None (all active)."""
    g = rng(w.index, vrank, "mask")
    if w.route_mask_frac > 0.0:
        m = (g.random((w.bs, w.topk)) >= w.route_mask_frac).astype(np.uint8)
        if w.inactive_frac > 0.0:
            m[g.random(w.bs) < w.inactive_frac, :] = 0     # whole tokens off
        return m
    if w.inactive_frac <= 0.0:
        return None
    return (g.random(w.bs) >= w.inactive_frac).astype(np.uint8)


@dataclass
class RankInputs:
    x: np.ndarray                    # bf16 bits [BS][H] uint16
    ids: np.ndarray                  # [BS][K] int32
    scales: np.ndarray               # [BS][K] float32
    mask: Optional[np.ndarray]       # [BS] uint8 or None
    shared: Optional[np.ndarray]     # bf16 bits [BS][H] or None


def rank_inputs(w: Workload, vrank: int, with_x: bool = True) -> RankInputs:
    x = normal_bf16(rng(w.index, vrank, "x"), (w.bs, w.hidden)) if with_x else None
    sh = normal_bf16(rng(w.index, vrank, "shared"), (w.bs, w.hidden)) if w.shared else None
    return RankInputs(x=x, ids=draw_routes(w, vrank), scales=draw_scales(w, vrank),
                      mask=draw_mask(w, vrank), shared=sh)


@dataclass
class World:
    w: Workload
    x: np.ndarray                    # [W][BS][H] uint16 (bf16 bits)
    ids: np.ndarray                  # [W][BS][K] int32
    scales: np.ndarray               # [W][BS][K] float32
    mask: Optional[np.ndarray]       # [W][BS] uint8 or None
    shared: Optional[np.ndarray]     # [W][BS][H] uint16 or None


def world_inputs(w: Workload) -> World:
    ranks = [rank_inputs(w, s) for s in range(w.world)]
    return World(
        w=w,
        x=np.stack([r.x for r in ranks]),
        ids=np.stack([r.ids for r in ranks]),
        scales=np.stack([r.scales for r in ranks]),
        mask=None if ranks[0].mask is None else np.stack([r.mask for r in ranks]),
        shared=None if ranks[0].shared is None else np.stack([r.shared for r in ranks]),
    )


@dataclass
class FfnWeights:
    w1: np.ndarray      # int8 [L][N][H]     (GMM1: H -> N)
    w1_scale: np.ndarray  # float32 [L][N]
    w2: np.ndarray      # int8 [L][H][N/2]   (GMM2: N/2 -> H)
    w2_scale: np.ndarray  # float32 [L][H]


def ffn_weights(w: Workload, rank: int = 0, inter: Optional[int] = None) -> FfnWeights:
    n = inter or w.inter
    L, H = w.local_experts, w.hidden
    g = rng(w.index, rank, "weights")
    w1 = g.integers(-127, 128, size=(L, n, H), dtype=np.int8)
    w2 = g.integers(-127, 128, size=(L, H, n // 2), dtype=np.int8)
    gs = rng(w.index, rank, "weight_scales")
    s1 = gs.uniform(1e-3, 1e-2, size=(L, n)).astype(np.float32)
    s2 = gs.uniform(1e-3, 1e-2, size=(L, H)).astype(np.float32)
    return FfnWeights(w1, s1, w2, s2)
