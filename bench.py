#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine, one GPU's share, on one MI355X.

One step = one pass of the hot path over one batch of synthetic input that is
already resident in HBM:
    mdc_dispatch_layout + mdc_dispatch_gather for destination rank 0 (reading
    the tokens of all 8 virtual source ranks), then mdc_combine for source
    rank 0 (reading the expert outputs of all 8 virtual destination ranks).
The expert between them is the identity (the combine reads the dispatched
rows), as in the workload definition.  Expert outputs of ranks 1..7 are
produced by their own dispatch calls before the timed region.

Several copies of every input buffer are rotated (--batches) so that no step
finds its inputs in the 256 MB Infinity Cache left there by the previous step.

Output: one JSON line with the metric, the roofline of the dominant kernel
(achieved algorithmic GB/s measured with HIP events on the launch stream
against the 8 TB/s HBM peak), per-kernel times and the CPU oracle's rate on
the same workload (cpu_baseline).
"""
from __future__ import annotations

import argparse
import gc
import json
import os
import statistics
import sys
import time
from dataclasses import replace

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch+combine tokens/s and achieved HBM GB/s (% of peak) on 1 MI355X"
HBM_PEAK_GBPS = 8000.0

DESCR = {
    "share": "one GPU's share: 8 virtual source ranks x 2048 tokens, H=7168 bf16, 128 experts (16 local), "
             "top-8 uniform distinct routes, fp32 softmax scales, shared expert, identity expert",
    "skewed": "share shapes with Zipf(1.2) routes and 10% inactive tokens",
    "decode": "8 virtual ranks x 32 tokens, H=7168, 256 experts (32 local), top-8, shared expert",
    "tiny": "1 virtual rank, 8 experts, 16 tokens, H=128, top-2",
    "ffn": "share routing, then per local expert int8 GMM1 7168->4096, SwiGLU + dynamic int8 quant, "
           "int8 GMM2 2048->7168 (mdc_ffn) on destination 0's rows, then combine",
    "special": "share shapes with 8 zero and 8 copy experts among the 144 ids drawn, a per-route [BS][K] "
               "mask with 5% of routes off, shared expert, identity expert",
}
INT8_PEAK_TOPS = 5000.0  # MI355X dense int8 MFMA


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="share", choices=sorted(DESCR))
    ap.add_argument("--batches", type=int, default=2, help="rotated copies of every input buffer")
    ap.add_argument("--event-samples", type=int, default=10,
                    help="timed steps that carry per-kernel HIP events (spread evenly, the first timed step "
                         "excluded)")
    ap.add_argument("--breakdown-steps", type=int, default=20,
                    help="steps of the per-kernel breakdown pass after the timed region")
    ap.add_argument("--no-ceilings", action="store_true", help="skip the memory-ceiling leg")
    ap.add_argument("--ceiling-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="oracle timing budget")
    ap.add_argument("--ffn-path", default="kernels", choices=("kernels", "fused", "pipeline"),
                    help="ffn workload: quantised gather then the FFN's stream-ordered kernels (mdc_dispatch_quant_"
                         "gather + mdc_ffn_quant_input); the same with the FFN as one persistent kernel "
                         "(MDC_FLAG_FFN_PIPELINE); or the dispatch and FFN as one pipeline (mdc_dispatch_ffn)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run three 256 MiB device copies (counter calibration)")
    return ap.parse_args()


def algorithmic_bytes(w, ids, mask, d=0, r=0):
    """What the method must move for one step (dispatch share d, combine share r).

    With the FFN workload the dispatch writes int8 rows plus a 4-byte scale.
    Zero-expert routes read nothing; copy-expert routes read the token's
    original row once per token.
    """
    import numpy as np
    W, BS, K = ids.shape
    L = w.experts // W
    H2 = 2 * w.hidden
    n_ids = w.experts + w.zero_experts + w.copy_experts
    if mask is None:
        act = np.ones((W, BS, K), bool)
    elif mask.ndim == 2:
        act = np.broadcast_to(mask.astype(bool)[:, :, None], (W, BS, K))
    else:
        act = mask.astype(bool)
    valid = (ids >= 0) & (ids < w.experts) & act
    local = valid & ((ids // L) == d)
    R = int(local.sum())                      # routed rows written on rank d
    U = int(local.any(axis=2).sum())          # distinct source tokens read
    present_r = (ids[r] >= 0) & (ids[r] < n_ids) & act[r]
    routed_r = int(valid[r].sum())            # routes of rank r that read an expert row
    copy_tok = int((present_r & (ids[r] >= w.experts + w.zero_experts)).any(axis=1).sum())
    tok_any = int(present_r.any(axis=1).sum())
    mask_bytes = 0 if mask is None else mask.size
    layout = ids.size * 4 + mask_bytes + L * W * 4 + L * 8
    gather = U * H2 + R * ((w.hidden + 4 if w.inter else H2) + 12 + 4) + ids.size * 4
    combine = (routed_r * H2 + BS * K * 12 + mask_bytes // W + copy_tok * H2
               + (tok_any * H2 if w.shared else 0) + BS * H2)
    return {"R": R, "U": U, "present": int(present_r.sum()), "layout": layout, "gather": gather,
            "combine": combine}


# sources of the dispatch/combine kernels (the ones the HBM-traffic summaries measure)
TRAFFIC_SOURCES = ("mdc_common.h", "mdc_route.h", "mdc_dispatch.hip")


def dispatch_source_sha(sources=TRAFFIC_SOURCES) -> str:
    """sha256 over the named kernel sources, in the given order."""
    import hashlib
    h = hashlib.sha256()
    for name in sources:
        h.update(open(os.path.join(ROOT, "combine_route_histogram_amd", "csrc", name), "rb").read())
    return h.hexdigest()


def measured_traffic(workload: str, kernels):
    """HBM bytes per launch from the committed counter summary, or None.

    `kernels` is a kernel-name prefix, or a tuple of prefixes whose per-launch
    bytes are summed (one launch of each, as one library call makes them).
    The summary records the sha256 of the kernel sources it was measured on
    (its `sources`, by default TRAFFIC_SOURCES); once they differ the figure
    no longer describes these kernels.
    """
    path = os.path.join(ROOT, "profiles", f"{workload}_hbm_traffic.json")
    try:
        prof = json.load(open(path))
        sha = dispatch_source_sha(tuple(prof.get("sources", TRAFFIC_SOURCES)))
    except (OSError, ValueError):
        return None
    if prof.get("source_sha256") != sha:
        return None
    total = 0.0
    for prefix in ((kernels,) if isinstance(kernels, str) else kernels):
        recs = [rec for name, rec in prof.get("kernels", {}).items() if name.startswith(prefix)]
        if len(recs) != 1:
            return None
        total += recs[0]["traffic_bytes"]
    return int(round(total))


def pct(v, q):
    """q-th percentile (linear interpolation) of a list."""
    v = sorted(v)
    if not v:
        return None
    x = (len(v) - 1) * q / 100.0
    lo = int(x)
    hi = min(lo + 1, len(v) - 1)
    return v[lo] + (v[hi] - v[lo]) * (x - lo)


def spread(samples_us):
    return {"median": round(statistics.median(samples_us), 3), "p10": round(pct(samples_us, 10), 3),
            "p90": round(pct(samples_us, 90), 3), "n": len(samples_us)}


class HipEvents:
    """Timing events created with hipEventDisableSystemFence through the HIP runtime torch loaded.

    A default event (torch.cuda.Event) writes back and invalidates the caches
    when it is recorded, which costs about 2.5 us of GPU time per event between
    kernels; an event without the system-scope fence only takes a timestamp,
    which is all a duration needs.
    """
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes
        self.ct = ctypes
        self.hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime already loaded by torch (same SONAME)
        self.hip.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p, ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.made = []

    def make(self):
        e = self.ct.c_void_p()
        st = self.hip.hipEventCreateWithFlags(self.ct.byref(e), self.DISABLE_SYSTEM_FENCE)
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({st})")
        self.made.append(e)
        return e

    def pair(self):
        return [self.make(), self.make()]

    def five(self):
        return [self.make() for _ in range(5)]

    def record(self, e, stream):
        if self.hip.hipEventRecord(e, stream.cuda_stream) != 0:
            raise RuntimeError("hipEventRecord failed")

    def elapsed_us(self, a, b):
        f = self.ct.c_float()
        if self.hip.hipEventElapsedTime(self.ct.byref(f), a, b) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return f.value * 1e3

    def __del__(self):
        try:
            for e in self.made:
                self.hip.hipEventDestroy(e)
        except Exception:   # interpreter shutdown: the runtime may already be gone
            pass


def ceiling_leg(torch, mdc, w, wi, batches, stream, reps):
    """Memory ceilings measured with the committed probe kernels (libmdc_probe), timed like the bench's kernels.

    Each probe launch is bracketed by two fence-free HIP events on the launch
    stream, after an untimed 512 MiB write that flushes the 256 MB Infinity Cache.  Streaming
    ceilings: 1 GiB read-only, 1 GiB write-only, 1 GiB copy (2 GiB moved).
    Pattern probes (dispatch/combine workloads): the gather's read half (the U
    distinct source rows), its write half (the R rows in the gather's
    token-major fan-out order), both in one kernel (each source row read once
    and written to its rows), and the combine's pattern (each token's present
    rows, each destination's in its own memory region, plus one more row read,
    one row written) at the workload's own sizes.
    """
    import numpy as np
    from combine_route_histogram_amd import probe
    dev = "cuda:0"
    st = stream.cuda_stream
    GiB = 1 << 30
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1024, dtype=torch.int32, device=dev)

    hip_ev = HipEvents()

    def timed(fn):
        out = []
        for i in range(reps + 2):
            probe.write(flush, flush.numel(), i, st)
            a, b = hip_ev.pair()
            hip_ev.record(a, stream)
            fn()
            hip_ev.record(b, stream)
            torch.cuda.synchronize()
            if i >= 2:
                out.append(hip_ev.elapsed_us(a, b))
        return out

    res = {}
    src = torch.empty(GiB, dtype=torch.uint8, device=dev)
    dst = torch.empty(GiB, dtype=torch.uint8, device=dev)
    probe.write(src, GiB, 1, st)
    for name, nbytes, fn in (("read_1GiB", GiB, lambda: probe.read(src, GiB, sink, st)),
                             ("write_1GiB", GiB, lambda: probe.write(dst, GiB, 3, st)),
                             ("copy_1GiB", 2 * GiB, lambda: probe.copy(src, dst, GiB, st))):
        t = timed(fn)
        rate = [nbytes / (x * 1e-6) / 1e9 for x in t]
        res[name] = {"bytes": nbytes, "us": spread(t), "gbps": round(statistics.median(rate), 1),
                     "gbps_p10": round(pct(rate, 10), 1), "gbps_p90": round(pct(rate, 90), 1)}
    del src, dst

    pats = None
    if not w.inter and w.name not in ("tiny",):
        H2 = 2 * w.hidden
        bt = batches[0]
        o0 = bt["outs"][0]
        # destination 0's dispatch of batch 0, so that its rows and triplets describe the step's pattern
        if bt["layout"] is not None:
            bt["layout"]()
        bt["gather"]()
        torch.cuda.synchronize()
        R = int(o0["ep_recv_counts"][-1].item())
        R = min(R, w.capacity)
        tri = o0["assist_info"][:R].cpu().numpy().astype(np.int64)
        tok = tri[:, 0] * w.bs + tri[:, 1]
        order = np.lexsort((tri[:, 2], tok))          # token-major, k ascending: the gather's write order
        tok_s, rows_s = tok[order], np.arange(R)[order]
        uniq, start = np.unique(tok_s, return_index=True)
        off = torch.from_numpy(np.concatenate([start, [R]]).astype(np.int32)).to(dev)
        src_rows = torch.from_numpy(uniq.astype(np.int32)).to(dev)
        dst_rows = torch.from_numpy(rows_s.astype(np.int32)).to(dev)
        xflat = bt["x"]
        spare = batches[1 % len(batches)]["outs"][0]["expand_x"]
        t_r = timed(lambda: probe.rows_read(xflat, src_rows, H2, sink, st))
        t_w = timed(lambda: probe.rows_write(spare, off, dst_rows, H2, st))
        t_f = timed(lambda: probe.rows_fanout(xflat, src_rows, off, dst_rows, spare, H2, st))
        # combine pattern: rank 0's routes read the rows they read in the step (row numbers within the
        # destination's buffer), here all from one buffer of the same size
        row0 = bt["row0"].cpu().numpy()
        ids0 = bt["ids0"].cpu().numpy()
        L = w.experts // w.world
        # destination j's rows live in region j of one buffer (regions sized by each destination's
        # received rows), so that, as in the step, rows of different destinations are different memory
        recv = np.array([min(int(o["ep_recv_counts"][-1].item()), w.capacity) for o in bt["outs"]], np.int64)
        start_j = np.concatenate([[0], np.cumsum(recv)[:-1]])
        dest = np.where((ids0 >= 0) & (ids0 < w.experts), ids0 // L, 0)
        ok = (ids0 >= 0) & (ids0 < w.experts) & (row0 >= 0) & (row0 < recv[dest])
        flat = start_j[dest] + row0
        ok &= flat < w.capacity
        rr = np.where(ok, flat, -1).astype(np.int32)
        if bt["mask0"] is not None:
            m0 = bt["mask0"].cpu().numpy().astype(bool)
            rr = np.where(m0 if m0.ndim == 2 else m0[:, None], rr, -1).astype(np.int32)
        rows_k = torch.from_numpy(np.ascontiguousarray(rr)).to(dev)
        own = bt["shared0"] if bt["shared0"] is not None else bt["x"][0]
        out = torch.empty_like(bt["x_out"])
        t_c = timed(lambda: probe.rows_reduce(bt["outs"][1]["expand_x"], rows_k, w.topk, own, out, H2, st))
        n_read = int((rr >= 0).sum())
        pats = {
            "gather_read_us": spread(t_r), "gather_read_bytes": len(uniq) * H2,
            "gather_write_us": spread(t_w), "gather_write_bytes": R * H2,
            "gather_read_plus_write_us": round(statistics.median(t_r) + statistics.median(t_w), 3),
            "gather_fanout_us": spread(t_f), "gather_fanout_bytes": (len(uniq) + R) * H2,
            "combine_pattern_us": spread(t_c), "combine_pattern_bytes": (n_read + 2 * w.bs) * H2,
            "what": "plain probe kernels (libmdc_probe) of each kernel's access pattern at this workload's sizes, "
                    "no metadata work; median of fence-free HIP-event durations with the Infinity Cache flushed",
        }
    del flush
    torch.cuda.synchronize()
    return res, pats


def cpu_baseline(wi, w, budget_s, fw=None):
    """Time the oracle (as it stands) on dispatch share 0 (+ FFN) + combine share 0 of the same workload."""
    import numpy as np
    from oracle import mdc_oracle as O
    segs = [O.dispatch(wi.x, wi.ids, wi.mask, d, w.experts, w.capacity) for d in range(w.world)]
    rates = []
    t_end = time.perf_counter() + budget_s
    reps = 0
    out = None
    while reps < 1 or (time.perf_counter() < t_end and reps < 20):
        t0 = time.perf_counter()
        s0 = O.dispatch(wi.x, wi.ids, wi.mask, 0, w.experts, w.capacity)
        y0 = s0.expand_x
        if fw is not None:
            n = s0.assist_info.shape[0]
            row_expert = np.repeat(np.arange(w.local_experts), s0.expert_token_nums)[:n]
            y0 = O.ffn(s0.expand_x, row_expert, fw.w1, fw.w1_scale, fw.w2, fw.w2_scale)
        ys = [y0] + [s.expand_x for s in segs[1:]]
        out = O.combine(ys, [s0.assist_info] + [s.assist_info for s in segs[1:]], 0, wi.ids[0],
                        None if wi.mask is None else wi.mask[0], wi.scales[0],
                        None if wi.shared is None else wi.shared[0], w.hidden, experts=w.experts,
                        zero_experts=w.zero_experts, copy_experts=w.copy_experts,
                        ori_r=wi.x[0] if w.copy_experts else None)
        rates.append(w.bs / (time.perf_counter() - t0))
        reps += 1
    what = "dispatch share 0 + FFN + combine share 0" if fw is not None else "dispatch share 0 + combine share 0"
    cores = 1
    if fw is not None:
        cores = os.cpu_count() or 1   # the FFN's float64 matrix products run on every host core (BLAS)
    return {"value": statistics.median(rates), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"the full timed step ({what} of the {w.name} workload), {reps} repetitions, median; "
                      f"numpy elementwise work on one thread"}, segs, out


def graph_replay_us(mdc, torch, shape, batches, replays):
    """Per-step time of the one-shot dispatch + combine replayed from a HIP graph.

    One graph holds one step per batch copy (launched on the capture stream);
    it is replayed back to back and the wall-clock time is divided by the steps.
    """
    cs = torch.cuda.Stream()
    calls = []
    for bt in batches:
        o0 = bt["outs"][0]
        calls.append(mdc.prepare_dispatch(shape, bt["x"], bt["ids"], bt["mask"], o0["expand_x"], o0["assist_info"],
                                          o0["ep_recv_counts"], o0["expert_token_nums"], bt["row_idx"],
                                          o0["workspace"], cs))
        calls.append(mdc.prepare_combine(shape, [o["expand_x"] for o in bt["outs"]],
                                         [o["assist_info"] for o in bt["outs"]],
                                         [o["ep_recv_counts"] for o in bt["outs"]], bt["row0"], bt["ids0"],
                                         bt["scales0"], bt["mask0"], bt["shared0"], bt["x_out"], stream=cs))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cs):
        for c in calls:
            c()
    torch.cuda.synchronize()
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(replays):
        g.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e6 / (replays * len(batches))


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on one GPU only (asked for --gpus {args.gpus}); the expert-parallel "
              "ranks are virtual buffers on that GPU. Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import combine_route_histogram_amd as mdc
    from workloads import gen

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = "cuda:0"
    torch.cuda.set_device(0)
    w = gen.workload(args.workload)
    print(f"[bench] generating {w.name} inputs", file=sys.stderr, flush=True)
    wi = gen.world_inputs(w)
    W, BS, K, H = w.world, w.bs, w.topk, w.hidden
    shape = mdc.Shape(W, 0, BS, H, K, w.experts, w.capacity, mask_per_route=1 if w.route_mask_frac > 0 else 0,
                      zero_experts=w.zero_experts, copy_experts=w.copy_experts)
    stream = torch.cuda.current_stream()

    def bf16(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)

    # ---- one set of device buffers per batch copy --------------------------------------------
    batches = []
    for b in range(args.batches):
        x = bf16(wi.x)
        ids = torch.from_numpy(wi.ids).to(dev)
        mask = None if wi.mask is None else torch.from_numpy(wi.mask).to(dev)
        scales0 = torch.from_numpy(wi.scales[0]).to(dev)
        shared0 = None if wi.shared is None else bf16(wi.shared[0])
        row_idx = torch.full((W, BS, K), -1, dtype=torch.int32, device=dev)
        outs = [mdc.alloc_dispatch_outputs(shape.with_rank(d), dev) for d in range(W)]
        for d in range(1, W):     # expert outputs of the other ranks (identity expert), untimed
            o = outs[d]
            mdc.mdc_dispatch(shape.with_rank(d), x, ids, mask, o["expand_x"], o["assist_info"],
                             o["ep_recv_counts"], o["expert_token_nums"], row_idx, o["workspace"])
        x_out = torch.empty((BS, H), dtype=torch.bfloat16, device=dev)
        if w.inter:
            outs[0]["y"] = torch.empty_like(outs[0]["expand_x"])
            outs[0]["expand_q"] = torch.empty((w.capacity, H), dtype=torch.int8, device=dev)
            outs[0]["dyn_scales"] = torch.empty((w.capacity,), dtype=torch.float32, device=dev)
        batches.append(dict(x=x, ids=ids, mask=mask, scales0=scales0, shared0=shared0, row_idx=row_idx,
                            outs=outs, x_out=x_out, ids0=ids[0].contiguous(), mask0=None if mask is None
                            else mask[0].contiguous(), row0=row_idx[0]))
    torch.cuda.synchronize()

    ffn_w = None
    if w.inter:
        print("[bench] generating int8 expert weights", file=sys.stderr, flush=True)
        fw = gen.ffn_weights(w, rank=0)
        ffn_w = [torch.from_numpy(a).to(dev) for a in (fw.w1, fw.w1_scale, fw.w2, fw.w2_scale)]
        ffn_ws = torch.empty(mdc.mdc_ffn_workspace_size(shape, w.inter), dtype=torch.uint8, device=dev)
        del fw

    # Arguments are marshalled once per batch so the host loop stays ahead of the GPU.
    # The launch-bound decode-size workloads dispatch with the one-shot call, which
    # runs the whole dispatch as one kernel at these sizes; the others use the two
    # stages so the rank and gather kernels are timed apart.
    one_shot = w.name in ("decode", "tiny")
    pipelined = bool(w.inter) and args.ffn_path == "pipeline"
    for bt in batches:
        o0 = bt["outs"][0]
        bt["layout"] = mdc.prepare_dispatch_layout(shape, bt["ids"], bt["mask"], o0["workspace"], stream)
        if one_shot:
            bt["layout"] = None
            bt["gather"] = mdc.prepare_dispatch(shape, bt["x"], bt["ids"], bt["mask"], o0["expand_x"],
                                                o0["assist_info"], o0["ep_recv_counts"], o0["expert_token_nums"],
                                                bt["row_idx"], o0["workspace"], stream)
        elif w.inter and pipelined:
            bt["gather"] = None   # the dispatch runs inside the FFN pipeline
        elif w.inter:
            # the FFN workload dispatches int8 rows with per-row scales and feeds them to the FFN
            bt["gather"] = mdc.prepare_dispatch_quant_gather(shape, bt["x"], o0["expand_q"], o0["dyn_scales"],
                                                             o0["assist_info"], o0["ep_recv_counts"],
                                                             o0["expert_token_nums"], bt["row_idx"],
                                                             o0["workspace"], stream)
        else:
            bt["gather"] = mdc.prepare_dispatch_gather(shape, bt["x"], o0["expand_x"], o0["assist_info"],
                                                       o0["ep_recv_counts"], o0["expert_token_nums"],
                                                       bt["row_idx"], o0["workspace"], stream)
        seg0 = o0["expand_x"]
        bt["ffn"] = None
        if ffn_w is not None and pipelined:
            bt["ffn"] = mdc.prepare_dispatch_ffn(shape, w.inter, bt["x"], o0["expand_q"], o0["dyn_scales"],
                                                 o0["assist_info"], o0["ep_recv_counts"], o0["expert_token_nums"],
                                                 bt["row_idx"], *ffn_w, o0["y"], o0["workspace"], ffn_ws, stream)
            seg0 = o0["y"]
        elif ffn_w is not None:
            fsh = replace(shape, flags=mdc.MDC_FLAG_FFN_PIPELINE) if args.ffn_path == "fused" else shape
            bt["ffn"] = mdc.prepare_ffn_quant_input(fsh, w.inter, o0["expand_q"], o0["dyn_scales"],
                                                    o0["expert_token_nums"], *ffn_w, o0["y"], ffn_ws, stream)
            seg0 = o0["y"]
        bt["combine"] = mdc.prepare_combine(shape, [seg0] + [o["expand_x"] for o in bt["outs"][1:]],
                                            [o["assist_info"] for o in bt["outs"]],
                                            [o["ep_recv_counts"] for o in bt["outs"]], bt["row0"], bt["ids0"],
                                            bt["scales0"], bt["mask0"], bt["shared0"], bt["x_out"],
                                            stream=stream, ori_x=bt["x"][0] if w.copy_experts else None)

    hip_ev = HipEvents()
    dom_stage = "ffn" if w.inter else "gather"   # the kernel the roofline is quoted on

    def step(bt, ev=None, bracket=None):
        """One step; ev = events to record: around stage `bracket` only (2), or around every stage (5)."""
        def rec(k):
            if ev is not None and k < len(ev):
                hip_ev.record(ev[k], stream)
        if ev is None or bracket is not None:
            if bt["layout"] is not None:
                bt["layout"]()
            if bracket == "gather":
                rec(0)
            if bt["gather"] is not None:
                bt["gather"]()
            if bracket == "gather":
                rec(1)
            if bt["ffn"] is not None:
                if bracket == "ffn":
                    rec(0)
                bt["ffn"]()
                if bracket == "ffn":
                    rec(1)
            bt["combine"]()
            return
        rec(0)
        if bt["layout"] is not None:
            bt["layout"]()
        rec(1)
        if bt["gather"] is not None:
            bt["gather"]()
        rec(2)
        if bt["ffn"] is not None:
            bt["ffn"]()
        rec(4)
        bt["combine"]()
        rec(3)

    ceil, pats = (None, None)
    if not args.no_ceilings:
        # also brings the GPU to its working clocks before the warmup
        print("[bench] memory-ceiling leg", file=sys.stderr, flush=True)
        ceil, pats = ceiling_leg(torch, mdc, w, wi, batches, stream, args.ceiling_reps)

    if args.calibrate_copy:
        # plain copy kernel of known size, for scaling the FETCH_SIZE / WRITE_SIZE counters
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    print(f"[bench] warmup {args.warmup} steps", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(batches[i % args.batches])
    torch.cuda.synchronize()

    # The dominant kernel is bracketed by two HIP events on the launch stream on
    # about --event-samples timed steps, spread evenly and never on the first
    # timed step (it starts from an idle queue, right after a synchronisation).
    # The events skip the system-scope fence (no cache write-back at the
    # event), so a bracketed step runs about as fast as the others; the
    # wall-clock total covers all steps.
    every = max(1, (args.steps - 1 + args.event_samples - 1) // max(1, args.event_samples))
    evs = {i: hip_ev.pair() for i in range(1, args.steps, every)}
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    gc.collect()
    gc.disable()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(batches[i % args.batches], evs.get(i), dom_stage)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    gc.enable()
    evs_idx = sorted(evs.keys())
    t_dom = [hip_ev.elapsed_us(evs[i][0], evs[i][1]) for i in evs_idx]

    # Per-kernel breakdown: a separate pass after the timed region, every step
    # carrying events around each stage (these steps are not part of `value`).
    br = [hip_ev.five() for _ in range(args.breakdown_steps)]
    torch.cuda.synchronize()
    for i, ev in enumerate(br):
        step(batches[i % args.batches], ev)
    torch.cuda.synchronize()
    t_layout = [hip_ev.elapsed_us(e[0], e[1]) for e in br]     # us
    t_gather = [hip_ev.elapsed_us(e[1], e[2]) for e in br]
    t_ffn = [hip_ev.elapsed_us(e[2], e[4]) for e in br]
    t_comb = [hip_ev.elapsed_us(e[4], e[3]) for e in br]
    t_step_ev = [hip_ev.elapsed_us(e[0], e[3]) for e in br]
    if dom_stage == "gather":
        t_gather_timed, t_ffn_timed = t_dom, t_ffn
    else:
        t_gather_timed, t_ffn_timed = t_gather, t_dom
    ms_per_step = elapsed * 1e3 / args.steps
    by = algorithmic_bytes(w, wi.ids, wi.mask)
    step_bytes = by["layout"] + by["gather"] + by["combine"]
    mean = statistics.fmean
    med = statistics.median
    gb_step = step_bytes / (ms_per_step * 1e-3) / 1e9
    if one_shot:
        # one launch (k_dispatch_small) does the layout and the gather
        d_kernel, d_bytes = "k_dispatch_small", by["layout"] + by["gather"]
    else:
        d_kernel, d_bytes = ("k_dispatch_gather_q" if w.inter else "k_dispatch_gather"), by["gather"]
    gb_gather = d_bytes / (med(t_gather_timed) * 1e-6) / 1e9
    gb_comb = by["combine"] / (med(t_comb) * 1e-6) / 1e9
    dom = (d_kernel, gb_gather, d_bytes, med(t_gather_timed), t_gather_timed)
    graph_info = None
    if one_shot:
        # launch-bound workloads: the same step replayed from a HIP graph
        graph_info = {"us_per_step": round(graph_replay_us(mdc, torch, shape, batches, args.steps), 3),
                      "replays": args.steps, "steps_per_graph": args.batches,
                      "what": "mdc_dispatch + mdc_combine captured once per batch copy, graph replayed back to back"}
    ffn_info = None
    if w.inter:
        ops = 2.0 * by["R"] * (w.inter * H + H * (w.inter // 2))
        tops = ops / (statistics.median(t_ffn_timed) * 1e-6) / 1e12
        ffn_info = {"us": round(statistics.median(t_ffn_timed), 2), "mean_us": round(mean(t_ffn_timed), 2),
                    "spread_us": spread(t_ffn_timed), "int8_ops": ops, "tops": round(tops, 1),
                    "mfma_frac": round(tops / INT8_PEAK_TOPS, 4)}

    roofline = {"bound": "hbm", "kernel": dom[0], "achieved": round(dom[1], 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(dom[1] / HBM_PEAK_GBPS, 4),
                "traffic": measured_traffic(w.name, dom[0]),
                "bytes_per_launch": dom[2], "avg_launch_us": round(dom[3], 3),
                "launch_us": spread(dom[4]),
                "launch_time_from": "median of two fence-free HIP events on the launch stream around the kernel, "
                                    f"on timed steps {evs_idx[:3]}..{evs_idx[-1:]} (never the first)"}
    if ceil is not None:
        roofline["frac_of_copy_ceiling"] = round(dom[1] / ceil["copy_1GiB"]["gbps"], 4)
    if ffn_info is not None and pipelined:
        roofline = {"bound": "mfma", "kernel": "mdc_dispatch_ffn (k_dfn_plan, k_dfn_route, k_ffn_fused: quantised "
                                              "dispatch, GMM1 + SwiGLU, quantisation of g, GMM2)",
                    "achieved": ffn_info["tops"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8)",
                    "frac": ffn_info["mfma_frac"],
                    "traffic": measured_traffic(w.name + "_pipeline", ("k_dfn_plan", "k_dfn_route", "k_ffn_fused")),
                    "ops_per_launch": ffn_info["int8_ops"],
                    "avg_launch_us": ffn_info["us"], "launch_us": ffn_info["spread_us"],
                    "launch_time_from": "median of two fence-free HIP events on the launch stream around the "
                                        f"mdc_dispatch_ffn call (its dispatch included), on timed steps "
                                        f"{evs_idx[:3]}..{evs_idx[-1:]}"}
    elif ffn_info is not None:
        roofline = {"bound": "mfma", "kernel": "mdc_ffn_quant_input (k_ffn_plan, k_ffn_fused: GMM1 + SwiGLU, quantisation "
                                              "of g, GMM2)" if args.ffn_path == "fused" else
                    "mdc_ffn_quant_input (k_ffn_plan, k_ffn_gemm GMM1 + SwiGLU, k_ffn_quant_rows, k_ffn_gemm GMM2)",
                    "achieved": ffn_info["tops"], "peak": INT8_PEAK_TOPS, "unit": "TOP/s (int8)",
                    "frac": ffn_info["mfma_frac"],
                    "traffic": None if args.ffn_path == "fused" else
                    measured_traffic(w.name, ("k_ffn_plan", "k_ffn_gemm<true", "k_ffn_quant_rows",
                                                         "k_ffn_gemm<false")),
                    "ops_per_launch": ffn_info["int8_ops"],
                    "avg_launch_us": ffn_info["us"], "launch_us": ffn_info["spread_us"],
                    "launch_time_from": "median of two fence-free HIP events on the launch stream around the "
                                        f"mdc_ffn_quant_input call, on timed steps {evs_idx[:3]}..{evs_idx[-1:]}"}
    result = {
        "metric": METRIC,
        "value": round(BS / (ms_per_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{w.name}: {DESCR[w.name]}", "world": W, "bs": BS, "hidden": H,
                   "experts": w.experts, "topk": K, "capacity": w.capacity, "batches": args.batches,
                   "rows_received": by["R"], "source_rows_read": by["U"],
                   "zero_experts": w.zero_experts, "copy_experts": w.copy_experts,
                   "mask": None if wi.mask is None else ("per route" if wi.mask.ndim == 3 else "per token"),
                   "dispatch_call": "mdc_dispatch (one launch)" if one_shot else
                   ("mdc_dispatch_layout + mdc_dispatch_ffn (dispatch inside the FFN pipeline)" if pipelined
                    else "mdc_dispatch_layout + gather")},
        "hbm_gbps": round(gb_step, 1),
        "hbm_frac_of_peak": round(gb_step / HBM_PEAK_GBPS, 4),
        "hbm_frac_of_copy_ceiling": None if ceil is None else round(gb_step / ceil["copy_1GiB"]["gbps"], 4),
        "step_bytes": step_bytes,
        "roofline": roofline,
        "ceilings": ceil,
        "pattern_probes": pats,
        # (with the one-shot dispatch no kernel runs between the first two events)
        "kernels_us": {"dispatch_layout": None if one_shot else spread(t_layout),
                       "dispatch_gather": spread(t_gather),
                       "combine": spread(t_comb), "step_events": spread(t_step_ev),
                       "gather_gbps": round(gb_gather, 1), "combine_gbps": round(gb_comb, 1),
                       "what": f"median, p10, p90 over a {args.breakdown_steps}-step pass after the timed region "
                               "with fence-free HIP events around every stage (not part of value); the dominant "
                               "kernel's in-region samples are under roofline.launch_us"},
    }
    if ffn_info is not None:
        result["ffn"] = ffn_info
    if graph_info is not None:
        result["graph_replay"] = graph_info

    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        fw = gen.ffn_weights(w, rank=0) if w.inter else None
        cb, segs, ref_out = cpu_baseline(wi, w, args.cpu_seconds, fw)
        result["cpu_baseline"] = cb
        # the GPU's last step on batch 0 has the oracle's inputs
        got = batches[0]["x_out"].view(torch.int16).cpu().numpy().view(np.uint16)
        if fw is None:
            result["parity_vs_oracle"] = bool(np.array_equal(got, ref_out))
        else:
            from oracle import mdc_oracle as O
            a = O.bf16_to_f32(got).astype(np.float64)
            b = O.bf16_to_f32(ref_out).astype(np.float64)
            err = float(np.linalg.norm(a - b) / np.linalg.norm(b))
            result["parity_vs_oracle"] = bool(err <= 2e-2)
            result["rel_l2_vs_oracle"] = err
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
