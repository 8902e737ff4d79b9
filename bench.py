#!/usr/bin/env python3
"""Dispatch + combine throughput on one MI355X, against the HBM roofline.

A step is one pass of the hot path over one batch: route (top-k) -> dispatch
(count, scan, place, scatter) -> combine (weighted gather-reduce).  The
experts' grouped GEMM is not part of the path; its per-expert scalar stand-in
runs once per buffer set before timing, so combine reads expert outputs that
are really in HBM.  Inputs are seeded synthetic data of the workload's shape,
resident in HBM before the timed region.

Cold (headline): each timed graph rotates through S buffer sets, S sized from
that graph's own bytes so that the bytes it touches between two uses of a set
exceed twice the 256 MB Infinity Cache.  Warm: one set, reused
(cache-assisted), reported alongside.  Stream floor: plain streaming read and
write kernels (libmoe_ceiling.so) over the payload size, timed the same way,
give what the memory system sustains at that size; one plain kernel per step
part that reads and writes exactly that part's bytes (the dispatch: the token
rows in, the payload out; the combine: the reverse) gives the floor the two
kernels are compared with; copy and gather kernels on the dispatch's and the
combine's own grids, handed their rows, give what their access patterns cost.

Timing: HIP graphs of back-to-back launches replayed between HIP events on the
launch stream.  A kernel's per-launch time is the difference of a graph of 2n
launches and one of n launches, divided by n (n = the smallest multiple of the
graph's S that is at least K), so the fixed cost of a replay cancels and the
buffer rotation continues unbroken from one replay to the next; the median and
the 10th and 90th percentiles over --reps replay pairs are reported.
ms_per_step is one replay of exactly K whole steps (route, dispatch, combine),
synchronised on both sides.

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
[--workload NAME] [--tokens T] (T tokens per source in place of the workload's own,
its fixed capacity resized with them).
"""
from __future__ import annotations

import argparse
import glob
import hashlib
import json
import math
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0      # MI355X HBM3E peak
ONE_LAUNCH_MAX_PAIRS = 8192  # T*k up to which the library dispatches in one launch
MALL_BYTES = 256 << 20     # Infinity Cache
METRIC = "dispatch+combine µs and HBM GB/s (% peak), DeepSeek-V3 shape, 128 tok/rank"


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_decode")
    ap.add_argument("--tokens", type=int, default=0,
                    help="tokens per source in place of the workload's own (a fixed receive capacity is resized with them); 0 = the workload's")
    ap.add_argument("--sets", type=int, default=0, help="cold buffer sets (0 = auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true")
    ap.add_argument("--split", action="store_true",
                    help="also time the receive-side shuffle into dense grouped-GEMM rows "
                         "(moe_dispatch_recv) and its inverse (moe_combine_send)")
    ap.add_argument("--no-floor", action="store_true",
                    help="skip the streaming read/write floor at the payload size")
    ap.add_argument("--groups", type=int, default=1,
                    help="route with group-limited top-k over this many expert groups")
    ap.add_argument("--topk-groups", type=int, default=1, help="groups kept per token")
    ap.add_argument("--combine", choices=("single", "two-stage"), default="single",
                    help="receiver-only combine, or sender-side partial reduction + receive")
    ap.add_argument("--no-next", action="store_true",
                    help="skip the timings of the adjacent paths (partial-reduction combine, "
                         "receive-side shuffle, group-limited router) in the default run")
    ap.add_argument("--reps", type=int, default=7,
                    help="timed replay pairs per graph (median and percentiles over them)")
    ap.add_argument("--summarize-profile", action="store_true",
                    help="print the summary of rocprofv3 output (--trace-dir, and optionally "
                         "--fetch-dir/--write-dir/--cal-fetch-dir/--cal-write-dir) for these "
                         "options instead of running")
    ap.add_argument("--trace-dir")
    ap.add_argument("--fetch-dir")
    ap.add_argument("--write-dir")
    ap.add_argument("--cal-fetch-dir")
    ap.add_argument("--cal-write-dir")
    ap.add_argument("--bench-json",
                    help="with --summarize-profile: the bench.py line of a run without the "
                         "profiler on the same sources (its algorithmic bytes and event timings "
                         "are compared with the profile)")
    ap.add_argument("--profiles-dir", default=os.path.join(ROOT, "profiles"),
                    help="with --summarize-profile --write-figures: where the profile summary "
                         "and figures files go")
    ap.add_argument("--write-figures", action="store_true",
                    help="with --summarize-profile: also write profiles/figures_<options>.txt")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (PMC scale factor)")
    ap.add_argument("--timeline", action="store_true",
                    help="instead of the benchmark: phase timeline of the one-launch dispatch "
                         "and the bf16 combine from libmoe_trace.so (the same sources with "
                         "phase stamps), on rotating cold buffer sets; one JSON line")
    ap.add_argument("--launches", type=int, default=0,
                    help="with --timeline: launches read back per kernel (0 = twice the sets)")
    return ap.parse_args(argv)


# ---------------------------------------------------------------------------
# algorithmic bytes per launch (what the method must move)
# ---------------------------------------------------------------------------
def algorithmic_bytes(w):
    T, H, E, k = w.tokens, w.H, w.E, w.k
    if w.payload == "fp8":
        row = H + 4 * (H // 128)
        dispatch = T * (2 * H + k * row + 8 * k)
        combine = T * (k * row + 8 * k + 2 * H)
    else:
        dispatch = T * (2 * H + 2 * H * k + 8 * k)
        combine = T * (2 * H * k + 8 * k + 2 * H)
    route = T * (4 * E + 8 * k) + (4 * E if w.zipf > 0 else 0)
    return {"route": route, "dispatch": dispatch, "combine": combine}


def nbytes_row(w):
    """Bytes of one receive-buffer row (payload plus fp8 scales)."""
    return w.H + 4 * (w.H // 128) if w.payload == "fp8" else 2 * w.H


# Sources that define each step's kernels (plus those every kernel shares):
# a PMC figure stays valid while these are unchanged.
KERNEL_SOURCES = {
    "route": ["route_topk.hip"],
    "dispatch": ["dispatch.hip", "sources.hip", "gemm_io.hip"],
    "combine": ["combine.hip", "combine_partial.hip"],
}
SHARED_SOURCES = ["device_common.h", "launch.h", "capi.hip"]


def source_sha(part):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "combine_moe_dispatch_amd", "csrc")
    files = [os.path.join(csrc, f) for f in KERNEL_SOURCES[part] + SHARED_SOURCES]
    files.append(os.path.join(ROOT, "include", "moe_dispatch.h"))
    for f in files:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def workload_of(args):
    """The workload the options name (at --tokens tokens per source if given)."""
    from combine_moe_dispatch_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    return inputs.with_tokens(w, args.tokens) if args.tokens else w


def profile_tag(args):
    """Name of the committed profile that matches these options."""
    tag = args.workload
    if args.tokens:
        tag += f"_T{args.tokens}"
    if args.combine == "two-stage":
        tag += "_two_stage"
    if args.groups > 1:
        tag += "_grouped"
    if args.split:
        tag += "_split"
    return tag


def read_figure(tag, part, key):
    """A figure of one step part from the committed profile summary of these
    options (PMC traffic per launch, rocprofv3 kernel durations), if it was
    taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"figures_{tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get(f"{part}_source_sha") != source_sha(part):
        return None
    val = kv.get(f"{part}_{key}")
    return None if val in (None, "", "None") else float(val)


# ---------------------------------------------------------------------------
def copy_calibration():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n, "copy_calibration_bytes_written": n,
                      "launches": 5}), flush=True)


class BufferSet:
    def __init__(self, api, w, shape, inp, torch, np, two_stage=False, split=False,
                 grouped=False):
        dev = "cuda"
        self.logits = torch.from_numpy(inp.logits).to(dev)
        self.bias = None if inp.bias is None else torch.from_numpy(inp.bias).to(dev)
        self.x = torch.from_numpy(inp.x_bits.view(np.int16).copy()).to(dev)
        self.alpha = torch.from_numpy(inp.alpha).to(dev)
        self.ids = torch.empty(w.tokens, w.k, dtype=torch.int32, device=dev)
        self.w = torch.empty(w.tokens, w.k, dtype=torch.float32, device=dev)
        self.src_counts = torch.empty(w.sources, w.E, dtype=torch.int32, device=dev)
        self.src_offsets = torch.empty(w.E, w.sources, dtype=torch.int32, device=dev)
        self.lay = api.Layout.empty(shape, dev)
        self.ws = api.alloc_workspace(shape, dev)
        self.recv, self.rs = api.alloc_recv(shape, dev)
        self.y, self.ys = api.alloc_recv(shape, dev)
        self.out = torch.empty(w.tokens, w.H, dtype=torch.int16, device=dev)
        M = api.partial_slots(shape) if two_stage else 0
        self.partial = torch.empty(w.tokens, M, w.H, dtype=torch.int16, device=dev)
        self.prank = torch.empty(w.tokens, M, dtype=torch.int32, device=dev)
        if grouped:  # the group-limited router's own outputs
            self.gids = torch.empty(w.tokens, w.k, dtype=torch.int32, device=dev)
            self.gw = torch.empty(w.tokens, w.k, dtype=torch.float32, device=dev)
        if split:  # dense grouped-GEMM rows, and regions the send half writes back into
            dense = api.Shape(shape.num_tokens, shape.hidden, shape.num_experts, shape.top_k,
                              shape.num_ranks, 0, shape.payload)
            self.gx, self.gs = api.alloc_recv(dense, dev)
            self.goff = torch.empty(w.E + 1, dtype=torch.int32, device=dev)
            self.ey, self.eys = api.alloc_recv(shape, dev)


def sets_for(nbytes, cap):
    """Buffer sets a timed graph rotates through so that the bytes it touches
    between two uses of one set exceed twice the Infinity Cache (at least 2,
    at most `cap`)."""
    return max(2, min(cap, math.ceil(2 * MALL_BYTES / max(nbytes, 1))))


class GraphTimer:
    """Per-launch time of one launch kind, measured as the difference of two
    HIP graphs of n and 2n back-to-back launches (n a whole multiple of the
    graph's S buffer sets, launch i using set i mod S), each replayed between
    HIP events on the launch stream: (t(2n) - t(n)) / n.  The fixed cost of a
    replay cancels, so the figure does not depend on --steps, and because each
    replay ends on set S-1 and the next starts on set 0, the rotation runs on
    unbroken across replays.  `reps` pairs of replays give the median and the
    10th and 90th percentiles of the estimate."""

    def __init__(self, torch, stream, reps):
        self.torch, self.stream, self.reps = torch, stream, reps

    def capture(self, launch, n):
        torch = self.torch
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=self.stream):
            for i in range(n):
                launch(i)
        return g

    def replay_us(self, g):
        torch = self.torch
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        # replay() launches on torch's current stream: make that the launch
        # stream and record the events on it
        with torch.cuda.stream(self.stream):
            e0.record(self.stream)
            g.replay()
            e1.record(self.stream)
        e1.synchronize()
        return e0.elapsed_time(e1) * 1e3

    def per_launch(self, launch, S, K):
        n1 = S * -(-K // S)
        g1, g2 = self.capture(launch, n1), self.capture(launch, 2 * n1)
        self.replay_us(g1)   # warm-up replays (code, page tables)
        self.replay_us(g2)
        d = []
        for _ in range(self.reps):
            t1 = self.replay_us(g1)
            t2 = self.replay_us(g2)
            d.append((t2 - t1) / n1)
        del g1, g2
        return summarize(d, n1, S)

    def one_replay_us(self, launch, n):
        """Time of one replay of a graph of exactly n launches (after one
        untimed replay), synchronized on both sides."""
        g = self.capture(launch, n)
        self.replay_us(g)
        self.torch.cuda.synchronize()
        t = self.replay_us(g)
        self.torch.cuda.synchronize()
        del g
        return t


def summarize(d, n, S):
    import numpy as np
    a = np.asarray(d, dtype=np.float64)
    return {"us": float(np.median(a)), "p10": float(np.percentile(a, 10)),
            "p90": float(np.percentile(a, 90)), "launches": [n, 2 * n], "sets": S}


def run_gpu(args, w, inp):
    import numpy as np
    import torch

    from combine_moe_dispatch_amd import api

    torch.cuda.set_device(0)
    one = api.Shape(w.T, w.H, w.E, w.k, w.N, w.C,
                    api.MOE_PAYLOAD_FP8_E4M3_B128 if w.payload == "fp8"
                    else api.MOE_PAYLOAD_BF16)
    shape = api.world_shape(one, w.sources)  # all sources' tokens together
    nbytes = algorithmic_bytes(w)
    cap = args.sets or 64
    # each timed graph rotates through as many sets as its own bytes need
    s_disp = sets_for(nbytes["dispatch"], cap)
    s_comb = sets_for(nbytes["combine"], cap)
    s_route = sets_for(nbytes["route"], cap)
    s_step = sets_for(nbytes["dispatch"] + nbytes["combine"] + nbytes["route"], cap)
    S = max(s_disp, s_comb)
    s_route = min(s_route, S)
    # adjacent paths timed beside the main one (cold only), on the same sets
    nxt = not args.no_next
    grouping = next_grouping(w) if nxt and args.groups <= 1 else None
    two_stage_t = args.combine == "two-stage" or nxt
    split_t = args.split or nxt
    sets = [BufferSet(api, w, shape, inp, torch, np, two_stage_t, split_t, grouping is not None)
            for _ in range(S)]
    stream = torch.cuda.Stream()

    def route(s):
        if args.groups > 1:
            api.moe_route_topk_grouped(s.logits, s.bias, w.k, w.score, args.groups,
                                       args.topk_groups, s.ids, s.w, stream=stream)
        else:
            api.moe_route_topk(s.logits, s.bias, w.k, w.score, s.ids, s.w, stream=stream)

    def dispatch(s):
        if w.sources > 1:
            api.moe_dispatch_sources(one, w.sources, s.x, s.ids, s.recv, s.rs, s.lay,
                                     s.src_counts, s.src_offsets, s.ws, stream=stream)
        else:
            api.moe_dispatch(shape, s.x, s.ids, s.recv, s.rs, s.lay, s.ws, stream=stream)

    two_stage = args.combine == "two-stage"

    def combine_send(s):
        api.moe_combine_partial_send(shape, s.y, s.ys, s.lay, s.ids, s.w, s.partial, s.prank,
                                     stream=stream)

    def combine_recv(s):
        api.moe_combine_partial_recv(shape, s.partial, s.prank, s.out, stream=stream)

    def combine(s):
        if two_stage:
            combine_send(s)
            combine_recv(s)
        else:
            api.moe_combine(shape, s.y, s.ys, s.lay, s.w, s.out, stream=stream)

    def step(s):
        route(s)
        dispatch(s)
        combine(s)

    def route_grouped(s):
        api.moe_route_topk_grouped(s.logits, s.bias, w.k, w.score, grouping[0], grouping[1],
                                   s.gids, s.gw, stream=stream)

    def dispatch_recv(s):  # receive regions -> dense grouped-GEMM input
        api.moe_dispatch_recv(shape, s.recv, s.rs, s.lay, s.gx, s.gs, s.goff, stream=stream)

    def combine_send_back(s):  # dense rows -> receive-region layout
        api.moe_combine_send(shape, s.gx, s.gs, s.lay, s.ey, s.eys, stream=stream)

    with torch.cuda.stream(stream):
        for s in sets:   # layout + expert outputs for every set (untimed)
            route(s)
            dispatch(s)
            api.moe_expert_scale(shape, s.recv, s.rs, s.lay, s.alpha, s.y, s.ys, stream=stream)
            combine(s)
            if two_stage_t and not two_stage:
                combine_send(s)
            if split_t:
                dispatch_recv(s)
    stream.synchronize()
    status = int(sets[0].lay.status.item())
    partial_rows = int((sets[0].prank >= 0).sum().item()) if two_stage_t else 0
    placed_rows = int((sets[0].lay.token_row >= 0).sum().item())

    timer = GraphTimer(torch, stream, args.reps)
    K, W = args.steps, args.warmup

    def on(fn, n_sets):
        return lambda i: fn(sets[i % n_sets])

    res = {"sets": {"dispatch": s_disp, "combine": s_comb, "route": s_route, "step": s_step},
           "status": status, "partial_rows": partial_rows, "placed_rows": placed_rows}
    for mode in ("cold", "warm"):
        if mode == "warm" and args.no_warm:
            continue
        cold = mode == "cold"
        sd, sc, sr, ss = (s_disp, s_comb, s_route, s_step) if cold else (1, 1, 1, 1)
        # W untimed eager steps, then the K-step graph of the contract
        with torch.cuda.stream(stream):
            for i in range(W):
                step(sets[i % ss])
        stream.synchronize()
        r = {"step_replay_us": timer.one_replay_us(on(step, ss), K),
             "step": timer.per_launch(on(step, ss), ss, K),
             "route": timer.per_launch(on(route, sr), sr, K),
             "dispatch": timer.per_launch(on(dispatch, sd), sd, K),
             "combine": timer.per_launch(on(combine, sc), sc, K)}
        if cold and (two_stage or two_stage_t):
            r["combine_send"] = timer.per_launch(on(combine_send, sc), sc, K)
            r["combine_recv"] = timer.per_launch(on(combine_recv, sc), sc, K)
        if cold and split_t:
            r["dispatch_recv"] = timer.per_launch(on(dispatch_recv, sd), sd, K)
            r["combine_send_back"] = timer.per_launch(on(combine_send_back, sc), sc, K)
        if cold and grouping is not None:
            r["route_grouped"] = timer.per_launch(on(route_grouped, sr), sr, K)
        res[mode] = r
    if not args.no_floor and w.payload == "bf16":
        res["dispatch_shape"] = dispatch_shape_floor(torch, stream, timer, w, sets[:s_disp], K)
        if w.tokens <= 65535:
            res["combine_shape"] = combine_shape_floor(torch, stream, timer, w, sets[:s_comb], K)
    del sets
    torch.cuda.empty_cache()
    if not args.no_floor:
        res["floor"] = stream_floor(torch, stream, timer, payload_bytes(w), K,
                                    side_bytes=w.tokens * w.H * 2)
    return res


# names of the phase stamps in a trace record (words 0-5)
TRACE_PHASES = {
    "route": ["entry", "logits_loaded", "sorted", "selected", "stored", "done"],
    "dispatch": ["entry", "lds_cleared", "histogram", "rows_known", "stores_issued",
                 "stores_done"],
    "combine": ["entry", "gathers_issued", "folded", "folded_", "store_issued", "store_done"],
}


def timeline_summary(recs, phases, first_slots=0):
    """Per-phase 10th/50th/90th percentile and maximum, in us from the launch's
    earliest entry, pooled over launches.  recs: [launches][slots][8] int64
    trace records (word 7 = 1 when written); the first `first_slots` slots of
    each launch (the dispatch's metadata block) are reported apart, by their
    entry and completion only."""
    import numpy as np
    out, meta = {}, []
    per_phase = {p: [] for p in phases if not p.endswith("_")}
    spans = []
    for r in recs:
        ok = r[:, 7] == 1
        if not ok.any():
            continue
        base = r[ok, 0].min()
        t = (r[:, :6] - base) * 0.01   # 100 MHz clock: ticks of 10 ns
        body = ok.copy()
        body[:first_slots] = False
        for i, p in enumerate(phases):
            if p in per_phase:
                per_phase[p].append(t[body, i])
        if first_slots:
            meta.append(t[:first_slots][ok[:first_slots]][:, [0, 5]])
        spans.append(t[ok, 5].max())
    for p, v in per_phase.items():
        a = np.concatenate(v)
        out[p] = {"p10": round(float(np.percentile(a, 10)), 3),
                  "p50": round(float(np.percentile(a, 50)), 3),
                  "p90": round(float(np.percentile(a, 90)), 3),
                  "max": round(float(a.max()), 3)}
    res = {"phases_us": out, "last_done_us_p50": round(float(np.median(spans)), 3),
           "records_per_launch": int(np.median([int((r[:, 7] == 1).sum()) for r in recs]))}
    if meta:
        m = np.concatenate(meta)
        res["metadata_block_us"] = {"entry_p50": round(float(np.median(m[:, 0])), 3),
                                    "done_p50": round(float(np.median(m[:, 1])), 3),
                                    "done_max": round(float(m[:, 1].max()), 3)}
    return res


def run_timeline(args, w, inp):
    """Phase timeline of the router, the one-launch dispatch (fused kernel,
    bf16 or fp8) and the bf16 combine, read from libmoe_trace.so -- the library's own sources compiled
    with -DMOE_PHASE_STAMPS, whose kernels record the 100 MHz wall clock at
    each phase of their path (the product library holds none of this).  The
    launches run back to back in HIP graphs that rotate over as many buffer
    sets as the timed graphs use, and the last launch of each replay is read
    back (cold, like every timed launch).  The stamps' own waits and stores
    add about 0.2 us, so the times locate the phases rather than time the
    kernels."""
    import ctypes

    import numpy as np
    import torch

    from combine_moe_dispatch_amd import api
    if w.sources != 1 or w.tokens * w.k > ONE_LAUNCH_MAX_PAIRS:
        return {"timeline": None,
                "reason": f"the trace covers the one-launch dispatch (T*k <= "
                          f"{ONE_LAUNCH_MAX_PAIRS}, one source) and the bf16 combine"}
    fp8 = w.payload == "fp8"
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_moe_dispatch_amd", "libmoe_trace.so"))
    for name in ("moe_route_topk", "moe_dispatch", "moe_expert_scale", "moe_combine",
                 "moe_recv_rows", "moe_dispatch_workspace_size", "moe_status_string"):
        f, g = getattr(lib, name), getattr(api._lib, name)
        f.argtypes, f.restype = g.argtypes, g.restype
    vp, u32 = ctypes.c_void_p, ctypes.c_uint32
    lib.moe_trace_set_route.argtypes = [vp, u32]
    lib.moe_trace_set_dispatch.argtypes = [vp, u32]
    lib.moe_trace_set_combine.argtypes = [vp, u32]
    api._lib = lib   # this process's binding calls now go to the tracing library
    torch.cuda.set_device(0)
    shape = api.Shape(w.T, w.H, w.E, w.k, w.N, w.C,
                      api.MOE_PAYLOAD_FP8_E4M3_B128 if fp8 else api.MOE_PAYLOAD_BF16)
    S = max(sets_for(algorithmic_bytes(w)["dispatch"], args.sets or 64),
            sets_for(algorithmic_bytes(w)["combine"], args.sets or 64))
    sets = [BufferSet(api, w, shape, inp, torch, np) for _ in range(S)]
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for s in sets:
            api.moe_route_topk(s.logits, s.bias, w.k, w.score, s.ids, s.w, stream=stream)
            api.moe_dispatch(shape, s.x, s.ids, s.recv, s.rs, s.lay, s.ws, stream=stream)
            api.moe_expert_scale(shape, s.recv, s.rs, s.lay, s.alpha, s.y, s.ys, stream=stream)
    stream.synchronize()
    nvec = w.H // 8
    d_slots = (1 + w.tokens * -(-nvec // 256)) * 4     # the fused grid's waves, at most
    # (fp8: 16 columns a unit, so fewer blocks than this bound)
    c_slots = w.tokens * -(-nvec // 64)                 # one-wave combine blocks
    r_slots = w.tokens                                  # one wave per token
    r_buf = torch.zeros(r_slots * 8, dtype=torch.int64, device="cuda")
    d_buf = torch.zeros(d_slots * 8, dtype=torch.int64, device="cuda")
    c_buf = torch.zeros(c_slots * 8, dtype=torch.int64, device="cuda")
    assert lib.moe_trace_set_route(r_buf.data_ptr(), r_slots) == 0
    assert lib.moe_trace_set_dispatch(d_buf.data_ptr(), d_slots) == 0
    assert lib.moe_trace_set_combine(c_buf.data_ptr(), c_slots) == 0
    # a graph of S back-to-back launches, one per set: each launch's records
    # overwrite the previous one's, so after a replay the buffer holds the
    # last launch's (on set S-1, cold: S launches have passed since it was
    # last used); each replay gives one launch
    timer = GraphTimer(torch, stream, 1)
    graphs = {
        "route": (timer.capture(lambda i: api.moe_route_topk(
            sets[i].logits, sets[i].bias, w.k, w.score, sets[i].ids, sets[i].w,
            stream=stream), S), r_buf),
        "dispatch": (timer.capture(lambda i: api.moe_dispatch(
            shape, sets[i].x, sets[i].ids, sets[i].recv, sets[i].rs, sets[i].lay, sets[i].ws,
            stream=stream), S), d_buf),
        "combine": (timer.capture(lambda i: api.moe_combine(
            shape, sets[i].y, sets[i].ys, sets[i].lay, sets[i].w, sets[i].out, stream=stream),
            S), c_buf)}
    if fp8:   # the fp8 combine carries no stamps
        del graphs["combine"]
    n = args.launches or 2 * S
    recs = {"route": [], "dispatch": [], "combine": []}
    for part, (g, buf) in graphs.items():
        timer.replay_us(g)   # warm-up
        for _ in range(n):
            buf.zero_()
            timer.replay_us(g)
            recs[part].append(buf.view(-1, 8).cpu().numpy())
    assert lib.moe_trace_set_route(None, 0) == 0
    assert lib.moe_trace_set_dispatch(None, 0) == 0
    assert lib.moe_trace_set_combine(None, 0) == 0
    return {"workload": w.name, "launches": n, "sets": S,
            "timeline": {
                "route": timeline_summary(recs["route"], TRACE_PHASES["route"]),
                "dispatch": timeline_summary(recs["dispatch"], TRACE_PHASES["dispatch"],
                                             first_slots=4),
                "combine": None if fp8 else timeline_summary(recs["combine"],
                                                             TRACE_PHASES["combine"])},
            "method": "libmoe_trace.so phase stamps (100 MHz wall clock), us from the "
                      "launch's earliest wave entry; the last launch of each replay of a graph "
                      "of back-to-back launches over the rotating cold sets; dispatch: "
                      "scatter-block waves (metadata block apart); combine: one-wave blocks; "
                      "route: one wave per token"}


def write_timeline_md(args, res):
    """profiles/<tag>_timeline.md (in --profiles-dir): the command, the
    method, one table of phase percentiles per kernel and the --timeline line."""
    tag = profile_tag(args)
    tl = res["timeline"]
    parts = [p for p in ("route", "dispatch", "combine") if tl.get(p)]
    names = {"route": "the router", "dispatch": "the one-launch dispatch",
             "combine": "the bf16 combine"}
    title = ", ".join(names[p] for p in parts[:-1]) + " and " + names[parts[-1]] \
        if len(parts) > 1 else names[parts[0]]
    md = [f"# {tag}: phase timeline of {title} (MI355X)", "",
          "Command, from the repository root (libmoe_trace.so is built with the library by "
          "`python -c \"import __graft_entry__ as g; g.build()\"`):", "",
          f"    python3 bench.py {bench_options(args)} --timeline --write-figures", "",
          "Microseconds from the launch's earliest wave entry, read from the phase stamps of "
          "the tracing library (the library's sources compiled with -DMOE_PHASE_STAMPS; the "
          "100 MHz wall clock, so 0.01 us steps). The last launch of each of "
          f"{res['launches']} replays of a graph of {res['sets']} back-to-back launches over "
          "the rotating cold buffer sets; percentiles over all waves of those launches. The "
          "stamps' own waits and stores add about 0.2 us: the figures place the phases; the "
          "kernel times are the `bench.py` line's of the same options.", ""]
    for part in parts:
        t = tl[part]
        md += [f"## {part}", "", "| phase | p10 | p50 | p90 | max |", "|---|---|---|---|---|"]
        for ph, v in t["phases_us"].items():
            md.append(f"| {ph} | {v['p10']} | {v['p50']} | {v['p90']} | {v['max']} |")
        extra = (f"Last wave done (median over launches): {t['last_done_us_p50']} us; "
                 f"records per launch: {t['records_per_launch']}.")
        if "metadata_block_us" in t:
            m = t["metadata_block_us"]
            extra += (f" Metadata block (block 0): entry {m['entry_p50']} us, done "
                      f"{m['done_p50']} us (median), {m['done_max']} us (max).")
        md += ["", extra, ""]
    md += ["## bench.py --timeline line", "", "    " + json.dumps(res), ""]
    os.makedirs(args.profiles_dir, exist_ok=True)
    with open(os.path.join(args.profiles_dir, f"{tag}_timeline.md"), "w") as f:
        f.write("\n".join(md))


def dispatch_columns(w):
    """(column chunks per token, 16-byte vectors per chunk) of the bf16
    dispatch's scatter grid, by its launcher's rule: on the one-launch path
    (T*k <= ONE_LAUNCH_MAX_PAIRS) up to two vectors per thread of a 256-thread
    block but no fewer chunks than give each of the 256 compute units a block,
    otherwise one vector per thread; chunks are whole multiples of 128
    columns."""
    nunits = w.H // 8
    ceil = lambda a, b: -(-a // b)
    if w.tokens * w.k <= ONE_LAUNCH_MAX_PAIRS:
        cc = max(ceil(nunits, 512), min(ceil(256, max(w.tokens, 1)), ceil(nunits, 256)))
    else:
        cc = ceil(nunits, 256)
    vpc = ceil(ceil(nunits, cc), 16) * 16
    return ceil(nunits, vpc), vpc


def dispatch_shape_floor(torch, stream, timer, w, sets, K):
    """The bf16 dispatch's data movement without the row derivation, one part
    at a time, on the dispatch's own grid (libmoe_ceiling's rows-copy kernel)
    and the same rotating sets: a constant stored to rows t*k+j (one contiguous
    region), the same after reading each token's x slice, a constant stored to
    the rows of the layout the dispatch wrote (its rank regions), and x copied
    to those rows -- what a dispatch that is handed its rows would take."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_moe_dispatch_amd", "libmoe_ceiling.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.moe_ceiling_rows_copy.argtypes = [vp, vp, vp, i32, i32, i32, i32, i32, i32, vp]
    cc, vpc = dispatch_columns(w)
    nvec = w.H // 8
    rows_total = w.N * w.C if w.C > 0 else w.tokens * w.k
    S = len(sets)
    st = stream.cuda_stream

    def timed(with_x, with_rows):
        def launch(i):
            s = sets[i % S]
            rc = lib.moe_ceiling_rows_copy(s.x.data_ptr() if with_x else None,
                                           s.lay.token_row.data_ptr() if with_rows else None,
                                           s.recv.data_ptr(), w.tokens, w.k, nvec, cc, vpc,
                                           rows_total, st)
            assert rc == 0, rc
        return timer.per_launch(launch, S, K)["us"]

    # the first timing of a kernel of this library in a process reads high
    # (measured 3.9 against 3.3 us at DeepSeek-V3 decode): one discarded pass
    timed(False, False)
    return {"column_chunks": cc, "fill_dense_us": timed(False, False),
            "copy_dense_us": timed(True, False), "fill_rows_us": timed(False, True),
            "copy_rows_us": timed(True, True)}


def combine_shape_floor(torch, stream, timer, w, sets, K):
    """The bf16 combine's data movement without the weighted sum, on the
    combine's own grid (one-wave blocks over (token, 64-vector chunk)) and the
    same rotating sets (libmoe_ceiling's rows-gather kernel): the k 16-byte
    gathers of each lane from rows t*k+j (one contiguous region; only where
    those rows exist) and from the rows of the layout the dispatch wrote (its
    rank regions, read through the token's row list like the combine), xored
    and stored as the token's output row -- what a combine that did not fold
    would take."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_moe_dispatch_amd", "libmoe_ceiling.so"))
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.moe_ceiling_rows_gather.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp]
    nvec = w.H // 8
    rows_total = w.N * w.C if w.C > 0 else w.tokens * w.k
    S = len(sets)
    st = stream.cuda_stream

    def timed(with_rows):
        def launch(i):
            s = sets[i % S]
            rc = lib.moe_ceiling_rows_gather(s.y.data_ptr(),
                                             s.lay.token_row.data_ptr() if with_rows else None,
                                             s.out.data_ptr(), w.tokens, w.k, nvec, rows_total,
                                             st)
            assert rc == 0, rc
        return timer.per_launch(launch, S, K)["us"]

    timed(True)   # one discarded pass, as for the dispatch's probe
    res = {"gather_rows_us": timed(True)}
    if w.tokens * w.k <= rows_total:
        res["gather_dense_us"] = timed(False)
    return res


def two_stage_bytes(w, partial_rows):
    """Algorithmic bytes of the partial-reduction combine.  Send: the k rows
    and (row, id, weight) per pair in, one bf16 row per used (token, rank) slot
    and the slot ranks out; recv: those rows and ranks in, the token out."""
    M = min(w.k, w.N)
    send = w.tokens * (nbytes_row(w) * w.k + 12 * w.k + 4 * M) + partial_rows * 2 * w.H
    recv = partial_rows * 2 * w.H + w.tokens * (4 * M + 2 * w.H)
    return send, recv


def next_grouping(w):
    """(groups, groups kept) for the group-limited router timing: DeepSeek-V3's
    8 groups with 4 kept where the experts divide into 8 groups that hold k;
    None where they do not."""
    G, kept = 8, 4
    if w.E % G or kept * (w.E // G) < w.k:
        return None
    return G, kept


def payload_bytes(w):
    """Payload bytes one dispatch writes (and one combine reads): k rows per token."""
    return w.tokens * w.k * nbytes_row(w)


def stream_floor(torch, stream, timer, nbytes, K, side_bytes=0):
    """What the memory system sustains at this size: plain streaming read and
    write of `nbytes` with 16-byte accesses, and an empty launch, timed like
    the kernels (graph differences over rotating buffers, cold).  Read: a
    non-temporal grid-stride loop, the best of three grid sizes.  Write: the
    best of that loop and of 64 KB blocks stored with each cache policy.
    Copy: read and write of `nbytes` each, the non-temporal loop.  With
    side_bytes (the token rows: x read by the dispatch, the output written by
    the combine), also the two kernels' own streams in one plain kernel each:
    read side_bytes while writing nbytes (the dispatch's bytes), read nbytes
    while writing side_bytes (the combine's), the best of three grid sizes."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_moe_dispatch_amd", "libmoe_ceiling.so"))
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.moe_ceiling_read.argtypes = [vp, sz, vp, i32, vp]
    lib.moe_ceiling_write.argtypes = [vp, sz, i32, vp]
    lib.moe_ceiling_write_blocked.argtypes = [vp, sz, i32, vp]
    lib.moe_ceiling_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.moe_ceiling_empty.argtypes = [vp]
    lib.moe_ceiling_read_write.argtypes = [vp, sz, vp, sz, vp, i32, vp]
    nbytes = (nbytes + 15) // 16 * 16
    S = sets_for(nbytes, 64)
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(S)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    nvec = nbytes // 16
    st = stream.cuda_stream

    def timed(fn):
        def launch(i):
            assert fn(i) == 0
        return timer.per_launch(launch, S, K)["us"]

    grids = (1024, 2048, 4096)
    rd = min(timed(lambda i, b=b: lib.moe_ceiling_read(bufs[i % S].data_ptr(), nvec,
                                                       sink.data_ptr(), b, st)) for b in grids)
    wr = min(timed(lambda i, b=b: lib.moe_ceiling_write(bufs[i % S].data_ptr(), nvec, b, st))
             for b in grids)
    # 64 KB per block with each cache policy (at some sizes faster than the loop)
    wr = min([wr] + [timed(lambda i, c=c: lib.moe_ceiling_write_blocked(bufs[i % S].data_ptr(),
                                                                       nvec, c, st))
                     for c in (0, 1, 2)])
    # copy: read one buffer, write the next (both rotate)
    cp = min(timed(lambda i, b=b: lib.moe_ceiling_copy(bufs[i % S].data_ptr(),
                                                       bufs[(i + 1) % S].data_ptr(), nvec, b, st))
             for b in grids)
    em = timed(lambda i: lib.moe_ceiling_empty(st))
    io = {}
    if side_bytes:
        side_bytes = (side_bytes + 15) // 16 * 16
        sides = [torch.empty(side_bytes, dtype=torch.uint8, device="cuda") for _ in range(S)]
        for b in sides:
            b.fill_(1)
        nside = side_bytes // 16
        io["dispatch_io_us"] = min(timed(lambda i, b=b: lib.moe_ceiling_read_write(
            sides[i % S].data_ptr(), nside, bufs[i % S].data_ptr(), nvec, sink.data_ptr(), b,
            st)) for b in grids)
        io["combine_io_us"] = min(timed(lambda i, b=b: lib.moe_ceiling_read_write(
            bufs[i % S].data_ptr(), nvec, sides[i % S].data_ptr(), nside, sink.data_ptr(), b,
            st)) for b in grids)
        del sides
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "sets": S, "read_us": rd, "write_us": wr, "copy_us": cp,
            "empty_launch_us": em, **io}


def cpu_baseline(w, inp, seconds):
    """The C oracle as it stands, single-threaded, on full steps of the same
    workload until about `seconds` of work; dispatch and combine timed apart."""
    import ctypes

    import numpy as np

    import oracle
    lib = oracle._load()
    ids, wt = oracle.route_topk(inp.logits, inp.bias, w.k, w.score)
    lay = oracle.layout(ids, w.E, w.N, w.C)
    rows = lay["rows"]
    tr = np.ascontiguousarray(lay["token_row"])
    x = np.ascontiguousarray(inp.x_bits)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    fp8 = w.payload == "fp8"
    if fp8:
        recv = np.zeros((rows, w.H), np.uint8)
        rs = np.zeros((rows, w.H // 128), np.float32)
    else:
        recv = np.zeros((rows, w.H), np.uint16)
        rs = None
    T = w.tokens
    out = np.empty((T, w.H), np.uint16)
    td = tc = 0.0
    reps = 0
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if fp8:
            lib.oracle_dispatch_fp8(p(x), T, w.H, w.k, p(tr), p(recv), p(rs))
        else:
            lib.oracle_dispatch_bf16(p(x), T, w.H, w.k, p(tr), p(recv))
        t1 = time.perf_counter()
        lib.oracle_combine_exact(p(recv), None if rs is None else p(rs), p(tr), p(wt), T,
                                 w.k, w.H, p(out))
        t2 = time.perf_counter()
        td += t1 - t0
        tc += t2 - t1
        reps += 1
        if time.perf_counter() - t_start >= seconds:
            break
    nbytes = algorithmic_bytes(w)
    gbs = (nbytes["dispatch"] + nbytes["combine"]) * reps / (td + tc) / 1e9
    return {"value": round(gbs, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{reps} full {w.name} steps (oracle dispatch + double-precision combine, "
                      f"C, one thread); {1e6 * td / reps:.0f} us dispatch + "
                      f"{1e6 * tc / reps:.0f} us combine per step",
            "host": cpu_model(),
            "nproc": os.cpu_count()}


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo where there is one)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


# ---------------------------------------------------------------------------
# rocprofv3 summaries (what profiles/ holds)
# ---------------------------------------------------------------------------
# kernels that make up each step part (name fragments as rocprofv3 prints them)
PART_KERNELS = {
    "route": ["route_topk_kernel"],
    "dispatch": ["dispatch_fused_kernel", "layout_chunk_kernel", "layout_scan_kernel",
                 "layout_bases_kernel", "dispatch_scatter_kernel", "source_counts_kernel",
                 "source_offsets_kernel"],
    "combine": ["combine_bf16_kernel", "combine_fp8_kernel", "combine_send_kernel",
                "combine_send_small_kernel", "combine_recv_kernel"],
}


def _csv_rows(directory, suffix):
    import csv
    files = sorted(glob.glob(os.path.join(directory, "**", f"*{suffix}"), recursive=True))
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _part_of(name):
    for part, frags in PART_KERNELS.items():
        for f in frags:
            if f in name:
                return part, f
    return None, None


def bench_options(args):
    """The bench.py options that select this workload and path."""
    opts = f"--workload {args.workload}"
    if args.tokens:
        opts += f" --tokens {args.tokens}"
    if args.groups > 1:
        opts += f" --groups {args.groups} --topk-groups {args.topk_groups}"
    if args.combine == "two-stage":
        opts += " --combine two-stage"
    if args.split:
        opts += " --split"
    return opts


def profile_header(args, w):
    """Title, workload and the commands that make a profile summary."""
    tag, o = profile_tag(args), bench_options(args)
    quiet = "--no-cpu-baseline --no-warm --no-next --no-floor"
    cmds = [
        f"python3 bench.py {o} --steps 200 --warmup 20 > bench_line.json",
        f"rocprofv3 --kernel-trace --stats --output-format csv -d <out>/kt -o run -- "
        f"python3 bench.py {o} --steps 200 --warmup 20 {quiet}",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/fetch -o run -- "
        f"python3 bench.py {o} --steps 5 --warmup 2 --reps 1 {quiet}",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/write -o run -- "
        f"python3 bench.py {o} --steps 5 --warmup 2 --reps 1 {quiet}",
        "rocprofv3 --pmc FETCH_SIZE --output-format csv -d <out>/cal_fetch -o run -- "
        "python3 bench.py --copy-calibration",
        "rocprofv3 --pmc WRITE_SIZE --output-format csv -d <out>/cal_write -o run -- "
        "python3 bench.py --copy-calibration",
        f"python3 bench.py --summarize-profile {o} --trace-dir <out>/kt --fetch-dir <out>/fetch "
        f"--write-dir <out>/write --cal-fetch-dir <out>/cal_fetch --cal-write-dir "
        f"<out>/cal_write --bench-json bench_line.json --write-figures"]
    return [f"# {tag}: kernel durations and HBM traffic (rocprofv3, MI355X)", "",
            f"Workload {w.name}: T={w.T} per source x {w.sources} source(s), H={w.H}, E={w.E}, "
            f"k={w.k}, N={w.N}, C={w.C} (0 = packed), payload={w.payload}.", "",
            "Commands, from the repository root (`cd /tmp && export TMPDIR=/tmp` first for "
            "rocprofv3, with `bench.py` given by its full path):", ""] + \
        [f"    {c}" for c in cmds] + [""]


def summarize_profile(args):
    """Markdown summary of a rocprofv3 kernel trace (and optional FETCH_SIZE /
    WRITE_SIZE counter runs with their copy calibration) for this workload and
    options, printed; with --write-figures also written, whole (the commands
    that make it, the --stats rows of the path's kernels, the summary and the
    bench.py line), as <tag>_kernels_and_traffic.md, beside the key = value
    file bench.py reads (figures_<tag>.txt), in --profiles-dir."""
    import numpy as np
    from combine_moe_dispatch_amd import inputs
    w = workload_of(args)
    nb = algorithmic_bytes(w)
    line = None
    if args.bench_json:
        with open(args.bench_json) as f:
            line = json.loads([x for x in f.read().splitlines() if x.strip()][-1])
        nb.update({k: v for k, v in line["algorithmic_bytes"].items() if k in nb})
    tag = profile_tag(args)
    out = []
    figures = {}
    parts_us = {}
    # kernel trace: per kernel, every dispatch's end - start
    rows = _csv_rows(args.trace_dir, "kernel_trace.csv")
    durs = {}
    for r in rows:
        durs.setdefault(r["Kernel_Name"], []).append(
            int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    out.append("| kernel | calls | mean ns | median ns | p10 ns | p90 ns | min ns | max ns |")
    out.append("|---|---|---|---|---|---|---|---|")
    per_frag = {}
    for name, d in sorted(durs.items(), key=lambda kv: -len(kv[1])):
        a = np.asarray(d, np.float64)
        short = name.replace("void ", "").replace("(anonymous namespace)::", "")
        short = short.replace("moe::", "").split("(")[0]
        out.append(f"| {short[:60]} | {len(a)} | {a.mean():.0f} | {np.median(a):.0f} | "
                   f"{np.percentile(a, 10):.0f} | {np.percentile(a, 90):.0f} | {a.min():.0f} | "
                   f"{a.max():.0f} |")
        part, frag = _part_of(name)
        if part:
            per_frag.setdefault((part, frag), []).extend(d)
    out.append("")
    out.append("| step part | kernels | rocprofv3 median us (sum over the part's kernels) | "
               "mean us | algorithmic bytes | GB/s at the median | fraction of 8 TB/s |")
    out.append("|---|---|---|---|---|---|---|")
    for part in ("route", "dispatch", "combine"):
        ks = [(f, d) for (p, f), d in per_frag.items() if p == part]
        if not ks:
            continue
        med = sum(float(np.median(d)) for _, d in ks) / 1e3
        mean = sum(float(np.mean(d)) for _, d in ks) / 1e3
        parts_us[part] = (med, mean)
        gbs = nb[part] / (med * 1e-6) / 1e9
        figures[f"{part}_rocprof_median_us"] = f"{med:.3f}"
        figures[f"{part}_rocprof_mean_us"] = f"{mean:.3f}"
        out.append(f"| {part} | {', '.join(f for f, _ in ks)} | {med:.3f} | {mean:.3f} | "
                   f"{nb[part]} | {gbs:.0f} | {gbs / HBM_PEAK_GBS:.4f} |")
    if line is not None:
        ev = {"route": line["route_us"], "dispatch": line["dispatch_us"],
              "combine": line["combine_us"]}
        out.append("")
        out.append("Event timing of the same sources without the profiler (per launch, graph "
                   "difference method) against the profiled kernel durations:")
        out.append("")
        out.append("| step part | bench.py us per launch | rocprofv3 median us | median / event | "
                   "rocprofv3 mean us | mean / event |")
        out.append("|---|---|---|---|---|---|")
        for part in ("route", "dispatch", "combine"):
            if part in parts_us:
                med, mean = parts_us[part]
                out.append(f"| {part} | {ev[part]:.3f} | {med:.3f} | {med / ev[part]:.3f} | "
                           f"{mean:.3f} | {mean / ev[part]:.3f} |")
    # counters, scaled by what the same counter reads for a copy of known size
    if args.fetch_dir and args.write_dir and args.cal_fetch_dir and args.cal_write_dir:
        def per_kernel(directory, counter):
            acc = {}
            for r in _csv_rows(directory, "counter_collection.csv"):
                if r["Counter_Name"] != counter:
                    continue
                acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
            return acc

        def copy_kib(directory, counter):
            vals = [v for name, v in per_kernel(directory, counter).items()
                    if "copy" in name.lower() or "elementwise" in name.lower()]
            best = max(vals, key=len)  # the copy launches (the most numerous)
            return float(np.median(best))
        gib_kib = float(1 << 20)  # 1 GiB in KiB
        fscale = gib_kib / copy_kib(args.cal_fetch_dir, "FETCH_SIZE")
        wscale = gib_kib / copy_kib(args.cal_write_dir, "WRITE_SIZE")
        fk = per_kernel(args.fetch_dir, "FETCH_SIZE")
        wk = per_kernel(args.write_dir, "WRITE_SIZE")
        out.append("")
        out.append(f"Copy calibration (a 1 GiB device copy): FETCH_SIZE x {fscale:.4f}, "
                   f"WRITE_SIZE x {wscale:.4f}.")
        out.append("")
        out.append("| kernel | FETCH_SIZE KiB per dispatch | WRITE_SIZE KiB per dispatch | "
                   "scaled bytes |")
        out.append("|---|---|---|---|")
        part_bytes = {}
        for name in sorted(set(fk) | set(wk)):
            part, frag = _part_of(name)
            if not part:
                continue
            f = float(np.median(fk.get(name, [0.0])))
            wv = float(np.median(wk.get(name, [0.0])))
            b = 1024.0 * (f * fscale + wv * wscale)
            part_bytes[part] = part_bytes.get(part, 0.0) + b
            out.append(f"| {frag} | {f:.1f} | {wv:.1f} | {b:.0f} |")
        out.append("")
        out.append("| step part | scaled bytes per launch | algorithmic bytes | ratio |")
        out.append("|---|---|---|---|")
        for part, b in part_bytes.items():
            figures[f"{part}_traffic_bytes_per_launch"] = f"{b:.0f}"
            out.append(f"| {part} | {b:.0f} | {nb[part]} | {b / nb[part]:.3f} |")
        figures["fetch_scale"] = f"{fscale:.6f}"
        figures["write_scale"] = f"{wscale:.6f}"
    print("\n".join(out))
    if args.write_figures:
        stats = ["| kernel | calls | average ns | min ns | max ns |", "|---|---|---|---|---|"]
        srows = [r for r in _csv_rows(args.trace_dir, "kernel_stats.csv") if _part_of(r["Name"])[0]]
        for r in sorted(srows, key=lambda r: -float(r["AverageNs"])):
            short = r["Name"].replace("void ", "").replace("(anonymous namespace)::", "")
            short = short.replace("moe::", "").split("(")[0]
            stats.append(f"| {short} | {r['Calls']} | {float(r['AverageNs']):.0f} | "
                         f"{r['MinNs']} | {r['MaxNs']} |")
        md = profile_header(args, w) + \
            ["## rocprofv3 --stats (kernels of the path; all launches of the traced run)", ""] + \
            stats + ["", "## Kernel trace, event timing and counters "
                     "(bench.py --summarize-profile)", ""] + out
        if line is not None:
            md += ["", "## bench.py line of the same sources (no profiler)", "",
                   "    " + json.dumps(line)]
        os.makedirs(args.profiles_dir, exist_ok=True)
        with open(os.path.join(args.profiles_dir, f"{tag}_kernels_and_traffic.md"), "w") as f:
            f.write("\n".join(md) + "\n")
        path = os.path.join(args.profiles_dir, f"figures_{tag}.txt")
        with open(path, "w") as f:
            f.write(f"# {tag}: figures from rocprofv3 (bench.py --summarize-profile); each part's\n"
                    f"# figures hold for the kernel sources with its hash\n")
            for part in ("route", "dispatch", "combine"):
                f.write(f"{part}_source_sha = {source_sha(part)}\n")
            for k, v in sorted(figures.items()):
                f.write(f"{k} = {v}\n")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share of the expert-parallel world; "
              f"--gpus {args.gpus} is not supported (multi-GPU dispatch is not built).",
              file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        copy_calibration()
        return
    if args.summarize_profile:
        summarize_profile(args)
        return

    from combine_moe_dispatch_amd import inputs
    w = workload_of(args)
    inp = inputs.generate_for(w)
    if args.timeline:
        res = run_timeline(args, w, inp)
        print(json.dumps(res), flush=True)
        if args.write_figures and res.get("timeline"):
            write_timeline_md(args, res)
        return
    print(f"[bench] workload {w.name}: T={w.T} x {w.sources} source(s) H={w.H} E={w.E} k={w.k} N={w.N} C={w.C} "
          f"payload={w.payload}", file=sys.stderr, flush=True)
    g = run_gpu(args, w, inp)
    print(f"[bench] gpu timing done: {json.dumps(g)}", file=sys.stderr, flush=True)
    nbytes = algorithmic_bytes(w)
    if args.combine == "two-stage":
        send, recv = two_stage_bytes(w, g["partial_rows"])
        nbytes["combine"] = send + recv
        nbytes["combine_send"], nbytes["combine_recv"] = send, recv
    cold = g["cold"]
    us = {k: v["us"] for k, v in cold.items() if isinstance(v, dict)}
    dc_us = us["dispatch"] + us["combine"]
    dc_bytes = nbytes["dispatch"] + nbytes["combine"]
    value = dc_bytes / (dc_us * 1e-6) / 1e9
    dom = "dispatch" if us["dispatch"] >= us["combine"] else "combine"
    achieved = nbytes[dom] / (us[dom] * 1e-6) / 1e9
    tag = profile_tag(args)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold["step_replay_us"] / args.steps / 1e3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.payload == "bf16" else "fp8-e4m3",
        "data": "synthetic (seeded N(0,1) logits and tokens of the workload's shape)",
        "config": {"workload": w.name, "tokens": w.T, "sources": w.sources,
                   "hidden": w.H, "experts": w.E,
                   "top_k": w.k, "ranks": w.N, "rank_capacity": w.C, "payload": w.payload,
                   "parallelism": "one source rank, N virtual destination ranks in HBM",
                   "combine": ("receiver-only" if args.combine == "single" else
                               "sender-side partial reduction, then receive"),
                   "router": ("top-k" if args.groups <= 1 else
                              f"group-limited top-k, {args.topk_groups} of {args.groups} groups"),
                   "cold_buffer_sets": g["sets"]},
        "dispatch_us": round(us["dispatch"], 3),
        "combine_us": round(us["combine"], 3),
        "dispatch_plus_combine_us": round(dc_us, 3),
        "route_us": round(us["route"], 3),
        "step_us": round(us["step"], 3),
        "hbm_frac_dispatch_plus_combine": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_figure(tag, dom, "traffic_bytes_per_launch"),
                     "timing": "HIP events on the launch stream: per-launch interval of "
                               "back-to-back launches (timing.method)"},
        "timing": {
            "method": "per launch = (t(2n) - t(n)) / n for HIP graphs of n and 2n back-to-back "
                      "launches, n a multiple of the graph's buffer sets; median and "
                      "10th/90th percentiles over replay pairs",
            "replay_pairs": args.reps,
            **{k: {"us": round(v["us"], 3), "p10": round(v["p10"], 3),
                   "p90": round(v["p90"], 3), "launches": v["launches"], "sets": v["sets"]}
               for k, v in cold.items() if isinstance(v, dict)}},
        "device_status": g["status"],
    }
    prof = {}
    for part in ("route", "dispatch", "combine"):
        med = read_figure(tag, part, "rocprof_median_us")
        mean = read_figure(tag, part, "rocprof_mean_us")
        if med is not None:
            prof[part] = {"median_us": med, "mean_us": mean,
                          "median_over_event": round(med / us[part], 3)}
    if prof:
        # kernel durations of the committed rocprofv3 trace of these sources
        line["rocprof_kernel_trace"] = prof
        if dom in prof:
            # the same roofline at the profiled kernel durations (each kernel
            # run on its own by the profiler), for reading against profiles/
            for stat in ("median", "mean"):
                d_us = prof[dom][f"{stat}_us"]
                if d_us:
                    line["roofline"][f"frac_rocprof_{stat}"] = round(
                        nbytes[dom] / (d_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)
    send_b, recv_b = two_stage_bytes(w, g["partial_rows"])
    # receive-side shuffle: each placed row read once and written once, plus
    # (counts, offsets) per expert read and the dense offsets written
    moved = 2 * g["placed_rows"] * nbytes_row(w) + 8 * w.E + 4 * (w.E + 1)
    extra = {}
    if "combine_send" in us:
        extra["combine_partial"] = {
            "send_us": round(us["combine_send"], 3), "recv_us": round(us["combine_recv"], 3),
            "partial_rows": g["partial_rows"], "rows_per_token": round(g["partial_rows"] / w.tokens, 3),
            "send_GBps": round(send_b / (us["combine_send"] * 1e-6) / 1e9, 1),
            "recv_GBps": round(recv_b / (us["combine_recv"] * 1e-6) / 1e9, 1)}
    if "dispatch_recv" in us:
        extra["split"] = {
            "dispatch_recv_us": round(us["dispatch_recv"], 3),
            "combine_send_us": round(us["combine_send_back"], 3),
            "bytes_each": moved,
            "dispatch_recv_GBps": round(moved / (us["dispatch_recv"] * 1e-6) / 1e9, 1),
            "combine_send_GBps": round(moved / (us["combine_send_back"] * 1e-6) / 1e9, 1)}
    if "route_grouped" in us:
        G, kept = next_grouping(w)
        extra["route_grouped"] = {"groups": G, "groups_kept": kept,
                                  "route_us": round(us["route_grouped"], 3)}
    if args.combine == "two-stage":
        line["two_stage_combine"] = extra.pop("combine_partial")
    if args.split:
        line["split"] = extra.pop("split")
    if extra:
        # adjacent paths on the same inputs, cold, timed like the main kernels
        line["next"] = extra
    if "warm" in g:
        wm = {k: v["us"] for k, v in g["warm"].items() if isinstance(v, dict)}
        wus = wm["dispatch"] + wm["combine"]
        line["warm_cache_assisted"] = {
            "dispatch_us": round(wm["dispatch"], 3), "combine_us": round(wm["combine"], 3),
            "route_us": round(wm["route"], 3), "step_us": round(wm["step"], 3),
            "GBps": round(dc_bytes / (wus * 1e-6) / 1e9, 2)}
    if "floor" in g:
        fl = g["floor"]
        line["stream_floor"] = {
            "payload_bytes": fl["bytes"], "sets": fl["sets"], "read_us": round(fl["read_us"], 3),
            "write_us": round(fl["write_us"], 3), "copy_us": round(fl["copy_us"], 3),
            "empty_launch_us": round(fl["empty_launch_us"], 3),
            "read_GBps": round(fl["bytes"] / (fl["read_us"] * 1e-6) / 1e9, 1),
            "write_GBps": round(fl["bytes"] / (fl["write_us"] * 1e-6) / 1e9, 1),
            "write_plus_read_us": round(fl["write_us"] + fl["read_us"], 3),
            "dispatch_over_write_floor": round(us["dispatch"] / fl["write_us"], 3),
            "combine_over_read_floor": round(us["combine"] / fl["read_us"], 3)}
        if "dispatch_io_us" in fl:
            # each kernel's own streams (token rows and payload) in one plain
            # kernel; their sum against the time the roofline fraction of
            # `value` would need at 60 % of the peak
            io_sum = fl["dispatch_io_us"] + fl["combine_io_us"]
            line["stream_floor"].update({
                "token_bytes": w.tokens * w.H * 2,
                "dispatch_io_us": round(fl["dispatch_io_us"], 3),
                "combine_io_us": round(fl["combine_io_us"], 3),
                "io_floor_sum_us": round(io_sum, 3),
                "io_floor_sum_frac": round(dc_bytes / (io_sum * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                "dispatch_over_io_floor": round(us["dispatch"] / fl["dispatch_io_us"], 3),
                "combine_over_io_floor": round(us["combine"] / fl["combine_io_us"], 3)})
        if "dispatch_shape" in g:
            ds = g["dispatch_shape"]
            line["stream_floor"]["dispatch_shape"] = {
                "column_chunks": ds["column_chunks"],
                **{k: round(v, 3) for k, v in ds.items() if k.endswith("_us")},
                "dispatch_over_copy_rows": round(us["dispatch"] / ds["copy_rows_us"], 3)}
        if "combine_shape" in g:
            cs = g["combine_shape"]
            line["stream_floor"]["combine_shape"] = {
                **{k: round(v, 3) for k, v in cs.items() if k.endswith("_us")},
                "combine_over_gather_rows": round(us["combine"] / cs["gather_rows_us"], 3)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
