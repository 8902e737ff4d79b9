#!/usr/bin/env python3
"""Dispatch + combine throughput on one MI355X, against the HBM roofline.

A step is one pass of the hot path over one batch: route (top-k) -> dispatch
(count, scan, place, scatter) -> combine (weighted gather-reduce).  The
experts' grouped GEMM is not part of the path; its per-expert scalar stand-in
runs once per buffer set before timing, so combine reads expert outputs that
are really in HBM.  Inputs are seeded synthetic data of the workload's shape,
resident in HBM before the timed region.

Cold (headline): S buffer sets rotate so that the bytes touched between two
uses of a set exceed twice the 256 MB Infinity Cache.  Warm: one set, reused
(cache-assisted), reported alongside.  Stream floor: plain streaming read and
write kernels (libmoe_ceiling.so) over the payload size, timed the same way,
give what the memory system sustains at that size.

Timing: HIP graphs of back-to-back launches replayed between HIP events on the
launch stream.  The step figure captures K whole steps (one timed replay);
each kernel's average launch duration comes from a graph of K launches of that
kernel alone (median of three timed replays).

Prints one JSON line.  Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
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
MALL_BYTES = 256 << 20     # Infinity Cache
METRIC = "dispatch+combine µs and HBM GB/s (% peak), DeepSeek-V3 shape, 128 tok/rank"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="dsv3_decode")
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
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (PMC scale factor)")
    return ap.parse_args()


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


def profile_tag(args):
    """Name of the committed profile that matches these options."""
    tag = args.workload
    if args.combine == "two-stage":
        tag += "_two_stage"
    if args.groups > 1:
        tag += "_grouped"
    if args.split:
        tag += "_split"
    return tag


def read_traffic(tag, kernel):
    """HBM bytes per launch from a committed PMC summary, if it was taken on
    the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{tag}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get(f"{kernel}_source_sha") != source_sha(kernel):
        return None
    val = kv.get(f"{kernel}_traffic_bytes_per_launch")
    return None if val is None else float(val)


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
    per_step = nbytes["dispatch"] + nbytes["combine"] + nbytes["route"]
    S = args.sets or min(64, max(2, math.ceil(2 * MALL_BYTES / per_step)))
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
    stream.synchronize()
    status = int(sets[0].lay.status.item())
    partial_rows = int((sets[0].prank >= 0).sum().item()) if two_stage_t else 0
    placed_rows = int((sets[0].lay.token_row >= 0).sum().item())

    def capture(fn_list, n, rotate):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                s = sets[i % len(sets)] if rotate else sets[0]
                for fn in fn_list:
                    fn(s)
        return g

    def time_graph(g, n, reps=1):
        # replay() launches on torch's current stream: make that the launch
        # stream, and bracket the replay with events recorded on it.  With
        # reps > 1 the median of that many timed replays is returned.
        ts = []
        for _ in range(reps):
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(stream):
                e0.record(stream)
                g.replay()
                e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3 / n)  # us per unit
        return sorted(ts)[len(ts) // 2]

    K, W = args.steps, args.warmup
    res = {"sets": S, "status": status, "partial_rows": partial_rows, "placed_rows": placed_rows}
    for mode, rotate in (("cold", True), ("warm", False)):
        if mode == "warm" and args.no_warm:
            continue
        # warm-up: W eager steps, then one replay of each graph
        with torch.cuda.stream(stream):
            for i in range(W):
                step(sets[i % len(sets)] if rotate else sets[0])
        stream.synchronize()
        g_step = capture([route, dispatch, combine], K, rotate)
        g_route = capture([route], K, rotate)
        g_disp = capture([dispatch], K, rotate)
        g_comb = capture([combine], K, rotate)
        with torch.cuda.stream(stream):
            for g in (g_step, g_route, g_disp, g_comb):
                g.replay()
        torch.cuda.synchronize()
        step_us = time_graph(g_step, K)
        r = {
            "step_us": step_us,
            "route_us": time_graph(g_route, K, reps=3),
            "dispatch_us": time_graph(g_disp, K, reps=3),
            "combine_us": time_graph(g_comb, K, reps=3),
        }
        if two_stage or (two_stage_t and mode == "cold"):
            g_send = capture([combine_send], K, rotate)
            g_recv = capture([combine_recv], K, rotate)
            with torch.cuda.stream(stream):
                g_send.replay()
                g_recv.replay()
            r["combine_send_us"] = time_graph(g_send, K, reps=3)
            r["combine_recv_us"] = time_graph(g_recv, K, reps=3)
            del g_send, g_recv
        if args.split or (split_t and mode == "cold"):
            g_dr = capture([dispatch_recv], K, rotate)
            g_cs = capture([combine_send_back], K, rotate)
            with torch.cuda.stream(stream):
                g_dr.replay()
                g_cs.replay()
            r["dispatch_recv_us"] = time_graph(g_dr, K, reps=3)
            r["combine_send_back_us"] = time_graph(g_cs, K, reps=3)
            del g_dr, g_cs
        if grouping is not None and mode == "cold":
            g_rg = capture([route_grouped], K, rotate)
            with torch.cuda.stream(stream):
                g_rg.replay()
            r["route_grouped_us"] = time_graph(g_rg, K, reps=3)
            del g_rg
        res[mode] = r
        del g_step, g_route, g_disp, g_comb
    if not args.no_floor:
        res["floor"] = stream_floor(torch, stream, time_graph, payload_bytes(w), min(K, 100))
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


def stream_floor(torch, stream, time_graph, nbytes, n):
    """What the memory system sustains at this size: plain streaming read and
    write of `nbytes` with 16-byte accesses, and an empty launch, timed like
    the kernels (graphs of n launches over rotating buffers, cold).  Read: a
    non-temporal grid-stride loop, the best of three grid sizes.  Write: the
    best of that loop and of 64 KB blocks stored with each cache policy.
    Copy: read and write of `nbytes` each, the non-temporal loop."""
    import ctypes
    lib = ctypes.CDLL(os.path.join(ROOT, "combine_moe_dispatch_amd", "libmoe_ceiling.so"))
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.moe_ceiling_read.argtypes = [vp, sz, vp, i32, vp]
    lib.moe_ceiling_write.argtypes = [vp, sz, i32, vp]
    lib.moe_ceiling_write_blocked.argtypes = [vp, sz, i32, vp]
    lib.moe_ceiling_copy.argtypes = [vp, vp, sz, i32, vp]
    lib.moe_ceiling_empty.argtypes = [vp]
    nbytes = (nbytes + 15) // 16 * 16
    S = min(64, max(2, math.ceil(2 * MALL_BYTES / nbytes)))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda") for _ in range(S)]
    for b in bufs:
        b.fill_(1)
    sink = torch.zeros(65536, dtype=torch.int32, device="cuda")
    nvec = nbytes // 16
    st = stream.cuda_stream

    def timed(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(n):
                assert fn(i) == 0
        with torch.cuda.stream(stream):
            g.replay()
        torch.cuda.synchronize()
        t = time_graph(g, n, reps=3)
        del g
        return t

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
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "read_us": rd, "write_us": wr, "copy_us": cp, "empty_launch_us": em}


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

    from combine_moe_dispatch_amd import inputs
    w = inputs.WORKLOADS[args.workload]
    inp = inputs.generate_for(w)
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
    dc_us = cold["dispatch_us"] + cold["combine_us"]
    dc_bytes = nbytes["dispatch"] + nbytes["combine"]
    value = dc_bytes / (dc_us * 1e-6) / 1e9
    dom = "dispatch" if cold["dispatch_us"] >= cold["combine_us"] else "combine"
    dom_us = cold[f"{dom}_us"]
    achieved = nbytes[dom] / (dom_us * 1e-6) / 1e9
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(cold["step_us"] / 1e3, 6),
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
        "dispatch_us": round(cold["dispatch_us"], 3),
        "combine_us": round(cold["combine_us"], 3),
        "dispatch_plus_combine_us": round(dc_us, 3),
        "route_us": round(cold["route_us"], 3),
        "step_us": round(cold["step_us"], 3),
        "hbm_frac_dispatch_plus_combine": round(value / HBM_PEAK_GBS, 4),
        "algorithmic_bytes": nbytes,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(profile_tag(args), dom)},
        "device_status": g["status"],
    }
    send_b, recv_b = two_stage_bytes(w, g["partial_rows"])
    # receive-side shuffle: each placed row read once and written once, plus
    # (counts, offsets) per expert read and the dense offsets written
    moved = 2 * g["placed_rows"] * nbytes_row(w) + 8 * w.E + 4 * (w.E + 1)
    extra = {}
    if "combine_send_us" in cold:
        extra["combine_partial"] = {
            "send_us": round(cold["combine_send_us"], 3), "recv_us": round(cold["combine_recv_us"], 3),
            "partial_rows": g["partial_rows"], "rows_per_token": round(g["partial_rows"] / w.tokens, 3),
            "send_GBps": round(send_b / (cold["combine_send_us"] * 1e-6) / 1e9, 1),
            "recv_GBps": round(recv_b / (cold["combine_recv_us"] * 1e-6) / 1e9, 1)}
    if "dispatch_recv_us" in cold:
        extra["split"] = {
            "dispatch_recv_us": round(cold["dispatch_recv_us"], 3),
            "combine_send_us": round(cold["combine_send_back_us"], 3),
            "bytes_each": moved,
            "dispatch_recv_GBps": round(moved / (cold["dispatch_recv_us"] * 1e-6) / 1e9, 1),
            "combine_send_GBps": round(moved / (cold["combine_send_back_us"] * 1e-6) / 1e9, 1)}
    if "route_grouped_us" in cold:
        G, kept = next_grouping(w)
        extra["route_grouped"] = {"groups": G, "groups_kept": kept,
                                  "route_us": round(cold["route_grouped_us"], 3)}
    if args.combine == "two-stage":
        line["two_stage_combine"] = extra.pop("combine_partial")
    if args.split:
        line["split"] = extra.pop("split")
    if extra:
        # adjacent paths on the same inputs, cold, one graph of K launches each
        line["next"] = extra
    if "warm" in g:
        wm = g["warm"]
        wus = wm["dispatch_us"] + wm["combine_us"]
        line["warm_cache_assisted"] = {
            "dispatch_us": round(wm["dispatch_us"], 3), "combine_us": round(wm["combine_us"], 3),
            "route_us": round(wm["route_us"], 3), "step_us": round(wm["step_us"], 3),
            "GBps": round(dc_bytes / (wus * 1e-6) / 1e9, 2)}
    if "floor" in g:
        fl = g["floor"]
        line["stream_floor"] = {
            "payload_bytes": fl["bytes"], "read_us": round(fl["read_us"], 3),
            "write_us": round(fl["write_us"], 3), "copy_us": round(fl["copy_us"], 3),
            "empty_launch_us": round(fl["empty_launch_us"], 3),
            "read_GBps": round(fl["bytes"] / (fl["read_us"] * 1e-6) / 1e9, 1),
            "write_GBps": round(fl["bytes"] / (fl["write_us"] * 1e-6) / 1e9, 1),
            "dispatch_over_write_floor": round(cold["dispatch_us"] / fl["write_us"], 3),
            "combine_over_read_floor": round(cold["combine_us"] / fl["read_us"], 3)}
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(w, inp, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
