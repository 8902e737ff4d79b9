"""Calls on several streams at once: four problems of different shapes (both
payloads, both dispatch paths), each with its own buffers and workspace,
launched route -> dispatch -> expert stand-in -> combine on four streams of
default priority without synchronising in between, give byte-identical
results to the same calls made one problem at a time.  The library keeps no
state between calls apart from the allocation-free dispatch's scratch, so the
calls are independent."""
import numpy as np
import pytest
import torch

from combine_moe_dispatch_amd import api, inputs

pytestmark = pytest.mark.gpu

PROBLEMS = [
    (128, 7168, 256, 8, 32, 1024, 0),   # one launch, fixed capacity
    (1000, 1024, 64, 8, 8, 0, 0),       # multi-kernel layout, packed
    (256, 2048, 64, 4, 8, 200, 1),      # fp8, capacity overflow
    (700, 512, 32, 6, 4, 0, 1),         # fp8, multi-kernel layout
]


def _setup(i, T, H, E, k, N, C, payload):
    dev = "cuda"
    shape = api.Shape(T, H, E, k, N, C, payload)
    inp = inputs.generate(T, H, E, 900 + i)
    b = {"shape": shape,
         "logits": torch.from_numpy(inp.logits).to(dev),
         "x": torch.from_numpy(inp.x_bits.view(np.int16).copy()).to(dev),
         "alpha": torch.from_numpy(inp.alpha).to(dev),
         "ids": torch.empty(T, k, dtype=torch.int32, device=dev),
         "w": torch.empty(T, k, dtype=torch.float32, device=dev),
         "lay": api.Layout.empty(shape, dev),
         "ws": api.alloc_workspace(shape, dev),
         "out": torch.empty(T, H, dtype=torch.int16, device=dev)}
    b["recv"], b["rs"] = api.alloc_recv(shape, dev)
    b["y"], b["ys"] = api.alloc_recv(shape, dev)
    return b


def _chain(b, stream):
    s = b["shape"]
    api.moe_route_topk(b["logits"], None, s.top_k, api.MOE_SCORE_SIGMOID, b["ids"], b["w"],
                       stream=stream)
    api.moe_dispatch(s, b["x"], b["ids"], b["recv"], b["rs"], b["lay"], b["ws"], stream=stream)
    api.moe_expert_scale(s, b["recv"], b["rs"], b["lay"], b["alpha"], b["y"], b["ys"],
                         stream=stream)
    api.moe_combine(s, b["y"], b["ys"], b["lay"], b["w"], b["out"], stream=stream)


def _snapshot(b):
    rows = b["lay"].token_row.flatten()
    used = rows[rows >= 0].long()
    snap = {"ids": b["ids"].clone(), "w": b["w"].clone(), "token_row": b["lay"].token_row.clone(),
            "counts": b["lay"].expert_counts.clone(), "status": b["lay"].status.clone(),
            "recv": b["recv"][used].clone(), "out": b["out"].clone()}
    if b["rs"] is not None:
        snap["rs"] = b["rs"][used].view(torch.int32).clone()
    return snap


def test_four_streams_match_one_at_a_time():
    print("[case] four problems on four streams", flush=True)
    bufs = [_setup(i, *p) for i, p in enumerate(PROBLEMS)]
    main = torch.cuda.current_stream()
    for b in bufs:                      # one at a time, synchronised
        _chain(b, main)
        torch.cuda.synchronize()
    ref = [_snapshot(b) for b in bufs]
    for b in bufs:                      # clear every output
        for key in ("ids", "w", "recv", "y", "out"):
            b[key].fill_(0)
        for key in ("rs", "ys"):
            if b[key] is not None:
                b[key].fill_(0)
        b["lay"].token_row.fill_(-5)
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in bufs]
    for rep in range(3):                # all at once, three times over
        for b, st in zip(bufs, streams):
            _chain(b, st)
        torch.cuda.synchronize()
        for i, b in enumerate(bufs):
            got = _snapshot(b)
            for key, v in ref[i].items():
                assert torch.equal(v, got[key]), (rep, i, key)
