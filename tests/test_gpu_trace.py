"""The tracing library (libmoe_trace.so: the same sources compiled with phase
stamps, read by bench.py --timeline) computes exactly what the product library
computes, and its router, one-launch dispatch and bf16 combine write one
record per wave whose stamps are in path order.  Run through the C ABI on the GPU."""
import ctypes
import os

import numpy as np
import pytest
import torch

from combine_moe_dispatch_amd import api, inputs

pytestmark = pytest.mark.gpu

TRACE_LIB = os.path.join(os.path.dirname(api.LIB_PATH), "libmoe_trace.so")
FUNCS = ("moe_route_topk", "moe_dispatch", "moe_expert_scale", "moe_combine")


def _run(lib, shape, inp, k, dev="cuda"):
    """route -> dispatch -> expert stand-in -> combine with `lib` behind the
    binding; returns every output on the host."""
    saved = api._lib
    try:
        api._lib = lib
        logits = torch.from_numpy(inp.logits).to(dev)
        x = torch.from_numpy(inp.x_bits.view(np.int16).copy()).to(dev)
        alpha = torch.from_numpy(inp.alpha).to(dev)
        ids, w = api.moe_route_topk(logits, None, k, api.MOE_SCORE_SIGMOID)
        lay = api.Layout.empty(shape, dev)
        recv, rs = api.alloc_recv(shape, dev, fill=0xFFFF)
        y, ys = api.alloc_recv(shape, dev, fill=0xFFFF)
        out = torch.empty(shape.num_tokens, shape.hidden, dtype=torch.int16, device=dev)
        api.moe_dispatch(shape, x, ids, recv, rs, lay, api.alloc_workspace(shape, dev))
        api.moe_expert_scale(shape, recv, rs, lay, alpha, y, ys)
        api.moe_combine(shape, y, ys, lay, w, out)
        torch.cuda.synchronize()
        return {"ids": ids.cpu(), "w": w.cpu(), "token_row": lay.token_row.cpu(),
                "expert_counts": lay.expert_counts.cpu(), "status": lay.status.cpu(),
                "recv": recv.cpu(), "y": y.cpu(), "out": out.cpu()}
    finally:
        api._lib = saved


def test_tracing_library_matches_and_records_in_order():
    T, H, E, k, N, C = 128, 1024, 64, 8, 8, 256
    print(f"[case] tracing library T={T} H={H} E={E} k={k} N={N} C={C}", flush=True)
    shape = api.Shape(T, H, E, k, N, C)
    inp = inputs.generate(T, H, E, 4242)
    lib = ctypes.CDLL(TRACE_LIB)
    for name in FUNCS:
        f, g = getattr(lib, name), getattr(api._lib, name)
        f.argtypes, f.restype = g.argtypes, g.restype
    lib.moe_trace_set_route.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
    lib.moe_trace_set_dispatch.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
    lib.moe_trace_set_combine.argtypes = [ctypes.c_void_p, ctypes.c_uint32]
    nvec = H // 8
    d_slots = (1 + T * -(-nvec // 256)) * 4
    c_slots = T * -(-nvec // 64)
    r_buf = torch.zeros(T * 8, dtype=torch.int64, device="cuda")
    d_buf = torch.zeros(d_slots * 8, dtype=torch.int64, device="cuda")
    c_buf = torch.zeros(c_slots * 8, dtype=torch.int64, device="cuda")
    assert lib.moe_trace_set_route(r_buf.data_ptr(), T) == 0
    assert lib.moe_trace_set_dispatch(d_buf.data_ptr(), d_slots) == 0
    assert lib.moe_trace_set_combine(c_buf.data_ptr(), c_slots) == 0
    try:
        traced = _run(lib, shape, inp, k)
    finally:
        assert lib.moe_trace_set_route(None, 0) == 0
        assert lib.moe_trace_set_dispatch(None, 0) == 0
        assert lib.moe_trace_set_combine(None, 0) == 0
    plain = _run(api._lib, shape, inp, k)
    for key in plain:
        assert torch.equal(plain[key], traced[key]), key
    # records: block 0 (metadata) and every scatter block's waves, stamps in
    # path order; every combine block
    d = d_buf.view(-1, 8).cpu().numpy()
    written = d[:, 7] == 1
    blocks = int(written.sum()) // 4
    assert written[:4].all() and blocks >= 1 + T and written[: 4 * blocks].all()
    assert not written[4 * blocks:].any()
    assert (np.diff(d[written, :6], axis=1) >= 0).all()
    rr = r_buf.view(-1, 8).cpu().numpy()
    assert (rr[:, 7] == 1).all()                      # one record per token
    assert (np.diff(rr[:, :6], axis=1) >= 0).all()
    c = c_buf.view(-1, 8).cpu().numpy()
    assert (c[:, 7] == 1).all()
    assert (np.diff(c[:, [0, 1, 2, 4, 5]], axis=1) >= 0).all()
