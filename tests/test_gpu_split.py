"""GPU parity of the send/receive split.

moe_dispatch (send half) -> moe_dispatch_recv (receive-side shuffle into the
grouped GEMM's dense input) -> experts on the dense rows -> moe_combine_send
(back to the receive regions) -> moe_combine (receive half): each shuffle
bit-exact against the oracle, the whole split chain bit-identical to the
one-call chain, and the chain captured in a HIP graph with other work (a
shared-expert stand-in) overlapping on a second stream.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api, inputs

from gpu_chain import dev_u16, host_u16

pytestmark = pytest.mark.gpu


def _dense_layout(shape, gemm_offsets):
    """A packed layout that describes the dense GEMM rows (for the stand-in)."""
    E = shape.num_experts
    lay = api.Layout.empty(api.Shape(shape.num_tokens, shape.hidden, E, shape.top_k,
                                     shape.num_ranks, 0, shape.payload), "cuda")
    lay.expert_offsets.copy_(gemm_offsets[:E])
    lay.expert_counts.copy_(gemm_offsets[1:] - gemm_offsets[:E])
    return lay


def _host(t, fp8):
    return t.cpu().numpy() if fp8 else host_u16(t)


@pytest.mark.parametrize("T,H,E,k,N,C,payload,hot", [
    (128, 7168, 256, 8, 32, 1024, 0, None),   # DeepSeek-V3 decode regions (with gaps)
    (128, 1024, 32, 8, 4, 200, 0, 3),         # capacity overflow: cut segments
    (200, 512, 64, 4, 8, 0, 0, None),         # packed regions
    (96, 1024, 32, 8, 4, 240, 1, 1),          # fp8 with overflow
    (0, 256, 8, 2, 2, 16, 0, None),           # no tokens
    (64, 512, 384, 8, 16, 192, 0, None),      # 384 experts: 8 per lane
    (32, 256, 1024, 8, 16, 0, 1, None),       # 1024 experts: 16 per lane, fp8
    (24, 8704, 64, 4, 4, 0, 0, None),         # rows of more than 1024 vectors: two passes
    (1040, 256, 64, 8, 8, 1000, 1, 2),        # > 8192 rows: 4 rows per wave, fp8, overflow
    (100, 512, 30, 4, 5, 100, 0, None),       # E not a multiple of 4: 4-byte count loads
    (60, 1024, 90, 6, 6, 0, 1, 2),            # the same, fp8, packed regions
    (40, 512, 256, 32, 32, 0, 0, None),       # k at the library maximum
])
def test_split_chain(T, H, E, k, N, C, payload, hot):
    print(f"[case] split T={T} H={H} E={E} k={k} N={N} C={C} p={payload}", flush=True)
    fp8 = payload == 1
    dev = "cuda"
    inp = inputs.generate(T, H, E, 700 + E)
    ids = inputs.random_ids(T, k, E, 701, hot=hot)
    wts = inputs.random_weights(T, k, 702)
    shape = api.Shape(T, H, E, k, N, C, payload)
    x = dev_u16(inp.x_bits) if T else torch.empty(0, H, dtype=torch.int16, device=dev)
    d_ids, d_w = torch.from_numpy(ids).to(dev), torch.from_numpy(wts).to(dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    lay = api.Layout.empty(shape, dev)
    ws = api.alloc_workspace(shape, dev)
    fill = 0x7F if fp8 else 0xFFFF
    recv, rs = api.alloc_recv(shape, dev, fill=fill)
    api.moe_dispatch(shape, x, d_ids, recv, rs, lay, ws)
    # receive half: dense GEMM input
    dense_shape = api.Shape(T, H, E, k, N, 0, payload)   # T*k rows
    gx, gs = api.alloc_recv(dense_shape, dev, fill=fill)
    goff = torch.full((E + 1,), -3, dtype=torch.int32, device=dev)
    api.moe_dispatch_recv(shape, recv, rs, lay, gx, gs, goff)
    # experts on the dense rows, then back to the regions, then the combine
    gy, gys = api.alloc_recv(dense_shape, dev, fill=fill)
    dlay = _dense_layout(shape, goff)
    api.moe_expert_scale(dense_shape, gx, gs, dlay, alpha, gy, gys)
    ey, eys = api.alloc_recv(shape, dev, fill=fill)
    api.moe_combine_send(shape, gy, gys, lay, ey, eys)
    out = torch.full((T, H), -1, dtype=torch.int16, device=dev)
    api.moe_combine(shape, ey, eys, lay, d_w, out)
    # the one-call chain on the regions
    y1, ys1 = api.alloc_recv(shape, dev, fill=fill)
    api.moe_expert_scale(shape, recv, rs, lay, alpha, y1, ys1)
    out1 = torch.full((T, H), -1, dtype=torch.int16, device=dev)
    api.moe_combine(shape, y1, ys1, lay, d_w, out1)
    torch.cuda.synchronize()

    counts, offs = lay.expert_counts.cpu().numpy(), lay.expert_offsets.cpu().numpy()
    o_dense, o_ds, o_off = oracle.gemm_io(True, _host(recv, fp8), None if rs is None else rs.cpu().numpy(),
                                          counts, offs, E, N, C, T * k, fill)
    assert np.array_equal(goff.cpu().numpy(), o_off)
    assert np.array_equal(_host(gx, fp8), o_dense)
    if fp8:
        assert np.array_equal(gs.cpu().numpy().view(np.uint32), o_ds.view(np.uint32))
    o_back, o_bs, _ = oracle.gemm_io(False, _host(gy, fp8), None if gys is None else gys.cpu().numpy(),
                                     counts, offs, E, N, C, api.moe_recv_rows(shape), fill)
    assert np.array_equal(_host(ey, fp8), o_back)
    if fp8:
        assert np.array_equal(eys.cpu().numpy().view(np.uint32), o_bs.view(np.uint32))
    # split chain == one-call chain, bit for bit
    assert torch.equal(out, out1)


def test_split_chain_graph_with_overlap():
    """The split chain captured once, with a shared-expert stand-in (fp32
    matmul) forked onto a second stream between the halves; every replay,
    with eager work in between, equals the eager result."""
    w = inputs.WORKLOADS["dsv3_decode"]
    inp = inputs.generate_for(w)
    dev = "cuda"
    shape = api.Shape(w.T, w.H, w.E, w.k, w.N, w.C)
    dense_shape = api.Shape(w.T, w.H, w.E, w.k, w.N, 0)
    lg = torch.from_numpy(inp.logits).to(dev)
    x = dev_u16(inp.x_bits)
    xf = torch.from_numpy(inp.x_bits.astype(np.uint32) << 16).view(torch.float32).to(dev)[:, :1024]
    wsh = torch.randn(1024, 256, device=dev)
    alpha = torch.from_numpy(inp.alpha).to(dev)
    ids = torch.empty(w.T, w.k, dtype=torch.int32, device=dev)
    wt = torch.empty(w.T, w.k, dtype=torch.float32, device=dev)
    lay = api.Layout.empty(shape, dev)
    recv, _ = api.alloc_recv(shape, dev, fill=0)
    gx, _ = api.alloc_recv(dense_shape, dev, fill=0)
    gy, _ = api.alloc_recv(dense_shape, dev, fill=0)
    ey, _ = api.alloc_recv(shape, dev, fill=0)
    goff = torch.zeros(w.E + 1, dtype=torch.int32, device=dev)
    dlay = api.Layout.empty(dense_shape, dev)
    out = torch.empty(w.T, w.H, dtype=torch.int16, device=dev)
    shared = torch.empty(w.T, 256, device=dev)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()

    def step():
        api.moe_route_topk(lg, None, w.k, w.score, ids, wt, stream=main)
        api.moe_dispatch(shape, x, ids, recv, None, lay, None, stream=main)
        side.wait_stream(main)
        with torch.cuda.stream(side):
            torch.matmul(xf, wsh, out=shared)          # overlaps the receive half
        api.moe_dispatch_recv(shape, recv, None, lay, gx, None, goff, stream=main)
        with torch.cuda.stream(main):
            dlay.expert_offsets.copy_(goff[:w.E])
            torch.sub(goff[1:], goff[:w.E], out=dlay.expert_counts)
        api.moe_expert_scale(dense_shape, gx, None, dlay, alpha, gy, None, stream=main)
        api.moe_combine_send(shape, gy, None, lay, ey, None, stream=main)
        api.moe_combine(shape, ey, None, lay, wt, out, stream=main)
        main.wait_stream(side)

    main.wait_stream(torch.cuda.current_stream())
    step()
    torch.cuda.synchronize()
    ref, ref_shared = out.clone(), shared.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=main):
        step()
    for i in range(3):
        out.zero_()
        shared.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(main):
            g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref), i
        assert torch.equal(shared, ref_shared), i
