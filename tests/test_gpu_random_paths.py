"""GPU parity of the adjacent paths on seeded random shapes (drawn as in
test_gpu_random_shapes): the sender-side partial-reduction combine (partial
rows, their ranks and the output bit-exact against the oracle's fp32 chains),
the send/receive split (both shuffles bit-exact, the split chain equal to the
one-call chain), every source dispatching at once (layout, per-source counts
and offsets, receive rows and the world's combine bit-exact) and the
allocation-free dispatch (equal to moe_dispatch); and the multi-kernel
layout with workspaces holding arbitrary bytes."""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api, inputs

from gpu_chain import dev_u16, host_u16
from test_gpu_random_shapes import draw_case

pytestmark = pytest.mark.gpu


def _case(seed, bad_ok=True):
    T, H, E, k, N, C, payload, distinct, bad = draw_case(1000 + seed)
    inp = inputs.generate(T, H, E, 1300 + seed)
    ids = inputs.random_ids(T, k, E, 1400 + seed, distinct=distinct)
    if bad and bad_ok and T:
        rng = np.random.default_rng(1500 + seed)
        for _ in range(1 + T // 50):
            ids[rng.integers(0, T), rng.integers(0, k)] = int(rng.choice([-1, E, E + 7]))
    wts = inputs.random_weights(T, k, 1600 + seed)
    return (T, H, E, k, N, C, payload), inp, ids, wts


def _host(t, fp8):
    return t.cpu().numpy() if fp8 else host_u16(t)


def _dispatch(shape, inp, ids, fill):
    T, H = shape.num_tokens, shape.hidden
    dev = "cuda"
    x = dev_u16(inp.x_bits) if T else torch.empty(0, H, dtype=torch.int16, device=dev)
    d_ids = torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to(dev)
    lay = api.Layout.empty(shape, dev)
    recv, rs = api.alloc_recv(shape, dev, fill=fill)
    api.moe_dispatch(shape, x, d_ids, recv, rs, lay, api.alloc_workspace(shape, dev))
    return x, d_ids, lay, recv, rs


@pytest.mark.parametrize("seed", range(20))
def test_random_two_stage_combine(seed):
    (T, H, E, k, N, C, payload), inp, ids, wts = _case(seed)
    print(f"[case] random two-stage seed={seed} T={T} H={H} E={E} k={k} N={N} C={C} "
          f"p={payload}", flush=True)
    dev = "cuda"
    shape = api.Shape(T, H, E, k, N, C, payload)
    M = api.partial_slots(shape)
    _, d_ids, lay, recv, rs = _dispatch(shape, inp, ids, 0x7F if payload else 0xFFFF)
    y, ys = api.alloc_recv(shape, dev)
    api.moe_expert_scale(shape, recv, rs, lay, torch.from_numpy(inp.alpha).to(dev), y, ys)
    partial = torch.full((T, M, H), -1, dtype=torch.int16, device=dev)
    prank = torch.full((T, M), -7, dtype=torch.int32, device=dev)
    d_w = torch.from_numpy(wts).to(dev)
    api.moe_combine_partial_send(shape, y, ys, lay, d_ids, d_w, partial, prank)
    out = torch.empty(T, H, dtype=torch.int16, device=dev)
    api.moe_combine_partial_recv(shape, partial, prank, out)
    torch.cuda.synchronize()
    if T == 0:
        return
    g_y, g_ys = _host(y, payload), (ys.cpu().numpy() if payload else None)
    tr = lay.token_row.cpu().numpy()
    g_partial, g_prank = host_u16(partial), prank.cpu().numpy()
    o_partial, o_prank = oracle.combine_send(g_y, g_ys, tr, ids, wts, E, N, exact=False)
    assert np.array_equal(g_prank, o_prank)
    assert np.array_equal(g_partial, o_partial)
    assert np.array_equal(host_u16(out), oracle.combine_recv(g_partial, g_prank, exact=False))


def _dense_layout(shape, gemm_offsets):
    E = shape.num_experts
    lay = api.Layout.empty(api.Shape(shape.num_tokens, shape.hidden, E, shape.top_k,
                                     shape.num_ranks, 0, shape.payload), "cuda")
    lay.expert_offsets.copy_(gemm_offsets[:E])
    lay.expert_counts.copy_(gemm_offsets[1:] - gemm_offsets[:E])
    return lay


@pytest.mark.parametrize("seed", range(20))
def test_random_split_chain(seed):
    (T, H, E, k, N, C, payload), inp, ids, wts = _case(100 + seed)
    print(f"[case] random split seed={seed} T={T} H={H} E={E} k={k} N={N} C={C} "
          f"p={payload}", flush=True)
    fp8, dev = payload == 1, "cuda"
    fill = 0x7F if fp8 else 0xFFFF
    shape = api.Shape(T, H, E, k, N, C, payload)
    _, _, lay, recv, rs = _dispatch(shape, inp, ids, fill)
    alpha, d_w = torch.from_numpy(inp.alpha).to(dev), torch.from_numpy(wts).to(dev)
    dense_shape = api.Shape(T, H, E, k, N, 0, payload)
    gx, gs = api.alloc_recv(dense_shape, dev, fill=fill)
    goff = torch.full((E + 1,), -3, dtype=torch.int32, device=dev)
    api.moe_dispatch_recv(shape, recv, rs, lay, gx, gs, goff)
    gy, gys = api.alloc_recv(dense_shape, dev, fill=fill)
    api.moe_expert_scale(dense_shape, gx, gs, _dense_layout(shape, goff), alpha, gy, gys)
    ey, eys = api.alloc_recv(shape, dev, fill=fill)
    api.moe_combine_send(shape, gy, gys, lay, ey, eys)
    out = torch.full((T, H), -1, dtype=torch.int16, device=dev)
    api.moe_combine(shape, ey, eys, lay, d_w, out)
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
    assert torch.equal(out, out1)


@pytest.mark.parametrize("seed", range(20))
def test_random_sources(seed):
    rng = np.random.default_rng(2000 + seed)
    (T0, H, E, k, N, C, payload), _, _, _ = _case(200 + seed)
    S = int(rng.integers(2, 9))
    T = int(T0 // S) if rng.random() < 0.5 else int(rng.choice([128, 256]) // max(1, k // 4))
    T = max(0, min(T, 4000 // S))
    if C:
        C = max(1, min(C, 4_000_000 // max(1, N * H)))
    print(f"[case] random sources seed={seed} S={S} T={T} H={H} E={E} k={k} N={N} C={C} "
          f"p={payload}", flush=True)
    inp = inputs.generate(S * T, H, E, 2100 + seed)
    ids = np.stack([inputs.random_ids(T, k, E, 2200 + 10 * seed + s) for s in range(S)]) if T else \
        np.zeros((S, 0, k), np.int32)
    wts = inputs.random_weights(S * T, k, 2300 + seed)
    one = api.Shape(T, H, E, k, N, C, payload)
    world = api.world_shape(one, S)
    dev = "cuda"
    x = dev_u16(inp.x_bits) if T else torch.empty(0, H, dtype=torch.int16, device=dev)
    d_ids = torch.from_numpy(ids.reshape(S * T, k).copy()).to(dev)
    lay = api.Layout.empty(world, dev)
    recv, rs = api.alloc_recv(world, dev, fill=0x7F if payload else 0xFFFF)
    sc = torch.full((S, E), -9, dtype=torch.int32, device=dev)
    so = torch.full((E, S), -9, dtype=torch.int32, device=dev)
    api.moe_dispatch_sources(one, S, x, d_ids, recv, rs, lay, sc, so, api.alloc_workspace(world, dev))
    torch.cuda.synchronize()
    o = oracle.layout_sources(ids, E, N, C)
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row",
                "source_counts", "source_offsets"):
        got = {"source_counts": sc, "source_offsets": so}.get(key)
        got = getattr(lay, key) if got is None else got
        assert np.array_equal(got.cpu().numpy().reshape(o[key].shape), o[key]), key
    assert int(lay.status.item()) == o["status"]
    if T == 0:
        return
    tr = o["token_row"]
    if payload:
        o_recv, o_rs = oracle.dispatch_fp8(inp.x_bits, tr, o["rows"], fill=0x7F)
        assert np.array_equal(recv.cpu().numpy(), o_recv)
        assert np.array_equal(rs.cpu().numpy().view(np.uint32), o_rs.view(np.uint32))
    else:
        assert np.array_equal(host_u16(recv), oracle.dispatch_bf16(inp.x_bits, tr, o["rows"], fill=0xFFFF))
    out = torch.empty(S * T, H, dtype=torch.int16, device=dev)
    api.moe_combine(world, recv, rs, lay, torch.from_numpy(wts).to(dev), out)
    torch.cuda.synchronize()
    y = recv.cpu().numpy() if payload else host_u16(recv)
    ys = rs.cpu().numpy() if payload else None
    assert np.array_equal(host_u16(out), oracle.combine_f32_ordered(y, ys, tr, wts))


@pytest.mark.parametrize("seed", range(12))
def test_random_static_dispatch(seed):
    (T, H, E, k, N, C, payload), inp, ids, _ = _case(300 + seed)
    shape = api.Shape(T, H, E, k, N, C, payload)
    if api.moe_dispatch_workspace_size(shape) > api.MOE_STATIC_SCRATCH_BYTES:
        pytest.skip("needs more scratch than the static array holds")
    print(f"[case] random static dispatch seed={seed} T={T} H={H} E={E} k={k} N={N} C={C} "
          f"p={payload}", flush=True)
    fill = 0x7F if payload else 0xFFFF
    x, d_ids, lay, recv, rs = _dispatch(shape, inp, ids, fill)
    lay2 = api.Layout.empty(shape, "cuda")
    recv2, rs2 = api.alloc_recv(shape, "cuda", fill=fill)
    api.moe_dispatch_static(shape, x, d_ids, recv2, rs2, lay2)
    torch.cuda.synchronize()
    for f in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row",
              "status"):
        assert torch.equal(getattr(lay, f), getattr(lay2, f)), f
    assert torch.equal(recv, recv2)
    if payload:
        assert torch.equal(rs.view(torch.int32), rs2.view(torch.int32))


@pytest.mark.parametrize("fill", [0x00, 0xFF, 0x7F, 0x80])
def test_workspace_contents_do_not_matter(fill):
    """The multi-kernel layout's workspace needs no initialisation: filled with
    any byte pattern before each call (and reused by the next, larger or
    smaller, call), every result still equals the oracle's."""
    import oracle
    from gpu_chain import check_chain, run_chain
    print(f"[case] workspace filled with {fill:#x}", flush=True)
    shapes = [(1500, 256, 64, 8, 8, 0, 0), (600, 512, 32, 8, 4, 900, 1),
              (3000, 128, 128, 4, 16, 0, 0)]
    big = max(api.moe_dispatch_workspace_size(api.Shape(*s)) for s in shapes)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    for i, (T, H, E, k, N, C, payload) in enumerate(shapes):
        shape = api.Shape(T, H, E, k, N, C, payload)
        inp = inputs.generate(T, H, E, 3100 + i)
        ids = inputs.random_ids(T, k, E, 3200 + i, distinct=(i != 1))
        wts = inputs.random_weights(T, k, 3300 + i)
        ws.fill_(fill)
        x = dev_u16(inp.x_bits)
        d_ids = torch.from_numpy(ids).cuda()
        lay = api.Layout.empty(shape, "cuda")
        recv, rs = api.alloc_recv(shape, "cuda", fill=0x7F if payload else 0xFFFF)
        need = api.moe_dispatch_workspace_size(shape)
        api.moe_dispatch(shape, x, d_ids, recv, rs, lay, ws[:need])
        torch.cuda.synchronize()
        o = oracle.layout(ids, E, N, C)
        for f in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row"):
            assert np.array_equal(getattr(lay, f).cpu().numpy().reshape(o[f].shape), o[f]), f
        assert int(lay.status.item()) == o["status"]
        if payload:
            o_recv, o_rs = oracle.dispatch_fp8(inp.x_bits, o["token_row"], o["rows"], fill=0x7F)
            assert np.array_equal(recv.cpu().numpy(), o_recv)
            assert np.array_equal(rs.cpu().numpy().view(np.uint32), o_rs.view(np.uint32))
        else:
            assert np.array_equal(host_u16(recv), oracle.dispatch_bf16(inp.x_bits, o["token_row"],
                                                                       o["rows"], fill=0xFFFF))
