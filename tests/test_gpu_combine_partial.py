"""GPU parity of the two-stage combine (sender-side partial reduction).

Stage 1 (moe_combine_partial_send) and stage 2 (moe_combine_partial_recv) through the C ABI
against the oracle fed the GPU's own inputs to each stage: bit-exact against
the fp32-chain forms, within 1 bf16 ulp of the double-precision forms; unused
partial rows stay poisoned.  The result's distance from the single-stage
combine is the precision cost of accumulating on the sender side.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api, inputs

from gpu_chain import host_u16, ulp_dist

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("T,H,E,k,N,C,payload,skew", [
    (128, 7168, 256, 8, 32, 1024, 0, False),   # DeepSeek-V3 decode, EP32
    (128, 7168, 256, 8, 8, 4096, 0, False),    # EP8: fewer ranks per token
    (512, 7168, 256, 8, 32, 4096, 1, False),   # fp8 payload
    (64, 1024, 32, 16, 16, 0, 0, False),       # up to 16 ranks per token: two passes
    (64, 512, 32, 16, 16, 0, 1, False),        # fp8, up to 16 ranks: four passes
    (100, 256, 16, 4, 4, 60, 0, True),         # capacity-skipped pairs
    (50, 536, 64, 8, 8, 0, 0, False),          # ragged row: last chunk has 3 live lanes < k
    (0, 256, 16, 4, 4, 0, 0, False),           # no tokens
    (2400, 7168, 256, 8, 32, 0, 0, False),     # 34 MB output: device-scope stores
    (60, 512, 1024, 32, 32, 0, 0, False),      # k and E at the library maximum
    (40, 1024, 1024, 32, 64, 0, 1, False),     # the same with fp8, 64 ranks
    (80, 256, 16, 4, 1, 0, 0, False),          # one rank: one partial row per token
])
def test_two_stage_combine(T, H, E, k, N, C, payload, skew):
    print(f"[case] two-stage T={T} H={H} E={E} k={k} N={N} C={C} p={payload}", flush=True)
    dev = "cuda"
    inp = inputs.generate(T, H, E, 500 + E + k)
    ids = inputs.random_ids(T, k, E, 501, distinct=True, hot=(0 if skew else None))
    wts = inputs.random_weights(T, k, 502)
    shape = api.Shape(T, H, E, k, N, C, payload)
    M = api.partial_slots(shape)
    x = torch.from_numpy(inp.x_bits.view(np.int16).copy()).to(dev)
    d_ids = torch.from_numpy(ids).to(dev)
    d_w = torch.from_numpy(wts).to(dev)
    lay = api.Layout.empty(shape, dev)
    ws = api.alloc_workspace(shape, dev)
    recv, rs = api.alloc_recv(shape, dev)
    api.moe_dispatch(shape, x, d_ids, recv, rs, lay, ws)
    y, ys = api.alloc_recv(shape, dev)
    api.moe_expert_scale(shape, recv, rs, lay, torch.from_numpy(inp.alpha).to(dev), y, ys)
    partial = torch.full((T, M, H), -1, dtype=torch.int16, device=dev)   # 0xFFFF poison
    prank = torch.full((T, M), -7, dtype=torch.int32, device=dev)
    api.moe_combine_partial_send(shape, y, ys, lay, d_ids, d_w, partial, prank)
    out = torch.empty(T, H, dtype=torch.int16, device=dev)
    api.moe_combine_partial_recv(shape, partial, prank, out)
    torch.cuda.synchronize()
    if T == 0:
        return
    g_y = y.cpu().numpy() if payload else host_u16(y)
    g_ys = ys.cpu().numpy() if payload else None
    tr = lay.token_row.cpu().numpy()
    g_partial, g_prank, g_out = host_u16(partial), prank.cpu().numpy(), host_u16(out)
    o_partial, o_prank = oracle.combine_send(g_y, g_ys, tr, ids, wts, E, N, exact=False)
    assert np.array_equal(g_prank, o_prank)
    assert np.array_equal(g_partial, o_partial)            # used slots and untouched poison
    assert np.array_equal(g_out, oracle.combine_recv(g_partial, g_prank, exact=False))
    x_partial, _ = oracle.combine_send(g_y, g_ys, tr, ids, wts, E, N, exact=True)
    used = g_prank >= 0
    assert ulp_dist(g_partial[used], x_partial[used]).max() <= 1
    assert ulp_dist(g_out, oracle.combine_recv(g_partial, g_prank, exact=True)).max() <= 1
    # precision cost against the single-stage combine (same-sign terms here)
    single = oracle.combine_exact(g_y, g_ys, tr, wts)
    d = ulp_dist(g_out, single)
    print(f"[two-stage] ulp vs single-stage: max {int(d.max())} mean {d.mean():.4f} "
          f"exact {(d == 0).mean():.4f} ranks/token {used.sum(1).mean():.2f}", flush=True)
    assert d.max() <= 2
