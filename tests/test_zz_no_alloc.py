"""moe_dispatch_static (no workspace argument, library-held scratch) against
moe_dispatch with a caller workspace, through the C ABI.

Each case makes two moe_dispatch_static calls in a row on one GPU, the second
with a smaller input, so the second reads scratch the first left behind.  The
layout metadata, the status word and the whole poisoned receive buffer
(canary rows included) must equal moe_dispatch's bit for bit.
"""
import numpy as np
import pytest
import torch

from combine_moe_dispatch_amd import api, inputs

from gpu_chain import CANARY_ROWS, _poisoned

pytestmark = pytest.mark.gpu

LAYOUT_FIELDS = ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row",
                 "row_src", "status")


def _dispatch(shape, x, ids, static):
    rows = api.moe_recv_rows(shape)
    lay = api.Layout.empty(shape, "cuda", with_row_src=True)
    lay.status.fill_(-1)
    full, recv, sfull, rs = _poisoned(shape, rows)
    if static:
        api.moe_dispatch_static(shape, x, ids, recv, rs, lay)
    else:
        api.moe_dispatch(shape, x, ids, recv, rs, lay, api.alloc_workspace(shape, "cuda"))
    return lay, full, sfull


def _inputs(T, H, E, k, seed, bad=False):
    inp = inputs.generate(T, H, E, seed)
    ids = inputs.random_ids(T, k, E, seed + 1, distinct=False)
    if bad and T:
        ids[::9, 0] = E + 1
    x = torch.from_numpy(inp.x_bits.view(np.int16).copy()).cuda()
    return x, torch.from_numpy(ids).cuda()


# pairs of calls: (T, H, E, k, N, C, payload), the second smaller
CASES = [
    ((3000, 512, 256, 8, 32, 0, 0), (700, 512, 256, 8, 32, 0, 0)),          # packed, multi-kernel
    ((1100, 1024, 64, 8, 8, 1200, 1), (600, 1024, 64, 8, 8, 1200, 1)),      # fp8, capacity overflow
    ((8192, 256, 1024, 8, 64, 0, 0), (600, 256, 1024, 4, 64, 0, 0)),        # E at the maximum
    ((2000, 256, 32, 8, 4, 0, 0), (128, 256, 32, 8, 4, 0, 0)),              # then the one-kernel path
]


@pytest.mark.parametrize("first,second", CASES, ids=lambda c: "T{}_E{}_k{}_C{}_p{}".format(
    c[0], c[2], c[3], c[5], c[6]))
def test_static_scratch_matches_workspace_dispatch(first, second):
    for n, (T, H, E, k, N, C, payload) in enumerate((first, second)):
        print(f"[case] moe_dispatch_static call {n}: T={T} H={H} E={E} k={k} N={N} C={C} "
              f"p={payload}", flush=True)
        shape = api.Shape(T, H, E, k, N, C, payload)
        assert api.moe_dispatch_workspace_size(shape) <= api.MOE_STATIC_SCRATCH_BYTES
        x, ids = _inputs(T, H, E, k, seed=31 * T + E + n, bad=(n == 1))
        ref_lay, ref_full, ref_sfull = _dispatch(shape, x, ids, static=False)
        lay, full, sfull = _dispatch(shape, x, ids, static=True)
        torch.cuda.synchronize()
        for f in LAYOUT_FIELDS:
            assert torch.equal(getattr(lay, f), getattr(ref_lay, f)), f
        assert torch.equal(full, ref_full), "receive rows"
        if payload:
            assert torch.equal(sfull.view(torch.int32), ref_sfull.view(torch.int32)), "scales"
        assert full.shape[0] == api.moe_recv_rows(shape) + CANARY_ROWS
