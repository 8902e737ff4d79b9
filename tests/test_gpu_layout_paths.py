"""GPU parity of the multi-kernel layout in both its forms and at many
chunks, and of every dispatch path with an id list that does not start on a
16-byte boundary.

The multi-kernel layout (past 8192 pairs) ranks pairs inside chunks of 1024
(token, slot) pairs and carries bases across chunks.  Up to 16 chunks it is
one launch whose blocks read the id list in 16-byte vectors, so a misaligned
list takes the two-launch form instead.  These cases reach 9, 16, 17, 64 and
65 chunks (ragged last chunks among them), k = 32 and one rank holding every
expert, and the one-kernel path at its limit.  Each case also runs with its id
list one element into its allocation (4 bytes past a 16-byte boundary), which
the C ABI accepts.  Every stage is checked against the oracle with the bars of
the other parity tests."""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api, inputs

from gpu_chain import check_chain, dev_u16, run_chain

pytestmark = pytest.mark.gpu

CASES = [
    # T, H, E, k, N, C, payload, bad ids
    (8192, 64, 256, 8, 32, 0, 0, False),     # 65536 pairs: 64 chunks
    (8193, 64, 256, 8, 32, 0, 0, True),      # 65 chunks, the last one ragged
    (8192, 128, 96, 8, 3, 21000, 1, False),  # fp8, 64 chunks, a capacity that overflows
    (1025, 64, 1024, 8, 4, 0, 0, True),      # 8200 pairs: just past the one-kernel dispatch
    (2000, 64, 256, 8, 32, 0, 0, True),      # 16 chunks, the last one ragged
    (2049, 64, 256, 8, 32, 0, 0, False),     # 17 chunks
    (2048, 64, 96, 32, 3, 21000, 0, False),  # k = 32, 64 chunks, a capacity that overflows
    (10000, 64, 8, 1, 1, 0, 0, False),       # k = 1, one rank, 10 chunks (ragged)
    (300, 256, 256, 8, 32, 0, 0, True),      # one-kernel dispatch (2400 pairs)
    (1024, 128, 256, 8, 32, 64, 1, False),   # one-kernel fp8 dispatch at its limit (8192 pairs)
]


@pytest.mark.parametrize("misalign", [False, True], ids=["aligned", "misaligned"])
@pytest.mark.parametrize("case", range(len(CASES)))
def test_layout_many_chunks(case, misalign):
    T, H, E, k, N, C, payload, bad = CASES[case]
    print(f"[case] layout case={case} misalign={misalign} T={T} H={H} E={E} k={k} N={N} "
          f"C={C} payload={payload} bad={bad}", flush=True)
    inp = inputs.generate(T, H, E, 700 + case)
    ids = inputs.random_ids(T, k, E, 710 + case, distinct=True)
    if bad:
        rng = np.random.default_rng(720 + case)
        for _ in range(1 + T // 50):
            ids[rng.integers(0, T), rng.integers(0, k)] = int(rng.choice([-1, E, E + 7]))
    wts = inputs.random_weights(T, k, 730 + case)
    shape = api.Shape(T, H, E, k, N, C, payload)
    g = run_chain(shape, inp.x_bits, inp.alpha, ids=ids, weights=wts, misalign_ids=misalign)
    check_chain(shape, g, inp.x_bits, inp.alpha)


@pytest.mark.parametrize("T", [1100, 2100], ids=["layout_one_launch", "layout_two_launches"])
def test_multi_kernel_dispatch_graph_replays(T):
    """The multi-kernel dispatch (8800 pairs: layout in one launch; 16800:
    in two) and the combine captured once in a HIP graph and replayed with
    eager work between replays that overwrites the workspace, the layout, the
    receive rows and the output: every replay equals the eager result, whose
    layout equals the oracle's."""
    H, E, k, N, C = 256, 64, 8, 8, 0
    print(f"[case] multi-kernel dispatch graph T={T} H={H} E={E} k={k} N={N}", flush=True)
    shape = api.Shape(T, H, E, k, N, C, api.MOE_PAYLOAD_BF16)
    inp = inputs.generate(T, H, E, 950)
    ids_np = inputs.random_ids(T, k, E, 951, distinct=True)
    x = dev_u16(inp.x_bits)
    ids = torch.from_numpy(ids_np).cuda()
    wt = torch.from_numpy(inputs.random_weights(T, k, 952)).cuda()
    lay = api.Layout.empty(shape, "cuda")
    recv, _ = api.alloc_recv(shape, "cuda", fill=0)
    ws = api.alloc_workspace(shape, "cuda")
    assert ws is not None
    out = torch.empty(T, H, dtype=torch.int16, device="cuda")

    def step(stream=None):
        api.moe_dispatch(shape, x, ids, recv, None, lay, ws, stream=stream)
        api.moe_combine(shape, recv, None, lay, wt, out, stream=stream)

    step()
    torch.cuda.synchronize()
    ref_out, ref_tr, ref_recv = out.clone(), lay.token_row.clone(), recv.clone()
    o = oracle.layout(ids_np, E, N, C)
    assert np.array_equal(ref_tr.cpu().numpy().reshape(o["token_row"].shape), o["token_row"])
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(stream=s)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        step(stream=s)
    for i in range(4):
        out.fill_(0)
        recv.fill_(-1)
        lay.token_row.fill_(-7)
        lay.expert_offsets.fill_(-7)
        ws.fill_((0x00, 0xFF, 0x7F, 0x80)[i])
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(lay.token_row, ref_tr), f"replay {i}: layout"
        assert torch.equal(recv, ref_recv), f"replay {i}: receive rows"
        assert torch.equal(out, ref_out), f"replay {i}: combine"
