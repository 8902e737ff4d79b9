"""GPU parity of the router at the library's advertised limits.

The header allows k up to 32 and E up to 1024.  These cases run the plain
router on every per-lane width the kernel is built for (1, 2, 4, 6, 8 and 16
logits per lane: E in 1..64, 65..128, 129..256, 257..384, 385..512 and
513..1024), with k past 8 (the top-k rounds beyond one DPP row of slots) and
past 16 (the weight sum over the second row of slot lanes), and the
group-limited router with k past 8, on both block layouts (one token per
block up to 2048 tokens, four past that).  Inputs: N(0,1) logits with an N(0,1)
bias, and integer logits with a half-integer bias (many exact ties, which the
selection breaks toward the lower expert id).  Bars as elsewhere: ids
bit-exact, weights within 2^-20 relative of the oracle's double-precision
weights rounded once to fp32.
"""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api

pytestmark = pytest.mark.gpu

WEIGHT_RTOL = 2.0 ** -20


def _logits(T, E, ties, seed):
    rng = np.random.default_rng(seed)
    if ties:
        lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
        bias = (rng.integers(-2, 3, size=E) * 0.5).astype(np.float32)
    else:
        lg = rng.standard_normal((T, E), dtype=np.float32)
        bias = rng.standard_normal(E, dtype=np.float32)
    return lg, bias


def _check(ids, w, o_ids, o_w):
    got_ids = ids.cpu().numpy()
    assert np.array_equal(got_ids, o_ids), np.argwhere(got_ids != o_ids)[:5]
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=WEIGHT_RTOL, atol=0)


# (E, k, T): per-lane width ceil(E / 64) in {1, 2, 4, 6, 8, 16}
PLAIN = [
    (32, 32, 77),      # k == E: every expert, in descending order
    (33, 17, 65),      # one logit per lane, lane 32 the only one past 31
    (64, 32, 70),
    (65, 9, 77),       # two per lane, lane 0 alone holds a second logit
    (96, 9, 130),
    (96, 17, 77),
    (128, 16, 77),
    (128, 32, 129),
    (256, 32, 40),
    (384, 16, 50),
    (385, 17, 66),     # eight per lane, mostly empty
    (512, 9, 77),
    (512, 17, 64),
    (512, 32, 33),
    (513, 16, 50),     # sixteen per lane
    (1000, 32, 45),
    (1024, 16, 77),
    (1024, 32, 130),
    # past 2048 tokens: four tokens per block instead of one
    (256, 8, 2500),
    (384, 17, 2049),
    (1024, 32, 2051),
]


@pytest.mark.parametrize("E,k,T", PLAIN, ids=lambda v: str(v))
@pytest.mark.parametrize("ties", [False, True], ids=["normal", "ties"])
def test_plain_router_at_limits(E, k, T, ties):
    print(f"[case] plain router E={E} k={k} T={T} ties={ties}", flush=True)
    lg, bias = _logits(T, E, ties, seed=1000 + E + 7 * k)
    d_lg = torch.from_numpy(lg).cuda()
    for use_bias in (False, True):
        b = bias if use_bias else None
        d_b = None if b is None else torch.from_numpy(b).cuda()
        for score in (api.MOE_SCORE_SIGMOID, api.MOE_SCORE_SOFTMAX):
            ids, w = api.moe_route_topk(d_lg, d_b, k, score)
            torch.cuda.synchronize()
            o_ids, o_w = oracle.route_topk(lg, b, k, score)
            _check(ids, w, o_ids, o_w)


# (E, groups, kept, k, T)
GROUPED = [
    (256, 8, 4, 16, 77),     # 8 lanes per group
    (256, 8, 4, 32, 50),     # k == the kept groups' experts
    (512, 8, 3, 17, 64),
    (1024, 16, 8, 32, 45),   # 4 lanes per group, 16 logits per lane
    (384, 8, 2, 9, 70),      # 6 logits per lane
    (160, 8, 3, 24, 60),     # groups off whole lanes (LDS path)
    (96, 3, 2, 17, 66),
    (256, 8, 4, 8, 2500),    # four tokens per block
    (160, 8, 3, 9, 2049),    # four tokens per block, LDS path
]


@pytest.mark.parametrize("E,G,TG,k,T", GROUPED, ids=lambda v: str(v))
@pytest.mark.parametrize("ties", [False, True], ids=["normal", "ties"])
def test_grouped_router_large_k(E, G, TG, k, T, ties):
    print(f"[case] grouped router E={E} G={G} TG={TG} k={k} T={T} ties={ties}", flush=True)
    lg, bias = _logits(T, E, ties, seed=2000 + E + 3 * k)
    d_lg = torch.from_numpy(lg).cuda()
    d_b = torch.from_numpy(bias).cuda()
    for score in (api.MOE_SCORE_SIGMOID, api.MOE_SCORE_SOFTMAX):
        ids, w = api.moe_route_topk_grouped(d_lg, d_b, k, score, G, TG)
        torch.cuda.synchronize()
        o_ids, o_w = oracle.route_topk_grouped(lg, bias, k, score, G, TG)
        _check(ids, w, o_ids, o_w)


@pytest.mark.parametrize("E,k,T", [(64, 8, 40), (256, 32, 70), (1024, 16, 2100)],
                         ids=lambda v: str(v))
def test_router_all_values_equal(E, k, T):
    """Every logit equal: every round's largest value is shared by every
    lane's head, so every slot is decided by the lowest id -- experts 0..k-1
    in order, weights all 1/k -- on the one- and four-token block layouts."""
    print(f"[case] router all equal E={E} k={k} T={T}", flush=True)
    lg = np.full((T, E), 0.25, np.float32)
    d_lg = torch.from_numpy(lg).cuda()
    for score in (api.MOE_SCORE_SIGMOID, api.MOE_SCORE_SOFTMAX):
        ids, w = api.moe_route_topk(d_lg, None, k, score)
        torch.cuda.synchronize()
        o_ids, o_w = oracle.route_topk(lg, None, k, score)
        assert np.array_equal(o_ids, np.tile(np.arange(k, dtype=np.int32), (T, 1)))
        _check(ids, w, o_ids, o_w)


def test_binding_refuses_bad_views_and_types():
    """Argument checks of the binding on the GPU: a transposed (non-contiguous)
    logits view, int64 ids and an undersized receive buffer are refused before
    any launch."""
    print("[case] binding argument checks", flush=True)
    T, E, k, H = 16, 64, 4, 256
    lg = torch.randn(E, T, device="cuda").t()          # a [T, E] view, not contiguous
    with pytest.raises(ValueError, match="contiguous"):
        api.moe_route_topk(lg, None, k, api.MOE_SCORE_SIGMOID)
    shape = api.Shape(T, H, E, k, 8, 0)
    x = torch.zeros(T, H, dtype=torch.int16, device="cuda")
    ids64 = torch.zeros(T, k, dtype=torch.int64, device="cuda")
    lay = api.Layout.empty(shape, "cuda")
    recv, _ = api.alloc_recv(shape, "cuda")
    with pytest.raises(TypeError, match="topk_ids must be torch.int32"):
        api.moe_dispatch(shape, x, ids64, recv, None, lay)
    ids = torch.zeros(T, k, dtype=torch.int32, device="cuda")
    with pytest.raises(ValueError, match="recv_x holds"):
        api.moe_dispatch(shape, x, ids, recv[:-1], None, lay)
