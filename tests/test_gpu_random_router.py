"""GPU parity of both routers on seeded random shapes: E up to 1024, k up to
min(32, E), T up to 3000 (one- and four-token blocks), with or without a
bias, sigmoid or softmax scores, N(0,1) logits or small integers (many exact
ties), and for the group-limited router any group count dividing E with the
kept groups holding at least k experts.  Bars: ids bit-exact, weights within
2^-20 relative of the oracle."""
import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import api

pytestmark = pytest.mark.gpu

WEIGHT_RTOL = 2.0 ** -20
MAX_GROUPS = 64


def draw(seed):
    rng = np.random.default_rng(70_000 + seed)
    E = int(rng.choice([int(rng.integers(1, 65)), int(rng.integers(65, 1025))]))
    k = int(rng.integers(1, min(32, E) + 1))
    T = int(rng.choice([int(rng.integers(0, 80)), int(rng.integers(80, 3001))]))
    ties = bool(rng.random() < 0.4)
    use_bias = bool(rng.random() < 0.5)
    score = int(rng.integers(0, 2))
    groups = [g for g in range(2, min(E, MAX_GROUPS) + 1) if E % g == 0]
    G = TG = 0
    if groups and rng.random() < 0.5:
        G = int(rng.choice(groups))
        fits = [tg for tg in range(1, G) if tg * (E // G) >= k]
        if fits:
            TG = int(rng.choice(fits))
        else:
            G = 0
    return E, k, T, ties, use_bias, score, G, TG


CASES = [draw(s) for s in range(40)]


@pytest.mark.parametrize("seed", range(len(CASES)))
def test_random_router(seed):
    E, k, T, ties, use_bias, score, G, TG = CASES[seed]
    print(f"[case] random router seed={seed} E={E} k={k} T={T} ties={ties} bias={use_bias} "
          f"score={score} groups={G}/{TG}", flush=True)
    rng = np.random.default_rng(80_000 + seed)
    if ties:
        lg = rng.integers(-3, 4, size=(T, E)).astype(np.float32)
        bias = (rng.integers(-2, 3, size=E) * 0.5).astype(np.float32)
    else:
        lg = rng.standard_normal((T, E), dtype=np.float32)
        bias = rng.standard_normal(E, dtype=np.float32)
    b = bias if use_bias else None
    d_lg = torch.from_numpy(lg).cuda()
    d_b = None if b is None else torch.from_numpy(b).cuda()
    if G:
        ids, w = api.moe_route_topk_grouped(d_lg, d_b, k, score, G, TG)
        o_ids, o_w = oracle.route_topk_grouped(lg, b, k, score, G, TG)
    else:
        ids, w = api.moe_route_topk(d_lg, d_b, k, score)
        o_ids, o_w = oracle.route_topk(lg, b, k, score)
    torch.cuda.synchronize()
    got = ids.cpu().numpy()
    assert np.array_equal(got, o_ids), np.argwhere(got != o_ids)[:5]
    np.testing.assert_allclose(w.cpu().numpy(), o_w, rtol=WEIGHT_RTOL, atol=0)
