"""Pins for the oracle's group-limited router.

The router that picks experts per group generalises the plain top-k: plain
routing is the case where the kept group set is all experts ("Lower Latency
and Higher Throughput with Multi-Node DeepSeek Deployment", MoE Router).
Checked against that reduction (one group; all groups kept), against numpy
sorts of the group scores and of the kept experts' logits, and against brute
force over all group subsets on small cases.
"""
import itertools

import numpy as np
import pytest

import oracle
from combine_moe_dispatch_amd import inputs


def test_one_group_is_plain_topk():
    inp = inputs.generate(64, 8, 256, seed=31, zipf=1.2)
    a = oracle.route_topk_grouped(inp.logits, inp.bias, 8, oracle.SCORE_SIGMOID, 1, 1)
    b = oracle.route_topk(inp.logits, inp.bias, 8, oracle.SCORE_SIGMOID)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_all_groups_kept_is_plain_topk():
    inp = inputs.generate(64, 8, 256, seed=32)
    a = oracle.route_topk_grouped(inp.logits, None, 8, oracle.SCORE_SOFTMAX, 8, 8)
    b = oracle.route_topk(inp.logits, None, 8, oracle.SCORE_SOFTMAX)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def _group_scores(lp, G):
    E = lp.shape[1]
    g = lp.reshape(lp.shape[0], G, E // G)
    top2 = -np.sort(-g, axis=2)[:, :, :2] if E // G > 1 else g[:, :, :1]
    return top2.sum(axis=2, dtype=np.float32).astype(np.float32)


@pytest.mark.parametrize("E,G,TG,k", [(256, 8, 4, 8), (64, 8, 3, 6), (384, 8, 2, 8), (32, 32, 8, 4)])
def test_grouped_matches_numpy_sorts(E, G, TG, k):
    inp = inputs.generate(200, 8, E, seed=E + G)
    ids, w = oracle.route_topk_grouped(inp.logits, None, k, oracle.SCORE_SIGMOID, G, TG)
    lp = inp.logits
    gs = _group_scores(lp, G)
    gsz = E // G
    for t in range(200):
        kept = np.argsort(-gs[t], kind="stable")[:TG]
        allowed = np.zeros(E, bool)
        for g in kept:
            allowed[g * gsz:(g + 1) * gsz] = True
        cand = np.nonzero(allowed)[0]
        order = cand[np.argsort(-lp[t, cand], kind="stable")][:k]
        assert list(ids[t]) == list(order), t
        assert np.all(allowed[ids[t]])
    s = 1.0 / (1.0 + np.exp(-lp[np.arange(200)[:, None], ids].astype(np.float64)))
    np.testing.assert_allclose(w, (s / s.sum(1, keepdims=True)).astype(np.float32), rtol=2.0 ** -23)


def test_grouped_brute_force_with_ties():
    rng = np.random.default_rng(7)
    E, G, TG, k = 12, 4, 2, 3
    logits = rng.integers(-2, 3, size=(60, E)).astype(np.float32)
    ids, _ = oracle.route_topk_grouped(logits, None, k, oracle.SCORE_SIGMOID, G, TG)
    gsz = E // G
    for t in range(60):
        l = logits[t]
        score = [float(sorted(l[g * gsz:(g + 1) * gsz])[-1] + sorted(l[g * gsz:(g + 1) * gsz])[-2])
                 for g in range(G)]
        gkey = lambda g: (score[g], -g)
        wins = [S for S in itertools.combinations(range(G), TG)
                if all(gkey(a) > gkey(b) for a in S for b in range(G) if b not in S)]
        assert len(wins) == 1
        cand = [e for e in range(E) if e // gsz in wins[0]]
        ekey = lambda e: (float(l[e]), -e)
        best = sorted(cand, key=ekey, reverse=True)[:k]
        assert list(ids[t]) == best


def test_grouped_rejects_bad_arguments():
    z = np.zeros((2, 16), np.float32)
    for args in ((3, 2), (4, 5), (4, 0)):
        with pytest.raises(ValueError):
            oracle.route_topk_grouped(z, None, 2, oracle.SCORE_SIGMOID, *args)
    with pytest.raises(ValueError):   # k larger than the kept experts
        oracle.route_topk_grouped(z, None, 9, oracle.SCORE_SIGMOID, 4, 2)
