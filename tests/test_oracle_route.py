"""Pins for the oracle's top-k router.

The router picks each token's k experts by biased logit, ties to the lower
expert id, slots in descending order, and weights that sum to one ("Enabling
trillion-parameter models on AWS EFA", Introduction; "Lower Latency and
Higher Throughput with Multi-Node DeepSeek Deployment", MoE Router).  Checked
against brute force over all k-subsets, numpy's stable argsort and float64
closed forms from torch.
"""
import itertools

import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import inputs


def _brute_topk(lp, k):
    """The unique k-subset S with key(i) > key(o) for i in S, o not in S, where
    key = (value, -index); slots sorted by key descending."""
    E = len(lp)
    key = lambda i: (float(lp[i]), -i)
    winners = []
    for S in itertools.combinations(range(E), k):
        rest = [o for o in range(E) if o not in S]
        if all(key(i) > key(o) for i in S for o in rest):
            winners.append(S)
    assert len(winners) == 1
    return sorted(winners[0], key=key, reverse=True)


@pytest.mark.parametrize("E,k", [(4, 1), (6, 2), (8, 3), (8, 8)])
def test_route_ids_brute_force_with_ties(E, k):
    rng = np.random.default_rng(E * 10 + k)
    # integer-valued logits produce many ties
    logits = rng.integers(-2, 3, size=(40, E)).astype(np.float32)
    ids, _ = oracle.route_topk(logits, None, k, oracle.SCORE_SIGMOID)
    for t in range(40):
        assert list(ids[t]) == _brute_topk(logits[t], k)


def test_route_ids_match_stable_argsort():
    inp = inputs.generate(64, 8, 256, seed=3)
    ids, _ = oracle.route_topk(inp.logits, None, 8, oracle.SCORE_SIGMOID)
    ref = np.argsort(-inp.logits, axis=1, kind="stable")[:, :8]
    assert np.array_equal(ids, ref)


def test_route_bias_is_added_before_selection():
    inp = inputs.generate(32, 8, 64, seed=4, zipf=1.2)
    ids_b, w_b = oracle.route_topk(inp.logits, inp.bias, 4, oracle.SCORE_SIGMOID)
    biased = (inp.logits + inp.bias[None, :]).astype(np.float32)  # fp32 add
    ids_r, w_r = oracle.route_topk(biased, None, 4, oracle.SCORE_SIGMOID)
    assert np.array_equal(ids_b, ids_r)
    assert np.array_equal(w_b, w_r)


def test_sigmoid_weights_closed_form():
    inp = inputs.generate(64, 8, 256, seed=5)
    ids, w = oracle.route_topk(inp.logits, None, 8, oracle.SCORE_SIGMOID)
    lt = torch.from_numpy(inp.logits).double()
    sel = torch.gather(lt, 1, torch.from_numpy(ids).long())
    s = torch.sigmoid(sel)
    ref = (s / s.sum(1, keepdim=True)).float().numpy()
    np.testing.assert_allclose(w, ref, rtol=2.0 ** -23, atol=0)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 8 * 2.0 ** -24)
    assert np.all(w > 0)


def test_softmax_weights_are_full_softmax_renormalised_over_topk():
    inp = inputs.generate(64, 8, 8, seed=6)
    ids, w = oracle.route_topk(inp.logits, None, 2, oracle.SCORE_SOFTMAX)
    p = torch.softmax(torch.from_numpy(inp.logits).double(), dim=1)
    sel = torch.gather(p, 1, torch.from_numpy(ids).long())
    ref = (sel / sel.sum(1, keepdim=True)).float().numpy()
    np.testing.assert_allclose(w, ref, rtol=2.0 ** -22, atol=0)
    # slot 0 holds the largest weight
    assert np.all(w[:, 0] >= w[:, 1])


def test_route_rejects_bad_arguments():
    with pytest.raises(ValueError):
        oracle.route_topk(np.zeros((2, 4), np.float32), None, 5, oracle.SCORE_SIGMOID)
    bad = np.zeros((2, 4), np.float32)
    bad[1, 2] = np.nan
    with pytest.raises(ValueError):
        oracle.route_topk(bad, None, 2, oracle.SCORE_SIGMOID)


def test_route_distinct_ids_and_k_equals_e():
    inp = inputs.generate(16, 8, 8, seed=8)
    ids, w = oracle.route_topk(inp.logits, None, 8, oracle.SCORE_SOFTMAX)
    for t in range(16):
        assert sorted(ids[t]) == list(range(8))
    np.testing.assert_allclose(w.astype(np.float64).sum(1), 1.0, atol=8 * 2.0 ** -24)
