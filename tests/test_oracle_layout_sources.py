"""Pins for the oracle's multi-source layout (every rank dispatching at once).

Ranks exchange per-expert counts first, after which each knows where its
writes go and at which offset it receives every rank's tokens ("Enabling
trillion-parameter models on AWS EFA", Send and Receive Buffers).  Checked
against a hand-worked example, numpy per-source bincounts and cumulative sums,
and the invariant that inside each expert segment the sources' blocks are
contiguous and in source order.
"""
import json
import os

import numpy as np

import oracle
from combine_moe_dispatch_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_sources_hand_worked.json")


def test_sources_hand_worked_example():
    g = json.load(open(GOLDEN))
    lay = oracle.layout_sources(np.array(g["ids"], np.int32), g["E"], g["N"], g["C"])
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row",
                "source_counts", "source_offsets"):
        assert lay[key].tolist() == g[key], key
    assert lay["status"] == 0


def test_sources_counts_offsets_and_blocks():
    S, T, k, E, N = 6, 40, 4, 32, 8
    ids = np.stack([inputs.random_ids(T, k, E, seed=s, distinct=(s % 2 == 0), hot=(s if s == 3 else None))
                    for s in range(S)])
    lay = oracle.layout_sources(ids, E, N, 0)
    sc = np.stack([np.bincount(ids[s].ravel(), minlength=E) for s in range(S)])
    assert np.array_equal(lay["source_counts"], sc)
    assert np.array_equal(sc.sum(0), lay["expert_counts"])
    off = lay["expert_offsets"][:, None] + np.concatenate(
        [np.zeros((E, 1), np.int64), np.cumsum(sc.T, axis=1)[:, :-1]], axis=1)
    assert np.array_equal(lay["source_offsets"], off)
    tr = lay["token_row"].reshape(S, T, k)
    for s in range(S):
        for e in range(E):
            rows = np.sort(tr[s][ids[s] == e])
            lo = lay["source_offsets"][e, s]
            assert np.array_equal(rows, np.arange(lo, lo + sc[s, e]))


def test_one_source_is_the_single_source_layout():
    ids = inputs.random_ids(50, 8, 64, seed=5)
    a = oracle.layout_sources(ids[None], 64, 8, 0)
    b = oracle.layout(ids, 64, 8, 0)
    for key in ("expert_counts", "expert_offsets", "rank_counts", "rank_offsets", "token_row"):
        assert np.array_equal(a[key], b[key])
