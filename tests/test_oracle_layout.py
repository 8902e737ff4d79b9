"""Pins for the oracle's layout: counts, offsets and destination rows.

The pages fix the structure (per-expert counts, their cumulative sum, offsets
into contiguous per-peer regions: "Enabling trillion-parameter models on AWS
EFA", sections Send and Receive Buffers and Dispatch and Combine).  Checked
here against a hand-worked example, numpy's bincount/cumsum/stable argsort and
invariants that any correct contiguous layout satisfies.
"""
import json
import os

import numpy as np
import pytest

import oracle
from combine_moe_dispatch_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "layout_hand_worked.json")


def test_layout_hand_worked_example():
    g = json.load(open(GOLDEN))
    ids = np.array(g["ids"], np.int32)
    for case in g["cases"]:
        lay = oracle.layout(ids, g["E"], g["N"], case["C"])
        for key in ("expert_counts", "rank_counts", "rank_offsets", "expert_offsets",
                    "token_row", "row_src"):
            assert lay[key].tolist() == case[key], (case["C"], key)
        assert lay["status"] == case["status"]


def _numpy_layout(ids, E, N, C):
    """Library cross-check: bincount, cumsum and a stable argsort of the
    (expert, token, slot) key."""
    T, k = ids.shape
    L = E // N
    flat = ids.reshape(-1)
    counts = np.bincount(flat, minlength=E)
    rank_counts = counts.reshape(N, L).sum(1)
    if C > 0:
        rank_off = np.arange(N) * C
    else:
        rank_off = np.concatenate([[0], np.cumsum(rank_counts)[:-1]])
    within = counts.reshape(N, L)
    exp_off = (rank_off[:, None] + np.concatenate(
        [np.zeros((N, 1), np.int64), np.cumsum(within, 1)[:, :-1]], 1)).reshape(-1)
    order = np.argsort(flat.astype(np.int64) * (T * k) + np.arange(T * k), kind="stable")
    token_row = np.empty(T * k, np.int64)
    pos_sorted = np.arange(T * k)
    rank_start_sorted = np.concatenate([[0], np.cumsum(rank_counts)[:-1]])
    r_of = flat[order] // L
    pos_in_rank = pos_sorted - rank_start_sorted[r_of]
    rows = rank_off[r_of] + pos_in_rank
    if C > 0:
        rows = np.where(pos_in_rank < C, rows, -1)
    token_row[order] = rows
    return counts, rank_counts, rank_off, exp_off, token_row.reshape(T, k)


@pytest.mark.parametrize("T,k,E,N,C", [
    (16, 2, 8, 2, 32), (128, 8, 256, 32, 1024), (128, 8, 384, 16, 1024),
    (300, 8, 256, 32, 0), (77, 3, 12, 4, 0), (50, 4, 16, 4, 5), (1, 1, 1, 1, 1),
])
def test_layout_matches_numpy(T, k, E, N, C):
    ids = inputs.random_ids(T, k, E, seed=T + E, distinct=True)
    lay = oracle.layout(ids, E, N, C)
    counts, rc, ro, eo, tr = _numpy_layout(ids, E, N, C)
    assert np.array_equal(lay["expert_counts"], counts)
    assert np.array_equal(lay["rank_counts"], rc)
    assert np.array_equal(lay["rank_offsets"], ro)
    assert np.array_equal(lay["expert_offsets"], eo)
    assert np.array_equal(lay["token_row"], tr)
    assert lay["expert_counts"].sum() == T * k
    overflow = C > 0 and (rc > C).any()
    assert lay["status"] == (oracle.ST_CAPACITY if overflow else 0)


def test_layout_invariants_with_duplicates_and_skew():
    T, k, E, N, C = 200, 6, 24, 4, 0
    ids = inputs.random_ids(T, k, E, seed=9, distinct=False, hot=5)
    lay = oracle.layout(ids, E, N, C)
    tr = lay["token_row"].reshape(-1)
    assert (tr >= 0).all()
    assert len(np.unique(tr)) == T * k                       # every row distinct
    flat = ids.reshape(-1)
    eo, ec = lay["expert_offsets"], lay["expert_counts"]
    assert ((tr >= eo[flat]) & (tr < eo[flat] + ec[flat])).all()   # inside its segment
    for e in range(E):                                       # (token, slot) ascending
        p = np.nonzero(flat == e)[0]
        assert np.all(np.diff(tr[p]) == 1)
    rs = lay["row_src"]
    assert np.array_equal(rs[tr], np.arange(T * k))          # row_src inverts token_row


def test_layout_capacity_keeps_first_pairs_of_each_rank():
    T, k, E, N, C = 64, 4, 8, 2, 100   # rank loads ~128 > 100
    ids = inputs.random_ids(T, k, E, seed=10, distinct=True)
    lay = oracle.layout(ids, E, N, C)
    assert lay["status"] == oracle.ST_CAPACITY
    flat = ids.reshape(-1)
    tr = lay["token_row"].reshape(-1)
    L = E // N
    for r in range(N):
        p = np.nonzero(flat // L == r)[0]
        key = flat[p].astype(np.int64) * (T * k) + p
        order = p[np.argsort(key)]
        placed = order[:C]
        dropped = order[C:]
        assert np.array_equal(tr[placed], r * C + np.arange(len(placed)))
        assert (tr[dropped] == -1).all()
    # counts stay true counts
    assert lay["expert_counts"].sum() == T * k


def test_layout_bad_ids_are_skipped():
    ids = np.array([[0, 9], [-1, 3], [2, 2]], np.int32)
    lay = oracle.layout(ids, 4, 2, 0)
    assert lay["status"] == oracle.ST_BAD_ID
    assert lay["token_row"][0, 1] == -1 and lay["token_row"][1, 0] == -1
    assert lay["expert_counts"].tolist() == [1, 0, 2, 1]
    # duplicates within one token are separate pairs, in slot order
    assert lay["token_row"][2].tolist() == [1, 2]


def test_layout_empty_and_invalid():
    lay = oracle.layout(np.zeros((0, 8), np.int32), 256, 32, 0)
    assert lay["expert_counts"].sum() == 0 and lay["status"] == 0
    assert (lay["rank_offsets"] == 0).all()
    with pytest.raises(ValueError):
        oracle.layout(np.zeros((2, 2), np.int32), 10, 4, 0)   # E % N != 0
