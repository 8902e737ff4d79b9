"""Pins for the oracle's receive-side shuffle into the grouped GEMM's input.

Once all tokens have arrived they are shuffled from the receive buffers into
the tensor passed to the grouped GEMM ("Enabling trillion-parameter models on
AWS EFA", Dispatch and Combine).  Checked: every placed pair's row lands at
dense[e] + its position in its segment, with dense the numpy cumulative sum of
the placed counts; the inverse restores the regions; with packed regions the
shuffle is the identity on the used rows.
"""
import numpy as np
import pytest

import oracle
from combine_moe_dispatch_amd import inputs


@pytest.mark.parametrize("T,k,E,N,C,fp8", [(64, 4, 16, 4, 100, False), (64, 4, 16, 4, 40, True),
                                            (50, 8, 64, 8, 0, False)])
def test_pack_places_each_pair_and_unpack_inverts(T, k, E, N, C, fp8):
    H = 256
    inp = inputs.generate(T, H, E, seed=T + C)
    ids = inputs.random_ids(T, k, E, seed=3, hot=1 if C == 40 else None)
    lay = oracle.layout(ids, E, N, C)
    if fp8:
        recv, rs = oracle.dispatch_fp8(inp.x_bits, lay["token_row"], lay["rows"])
        fill = 0x7F
    else:
        recv, rs = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"]), None
        fill = 0xFFFF
    dense, ds, off = oracle.gemm_io(True, recv, rs, lay["expert_counts"], lay["expert_offsets"],
                                    E, N, C, T * k, fill)
    tr = lay["token_row"]
    placed = tr >= 0
    # dense offsets: cumulative sum of the placed pairs per expert
    pc = np.bincount(ids[placed], minlength=E)
    assert np.array_equal(off, np.concatenate([[0], np.cumsum(pc)]))
    for t in range(T):
        for j in range(k):
            if tr[t, j] < 0:
                continue
            e = ids[t, j]
            d = off[e] + (tr[t, j] - lay["expert_offsets"][e])
            assert np.array_equal(dense[d], recv[tr[t, j]])
            if fp8:
                assert np.array_equal(ds[d], rs[tr[t, j]])
    assert (dense[off[E]:] == fill).all()
    back, bs, off2 = oracle.gemm_io(False, dense, ds, lay["expert_counts"], lay["expert_offsets"],
                                    E, N, C, lay["rows"], fill)
    assert np.array_equal(off, off2)
    assert np.array_equal(back, recv)  # unplaced rows hold the same poison in both
    if fp8:
        assert np.array_equal(back.view(np.uint8)[tr[placed]], recv[tr[placed]])


def test_packed_regions_shuffle_is_identity_on_used_rows():
    T, k, E, N = 40, 4, 32, 8
    inp = inputs.generate(T, 64, E, seed=9)
    ids = inputs.random_ids(T, k, E, seed=10)
    lay = oracle.layout(ids, E, N, 0)
    recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    dense, _, off = oracle.gemm_io(True, recv, None, lay["expert_counts"], lay["expert_offsets"],
                                   E, N, 0, T * k, 0xFFFF)
    assert off[E] == T * k
    assert np.array_equal(dense, recv)
