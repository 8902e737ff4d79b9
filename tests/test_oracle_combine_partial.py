"""Pins for the oracle's sender-side partial reduction (two-stage combine).

The alternative to receiver-only accumulation: each destination rank first
sums a token's rows for its own experts, sending less data, with possible
precision implications ("Enabling trillion-parameter models on AWS EFA",
Evaluation).  Checked against: the one-rank special case (stage 1 is the whole
combine, stage 2 the identity); numpy float64 group sums and numpy's unique
for the rank slots; exact rational emulation of the fp32 chains; and the error
bound against the single-stage combine.
"""
from fractions import Fraction

import numpy as np
import pytest

import oracle
from combine_moe_dispatch_amd import inputs


def _case(T, H, E, k, N, seed, fp8=False):
    inp = inputs.generate(T, H, E, seed)
    ids, w = oracle.route_topk(inp.logits, None, k, oracle.SCORE_SIGMOID)
    lay = oracle.layout(ids, E, N, 0)
    if fp8:
        recv, sc = oracle.dispatch_fp8(inp.x_bits, lay["token_row"], lay["rows"])
        y, ys = oracle.expert_scale_fp8(recv, sc, ids, lay["token_row"], inp.alpha)
    else:
        recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
        y, ys = oracle.expert_scale_bf16(recv, ids, lay["token_row"], inp.alpha), None
    return ids, w, lay, y, ys


def _bits_f64(b):
    return (np.asarray(b, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ulp(a, b):
    key = lambda u: np.where(np.asarray(u, np.int64) & 0x8000, -(np.asarray(u, np.int64) & 0x7FFF),
                             np.asarray(u, np.int64))
    return np.abs(key(a) - key(b))


@pytest.mark.parametrize("exact", [True, False])
def test_one_rank_is_the_plain_combine(exact):
    ids, w, lay, y, ys = _case(20, 64, 8, 4, 1, seed=1)
    partial, prank = oracle.combine_send(y, ys, lay["token_row"], ids, w, 8, 1, exact)
    assert (prank == 0).all()
    ref = (oracle.combine_exact if exact else oracle.combine_f32_ordered)(y, ys, lay["token_row"], w)
    assert np.array_equal(partial[:, 0], ref)
    assert np.array_equal(oracle.combine_recv(partial, prank, exact), ref)


def test_partial_rows_are_group_sums_over_ranks():
    T, H, E, k, N = 30, 32, 32, 6, 8
    ids, w, lay, y, ys = _case(T, H, E, k, N, seed=2)
    partial, prank = oracle.combine_send(y, ys, lay["token_row"], ids, w, E, N, True)
    L = E // N
    yv = _bits_f64(y)
    for t in range(T):
        ranks = np.unique(ids[t] // L)
        assert list(prank[t, :len(ranks)]) == list(ranks)
        assert (prank[t, len(ranks):] == -1).all()
        assert (partial[t, len(ranks):] == 0xFFFF).all()     # unused slots untouched
        for i, r in enumerate(ranks):
            sel = np.nonzero(ids[t] // L == r)[0]
            ref = (w[t, sel].astype(np.float64)[:, None] * yv[lay["token_row"][t, sel]]).sum(0)
            exp = np.array([oracle.f64_to_bf16(v) for v in ref], np.uint16)
            # numpy sums in another order; the two doubles round to bf16 alike
            # except at an exact tie, so allow one ulp
            assert _ulp(partial[t, i], exp).max() <= 1


def _round_f32(q: Fraction) -> Fraction:
    if q == 0:
        return Fraction(0)
    s = -1 if q < 0 else 1
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (e - 23)
    m = a / ulp
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * ulp


def test_fp32_chains_exactly():
    T, H, E, k, N = 3, 8, 16, 6, 4
    ids, w, lay, y, ys = _case(T, H, E, k, N, seed=3)
    partial, prank = oracle.combine_send(y, ys, lay["token_row"], ids, w, E, N, False)
    out = oracle.combine_recv(partial, prank, False)
    L = E // N
    yv = _bits_f64(y)
    for t in range(T):
        for i, r in enumerate(prank[t]):
            if r < 0:
                continue
            for c in range(H):
                acc = Fraction(0)
                for j in range(k):
                    if ids[t, j] // L == r:
                        acc = _round_f32(Fraction(float(w[t, j])) *
                                         Fraction(float(yv[lay["token_row"][t, j], c])) + acc)
                assert partial[t, i, c] == oracle.f64_to_bf16(float(acc))
        for c in range(H):
            acc = Fraction(0)
            for i in range(prank.shape[1]):
                if prank[t, i] >= 0:
                    acc = _round_f32(acc + Fraction(float(_bits_f64(partial[t, i, c]))))
            assert out[t, c] == oracle.f64_to_bf16(float(acc))


@pytest.mark.parametrize("fp8", [False, True])
def test_two_stage_error_against_single_stage(fp8):
    """Positive weights and same-sign terms: each partial is within half an
    ulp of its exact sum, so the result stays within 2 ulps of the
    single-stage combine (the precision cost the pages mention)."""
    T, H, E, k, N = 64, 256, 256, 8, 32
    ids, w, lay, y, ys = _case(T, H, E, k, N, seed=4, fp8=fp8)
    partial, prank = oracle.combine_send(y, ys, lay["token_row"], ids, w, E, N, True)
    out = oracle.combine_recv(partial, prank, True)
    ref = oracle.combine_exact(y, ys, lay["token_row"], w)
    d = _ulp(out, ref)
    assert d.max() <= 2
