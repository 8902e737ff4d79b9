"""Pins for the oracle's dispatch, expert stand-in and combine.

Dispatch copies (or block-quantises) each token to every destination row of
its pairs; combine forms the router-weighted sum of the returned rows on the
receiving side ("Enabling trillion-parameter models on AWS EFA", Introduction,
Send and Receive Buffers, Evaluation; "Lower Latency and Higher Throughput
with Multi-Node DeepSeek Deployment", Quantization).  Pins: bitwise equality
of copied rows, permutation of the replicated rows, torch's fp8/bf16 casts for
the quantiser, exact rational arithmetic for the fp32 fused multiply-add
chain, numpy float64 sums, and closed-form special cases (k = 1, identity
experts with normalised weights).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from combine_moe_dispatch_amd import inputs


def _case(T, H, E, k, N, C, seed, expert="scale"):
    inp = inputs.generate(T, H, E, seed, expert=expert)
    ids, w = oracle.route_topk(inp.logits, None, k, oracle.SCORE_SIGMOID)
    lay = oracle.layout(ids, E, N, C)
    return inp, ids, w, lay


def test_dispatch_bf16_rows_are_copies_and_a_permutation():
    inp, ids, w, lay = _case(40, 64, 16, 4, 4, 0, seed=1)
    recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    tr = lay["token_row"]
    for t in range(40):
        for j in range(4):
            assert np.array_equal(recv[tr[t, j]], inp.x_bits[t])
    rep = np.repeat(inp.x_bits, 4, axis=0)
    a = np.sort(recv.view(np.dtype((np.void, 128))).ravel())
    b = np.sort(rep.view(np.dtype((np.void, 128))).ravel())
    assert np.array_equal(a, b)


def test_dispatch_leaves_unplaced_rows_untouched():
    inp, ids, w, lay = _case(8, 16, 8, 2, 2, 16, seed=2)
    recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"], fill=0xABCD)
    placed = np.zeros(lay["rows"], bool)
    placed[lay["token_row"].reshape(-1)] = True
    assert (recv[~placed] == 0xABCD).all()


def test_quantize_fp8_matches_numpy_and_torch():
    inp = inputs.generate(6, 512, 4, seed=3)
    x = inp.x_bits.copy()
    x[2, 128:256] = 0          # an all-zero block
    x[3, :128] = 0x8000        # an all-negative-zero block
    x[4, 10] = 0x8000          # signed zeros beside non-zero entries: -0 / s = -0 (code
    x[4, 11] = 0               # 0x80), +0 / s = +0 (code 0x00)
    for t in range(6):
        q, s = oracle.quantize_row_fp8(x[t])
        xf = (x[t].astype(np.uint32) << 16).view(np.float32).reshape(-1, 128)
        amax = np.abs(xf).max(1)
        s_ref = (amax / np.float32(448.0)).astype(np.float32)   # fp32 IEEE division
        assert np.array_equal(s.view(np.uint32), s_ref.view(np.uint32))
        for b in range(xf.shape[0]):
            if amax[b] == 0:
                assert (q[b * 128:(b + 1) * 128] == 0).all()
                continue
            ratio = (xf[b] / s_ref[b]).astype(np.float32)        # fp32 IEEE division
            assert np.abs(ratio).max() < 464.0
            ref = torch.from_numpy(ratio).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[b * 128:(b + 1) * 128], ref)
    # the largest magnitude of each block maps to 448 (code 0x7E / 0xFE)
    q, s = oracle.quantize_row_fp8(inp.x_bits[0])
    xf = (inp.x_bits[0].astype(np.uint32) << 16).view(np.float32).reshape(-1, 128)
    for b in range(4):
        i = int(np.argmax(np.abs(xf[b])))
        assert q[b * 128 + i] & 0x7F == 0x7E


def test_fp8_roundtrip_error_bound():
    inp = inputs.generate(4, 1024, 4, seed=4)
    for t in range(4):
        q, s = oracle.quantize_row_fp8(inp.x_bits[t])
        xf = (inp.x_bits[t].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        deq = torch.from_numpy(q).view(torch.float8_e4m3fn).double().numpy() * np.repeat(s, 128)
        # half an e4m3 ulp: 2^-4 relative for normals, 2^-10 * s absolute for subnormals
        bound = np.maximum(np.abs(xf) * 2.0 ** -4, np.repeat(s, 128) * 2.0 ** -10) * (1 + 1e-6)
        assert (np.abs(deq - xf) <= bound).all()


def test_dispatch_fp8_copies_payload_and_scales():
    inp, ids, w, lay = _case(10, 256, 8, 3, 2, 0, seed=5)
    recv, sc = oracle.dispatch_fp8(inp.x_bits, lay["token_row"], lay["rows"])
    for t in range(10):
        q, s = oracle.quantize_row_fp8(inp.x_bits[t])
        for j in range(3):
            r = lay["token_row"][t, j]
            assert np.array_equal(recv[r], q) and np.array_equal(sc[r], s)


def test_expert_scale_bf16_matches_torch():
    inp, ids, w, lay = _case(12, 64, 8, 2, 2, 0, seed=6)
    recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    y = oracle.expert_scale_bf16(recv, ids, lay["token_row"], inp.alpha)
    for t in range(12):
        for j in range(2):
            r = lay["token_row"][t, j]
            xf = torch.from_numpy(inp.x_bits[t].view(np.int16).copy()).view(torch.bfloat16).float()
            ref = (xf * torch.tensor(inp.alpha[ids[t, j]])).to(torch.bfloat16)
            assert np.array_equal(y[r], ref.view(torch.int16).numpy().view(np.uint16))


def test_expert_scale_fp8_scales_only():
    inp, ids, w, lay = _case(12, 256, 8, 2, 2, 0, seed=7)
    recv, sc = oracle.dispatch_fp8(inp.x_bits, lay["token_row"], lay["rows"])
    y, ys = oracle.expert_scale_fp8(recv, sc, ids, lay["token_row"], inp.alpha)
    assert np.array_equal(y, recv)
    tr, flat = lay["token_row"].reshape(-1), ids.reshape(-1)
    ref = (sc[tr] * inp.alpha[flat][:, None]).astype(np.float32)
    assert np.array_equal(ys[tr].view(np.uint32), ref.view(np.uint32))


def _bf16_to_f64(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _ulp_dist(a, b):
    """Distance between bf16 bit patterns on the ordered number line (+0 == -0)."""
    def key(u):
        u = np.asarray(u, np.int64)
        return np.where(u & 0x8000, -(u & 0x7FFF), u)
    return np.abs(key(a) - key(b))


def test_combine_k1_unit_weight_is_identity():
    inp, ids, w, lay = _case(20, 64, 8, 1, 2, 0, seed=8)
    y = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    ones = np.ones_like(w)
    for fn in (oracle.combine_exact, oracle.combine_f32_ordered):
        out = fn(y, None, lay["token_row"], ones)
        assert np.array_equal(out, inp.x_bits)


@pytest.mark.parametrize("k,E,N", [(2, 8, 2), (8, 256, 32), (8, 384, 16)])
def test_identity_experts_with_normalised_weights_return_the_input(k, E, N):
    inp, ids, w, lay = _case(24, 128, E, k, N, 0, seed=9, expert="identity")
    y = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    for fn in (oracle.combine_exact, oracle.combine_f32_ordered):
        out = fn(y, None, lay["token_row"], w)
        assert np.array_equal(out, inp.x_bits)


def test_combine_exact_matches_numpy_float64():
    inp, ids, w, lay = _case(32, 256, 16, 4, 4, 0, seed=10)
    rng = np.random.default_rng(0)
    # arbitrary returned rows (mixed signs) to exercise cancellation
    y = inputs.bf16_bits_from_f32(rng.standard_normal((lay["rows"], 256)).astype(np.float32))
    out = oracle.combine_exact(y, None, lay["token_row"], w)
    yv = _bf16_to_f64(y)[lay["token_row"]]               # [T,k,H]
    ref = (w.astype(np.float64)[:, :, None] * yv).sum(1)
    ref_bits = np.array([oracle.f64_to_bf16(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    d = _ulp_dist(out, ref_bits)
    assert d.max() <= 1 and (d == 0).mean() > 0.999


def test_combine_scalar_experts_closed_form():
    inp, ids, w, lay = _case(16, 64, 8, 3, 2, 0, seed=11)
    recv = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    y = oracle.expert_scale_bf16(recv, ids, lay["token_row"], inp.alpha)
    out = oracle.combine_exact(y, None, lay["token_row"], w)
    # y = bf16(alpha*x) carries a relative error of at most 2^-9 per row, so the
    # result is x * sum_j w_j alpha_j within 2^-9 relative before rounding
    scale = (w.astype(np.float64) * inp.alpha[ids].astype(np.float64)).sum(1)
    ref = _bf16_to_f64(inp.x_bits) * scale[:, None]
    got = _bf16_to_f64(out)
    assert np.all(np.abs(got - ref) <= np.abs(ref) * (2.0 ** -9 + 2.0 ** -8) + 1e-30)


def _round_f32(q: Fraction) -> Fraction:
    """Round a rational to the nearest fp32 value, ties to even (normal range)."""
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


def test_combine_f32_ordered_is_a_chain_of_fused_multiply_adds():
    inp, ids, w, lay = _case(4, 16, 16, 8, 4, 0, seed=12)
    rng = np.random.default_rng(1)
    y = inputs.bf16_bits_from_f32(rng.standard_normal((lay["rows"], 16)).astype(np.float32))
    out = oracle.combine_f32_ordered(y, None, lay["token_row"], w)
    yv = _bf16_to_f64(y)
    for t in range(4):
        for i in range(16):
            acc = Fraction(0)
            for j in range(8):
                acc = _round_f32(Fraction(float(w[t, j])) * Fraction(float(yv[lay["token_row"][t, j], i])) + acc)
            ref = oracle.f64_to_bf16(float(acc))   # acc is an fp32 value: exact in double
            assert out[t, i] == ref


def _cancelling_terms(T, k, H, fp8, seed):
    """Rows whose slot pairs nearly cancel (opposite signs, weights and scales
    a few fp32 ulps apart), so each fp32 rounding in the chain reaches the
    bf16 result; token_row = t * k + j."""
    rng = np.random.default_rng(seed)
    rows = T * k
    w = rng.uniform(0.1, 0.2, size=(T, k)).astype(np.float32)
    w[:, 1::2] = (w[:, 0::2].astype(np.float64)
                  * (1 + rng.integers(-64, 64, size=(T, k // 2)) * 2.0 ** -23)).astype(np.float32)
    tr = np.arange(rows, dtype=np.int32).reshape(T, k)
    if fp8:
        mag = rng.integers(0x38, 0x7E, size=(T, k // 2, H)).astype(np.uint8)  # 1.0 .. 448
        codes = np.empty((T, k, H), np.uint8)
        codes[:, 0::2] = mag
        codes[:, 1::2] = mag | 0x80
        ys = (np.float32(0.0123) * (1 + rng.integers(0, 1 << 12, size=(rows, H // 128))
                                    * 2.0 ** -23)).astype(np.float32)
        return codes.reshape(rows, H), ys, tr, w
    v = rng.standard_normal((T, k // 2, H)).astype(np.float32)
    y = np.empty((T, k, H), np.float32)
    y[:, 0::2] = v
    y[:, 1::2] = -v
    return inputs.bf16_bits_from_f32(y.reshape(rows, H)), None, tr, w


def test_combine_f32_ordered_fp8_is_one_rounded_product_then_fused_adds():
    """fp8 payload: each term's value is fp32(code) * scale rounded once to
    fp32, then folded by a fused multiply-add in slot order from 0.  Codes are
    decoded by torch's e4m3fn cast (not the oracle's decoder) and every step
    is exact rational arithmetic with one explicit rounding.  On rows whose
    terms nearly cancel, the chains with the weight folded into the scale or
    with the product left unrounded give different bf16 results, and the test
    asserts that they do, so it tells those mistakes apart."""
    T, k, H = 4, 8, 256
    y, ys, tr, w = _cancelling_terms(T, k, H, fp8=True, seed=3)
    out = oracle.combine_f32_ordered(y, ys, tr, w)
    dec = torch.from_numpy(y).view(torch.float8_e4m3fn).double().numpy()
    folded = unrounded = 0
    for t in range(T):
        for i in range(H):
            acc = a_fold = a_unr = Fraction(0)
            for j in range(k):
                r = tr[t, j]
                c, s = Fraction(float(dec[r, i])), Fraction(float(ys[r, i // 128]))
                wj = Fraction(float(w[t, j]))
                acc = _round_f32(wj * _round_f32(c * s) + acc)
                a_fold = _round_f32(_round_f32(wj * s) * c + a_fold)
                a_unr = _round_f32(wj * c * s + a_unr)
            assert out[t, i] == oracle.f64_to_bf16(float(acc)), (t, i)
            folded += out[t, i] != oracle.f64_to_bf16(float(a_fold))
            unrounded += out[t, i] != oracle.f64_to_bf16(float(a_unr))
    assert folded > 0 and unrounded > 0


def test_combine_f32_ordered_bf16_fused_on_cancelling_rows():
    """bf16 payload on rows whose slot pairs nearly cancel: the result is the
    chain of fused multiply-adds (one rounding per step), and a chain of
    separately rounded products and sums gives a different bf16 result."""
    T, k, H = 4, 8, 256
    y, _, tr, w = _cancelling_terms(T, k, H, fp8=False, seed=4)
    out = oracle.combine_f32_ordered(y, None, tr, w)
    yv = _bf16_to_f64(y)
    unfused = 0
    for t in range(T):
        for i in range(H):
            acc = a_unf = Fraction(0)
            for j in range(k):
                v, wj = Fraction(float(yv[tr[t, j], i])), Fraction(float(w[t, j]))
                acc = _round_f32(wj * v + acc)
                a_unf = _round_f32(_round_f32(wj * v) + a_unf)
            assert out[t, i] == oracle.f64_to_bf16(float(acc)), (t, i)
            unfused += out[t, i] != oracle.f64_to_bf16(float(a_unf))
    assert unfused > 0


def test_combine_skipped_pairs_add_nothing():
    inp, ids, w, lay = _case(16, 32, 8, 4, 2, 0, seed=13)
    y = oracle.dispatch_bf16(inp.x_bits, lay["token_row"], lay["rows"])
    tr = lay["token_row"].copy()
    tr[::3, 1] = -1
    w0 = w.copy()
    w0[::3, 1] = 0.0
    for fn in (oracle.combine_exact, oracle.combine_f32_ordered):
        a = fn(y, None, tr, w)
        b = fn(y, None, lay["token_row"], w0)
        assert np.array_equal(a, b)
    allskip = np.full_like(tr, -1)
    assert (oracle.combine_exact(y, None, allskip, w) == 0).all()


def test_combine_fp8_matches_numpy_float64():
    inp, ids, w, lay = _case(12, 256, 8, 4, 2, 0, seed=14)
    recv, sc = oracle.dispatch_fp8(inp.x_bits, lay["token_row"], lay["rows"])
    y, ys = oracle.expert_scale_fp8(recv, sc, ids, lay["token_row"], inp.alpha)
    out = oracle.combine_exact(y, ys, lay["token_row"], w)
    tr = lay["token_row"]
    deq = torch.from_numpy(y).view(torch.float8_e4m3fn).double().numpy() * np.repeat(ys, 128, axis=1)
    ref = (w.astype(np.float64)[:, :, None] * deq[tr]).sum(1)
    ref_bits = np.array([oracle.f64_to_bf16(v) for v in ref.ravel()], np.uint16).reshape(ref.shape)
    d = _ulp_dist(out, ref_bits)
    assert d.max() <= 1 and (d == 0).mean() > 0.999
    out32 = oracle.combine_f32_ordered(y, ys, tr, w)
    assert _ulp_dist(out32, out).max() <= 1
