"""Pins for the oracle's number-format codecs (bf16 and OCP e4m3fn).

Each check is independent of the oracle's own code: torch's CPU conversions,
brute-force nearest-value search over every representable value, and the
formats' closed-form decoding.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def _torch_bf16_bits(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_round_to_nearest_even_examples():
    # 1 + 2^-8 is the midpoint between 1.0 and 1 + 2^-7: ties to even -> 1.0
    assert oracle.f32_to_bf16(1.0 + 2.0 ** -8) == 0x3F80
    # 1 + 3*2^-8 is the midpoint between 1+2^-7 (odd) and 1+2^-6 (even)
    assert oracle.f32_to_bf16(1.0 + 3 * 2.0 ** -8) == 0x3F82
    assert oracle.f32_to_bf16(-0.0) == 0x8000
    assert oracle.f32_to_bf16(0.0) == 0x0000
    assert oracle.f32_to_bf16(float("inf")) == 0x7F80
    assert oracle.f32_to_bf16(3.4e38) == 0x7F80  # beyond max + half ulp
    assert math.isnan(oracle.bf16_to_f32(oracle.f32_to_bf16(float("nan"))))


def test_bf16_matches_torch_on_random_fp32():
    rng = np.random.default_rng(7)
    vals = np.concatenate([
        rng.standard_normal(4000).astype(np.float32),
        (rng.standard_normal(2000) * 1e30).astype(np.float32),
        (rng.standard_normal(2000) * 1e-39).astype(np.float32),  # fp32 subnormals
        rng.integers(0, 2 ** 32, 4000, dtype=np.uint64).astype(np.uint32).view(np.float32),
    ])
    vals = vals[np.isfinite(vals)]
    ref = _torch_bf16_bits(vals)
    got = np.array([oracle.f32_to_bf16(float(v)) for v in vals], np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_decode_is_bit_shift():
    for b in [0x0000, 0x3F80, 0xBF80, 0x0001, 0x7F7F, 0xC2F7]:
        assert np.float32(oracle.bf16_to_f32(b)).view(np.uint32) == (b << 16)


def _all_bf16_positive_finite():
    bits = np.arange(0, 0x7F80, dtype=np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def test_f64_to_bf16_is_nearest_with_ties_to_even():
    """Brute force: the nearest of all finite bf16 values, ties to even bits."""
    table = _all_bf16_positive_finite()
    rng = np.random.default_rng(11)
    samples = list(rng.standard_normal(3000) * np.exp(rng.uniform(-30, 30, 3000)))
    # exact midpoints between neighbours, and points just off them
    idx = rng.integers(0, len(table) - 1, 500)
    mids = (table[idx] + table[idx + 1]) / 2
    samples += list(mids) + list(np.nextafter(mids, np.inf)) + list(np.nextafter(mids, -np.inf))
    for v in samples:
        a = abs(v)
        i = np.searchsorted(table, a)
        cands = [c for c in (i - 1, i) if 0 <= c < len(table)]
        d = [abs(table[c] - a) for c in cands]
        best = min(d)
        ties = [c for c, dd in zip(cands, d) if dd == best]
        exp_bits = ties[0] if len(ties) == 1 else [c for c in ties if c % 2 == 0][0]
        if v < 0:
            exp_bits |= 0x8000
        assert oracle.f64_to_bf16(float(v)) == exp_bits, v


def _e4m3_closed_form(c):
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 15
    m = c & 7
    if e == 15 and m == 7:
        return float("nan")
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (1 + m / 8) * 2.0 ** (e - 7)


def test_e4m3_decode_all_codes():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float32).numpy()
    for c in range(256):
        got = oracle.e4m3_to_f32(c)
        cf = _e4m3_closed_form(c)
        if math.isnan(cf):
            assert math.isnan(got) and math.isnan(ref[c])
        else:
            assert got == cf == ref[c], c
            assert math.copysign(1, got) == math.copysign(1, cf)
    assert oracle.e4m3_to_f32(0x7E) == 448.0


def test_e4m3_encode_roundtrip_and_midpoints():
    finite_pos = [c for c in range(0x7F)]  # 0x00..0x7E
    for c in finite_pos:
        v = _e4m3_closed_form(c)
        assert oracle.f32_to_e4m3(v) == c
        assert oracle.f32_to_e4m3(-v) == (c | 0x80)
    for c in range(0x7E):
        lo, hi = _e4m3_closed_form(c), _e4m3_closed_form(c + 1)
        mid = (lo + hi) / 2  # exact in fp32
        even = c if c % 2 == 0 else c + 1
        assert oracle.f32_to_e4m3(mid) == even, (c, mid)
        assert oracle.f32_to_e4m3(float(np.nextafter(np.float32(mid), np.float32(np.inf)))) == c + 1
        assert oracle.f32_to_e4m3(float(np.nextafter(np.float32(mid), np.float32(-np.inf)))) == c


def test_e4m3_saturates_and_nan():
    for v in [448.0, 449.0, 463.99, 464.0, 1e9, float("inf")]:
        assert oracle.f32_to_e4m3(v) == 0x7E
        assert oracle.f32_to_e4m3(-v) == 0xFE
    assert oracle.f32_to_e4m3(float("nan")) == 0x7F
    assert oracle.f32_to_e4m3(2.0 ** -10) == 0x00   # half of the smallest subnormal -> even (0)
    assert oracle.f32_to_e4m3(3 * 2.0 ** -10) == 0x02  # 1.5 ulps -> 2 (even)


def test_e4m3_matches_torch_inside_range():
    """torch's cast is round-to-nearest-even and does not saturate; below 464
    in magnitude the two must agree exactly."""
    rng = np.random.default_rng(5)
    vals = np.concatenate([
        rng.uniform(-463.9, 463.9, 5000),
        rng.standard_normal(5000) * 2.0 ** rng.uniform(-12, 8, 5000),
    ]).astype(np.float32)
    vals = vals[np.abs(vals) < 464.0]
    ref = torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = np.array([oracle.f32_to_e4m3(float(v)) for v in vals], np.uint8)
    assert np.array_equal(got, ref)
