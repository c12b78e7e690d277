"""Pins of the oracle's number formats (CPU only).

e4m3fn: the decode table is pinned to torch's own float8_e4m3fn (a library
special case) and to closed-form values the pages fix (448 is the largest
magnitude: Admin Guide 8.5.1); the encoder is pinned to torch's cast, which is
round-to-nearest-even but does not saturate, for |v| < 464, to an exact
rational search, and to the round-trip and tie rules.  bf16 rounding is pinned
to torch's cast and to an exact rational evaluation.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F

ALL_CODES = np.arange(256, dtype=np.uint8)


def torch_decode(codes):
    t = torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn)
    return t.to(torch.float64).numpy()


def torch_encode(v):
    t = torch.from_numpy(np.asarray(v, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_decode_matches_torch_all_codes():
    ours = F.e4m3_decode(ALL_CODES)
    ref = torch_decode(ALL_CODES)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_decode_closed_forms():
    d = F.e4m3_decode
    assert d(0x7E) == 448.0                # largest magnitude, Admin Guide 8.5.1
    assert d(0xFE) == -448.0
    assert d(0x08) == 2.0 ** -6            # smallest normal
    assert d(0x01) == 2.0 ** -9            # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9        # largest subnormal
    assert d(0x38) == 1.0                  # e = 7, m = 0
    assert d(0x39) == 1.125
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    finite = F.e4m3_decode(ALL_CODES)
    assert np.nanmax(np.abs(finite)) == 448.0
    assert np.sum(np.isnan(finite)) == 2   # no infinities, two NaN codes


def test_exact_value_agrees_with_decode():
    for c in range(256):
        if c & 0x7F == 0x7F:
            continue
        assert float(F.e4m3_value_exact(c)) == F.e4m3_decode(c)


def test_encode_roundtrip_every_code():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    vals = F.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(F.e4m3_encode(vals), codes)   # includes -0 -> 0x80


def _bf16_grid():
    """Every finite bf16 value, as fp32."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = F.bf16_to_f32(bits)
    return v[np.isfinite(v)]


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -5, 1.0 / 448.0, 0.37, 3.1e-3, 117.0])
def test_encode_matches_torch_below_saturation(scale):
    v = (_bf16_grid() * np.float32(scale)).astype(np.float32)
    v = v[np.isfinite(v) & (np.abs(v) < 464.0)]
    assert np.array_equal(F.e4m3_encode(v), torch_encode(v))


def test_encode_matches_torch_random_fp32():
    g = np.random.default_rng(1)
    v = (g.standard_normal(200_000) * np.exp(g.uniform(-12, 6, 200_000))).astype(np.float32)
    v = v[np.abs(v) < 464.0]
    assert np.array_equal(F.e4m3_encode(v), torch_encode(v))


def test_encode_saturates():
    big = np.array([448.0, 448.00003, 463.99, 464.0, 464.01, 479.0, 480.0, 512.0, 1e6, 3e38], np.float32)
    assert np.all(F.e4m3_encode(big) == 0x7E)
    assert np.all(F.e4m3_encode(-big) == 0xFE)
    # torch does not saturate: the documented difference starts above the midpoint 464
    assert np.all(torch_encode(np.array([480.0], np.float32)) & 0x7F == 0x7F)


def test_encode_ties_to_even():
    pos = [c for c in range(0x7E)]
    for c in pos:
        lo, hi = F.e4m3_value_exact(c), F.e4m3_value_exact(c + 1)
        mid = (lo + hi) / 2
        fm = np.float32(float(mid))
        assert Fraction(float(fm)) == mid       # every e4m3 midpoint is an fp32 value
        want = c if c % 2 == 0 else c + 1
        assert F.e4m3_encode(np.array([fm]))[0] == want
        assert F.e4m3_encode(np.array([-fm]))[0] == want | 0x80


def test_encode_signed_zero_and_underflow():
    v = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0001], np.float32)
    assert list(F.e4m3_encode(v)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x01]


def test_encode_vectorised_equals_exact_search():
    g = np.random.default_rng(2)
    v = np.concatenate([
        (g.standard_normal(3000) * np.exp(g.uniform(-14, 7, 3000))).astype(np.float32),
        np.array([0.0, -0.0, 448.0, 470.0, -500.0, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -11], np.float32),
    ])
    vec = F.e4m3_encode(v)
    for x, c in zip(v, vec):
        assert F.e4m3_encode_scalar(x) == c, x


def test_encode_rejects_nonfinite():
    with pytest.raises(ValueError):
        F.e4m3_encode(np.array([np.inf], np.float32))


def test_bf16_widen_exact():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = F.bf16_to_f32(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))


def test_bf16_round_matches_torch():
    g = np.random.default_rng(3)
    v = (g.standard_normal(500_000) * np.exp(g.uniform(-80, 80, 500_000))).astype(np.float32)
    # exact ties: bf16 value + half an ulp, both parities
    base = F.bf16_to_f32(g.integers(0, 0x7F00, 20_000).astype(np.uint16))
    ties = (base.view(np.uint32) | np.uint32(0x8000)).view(np.float32)
    v = np.concatenate([v, ties, -ties, np.array([0.0, -0.0, 3.3e38, 1e-40, -1e-42], np.float32)])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(F.f32_to_bf16(v), ref)


def test_bf16_round_matches_exact_scalar():
    g = np.random.default_rng(4)
    v = np.concatenate([
        (g.standard_normal(2000) * np.exp(g.uniform(-90, 90, 2000))),
        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 2.0 ** -130, 1.5 * 2.0 ** -133, -0.0, 3.39e38]),
    ])
    vec = F.f32_to_bf16(v)
    for x, b in zip(v, vec):
        assert F.f32_to_bf16_scalar(x) == b, x
