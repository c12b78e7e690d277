"""Pins of the oracle's quantisers (CPU only).

act_quant (Admin Guide 8.5.1; ue8m0: User Guide FAQ) is pinned by a
hand-worked block, an exact rational re-derivation on small inputs, and the
invariants the definition implies: the block maximum encodes to +-448, the
round trip is within half an e4m3 ulp (plus the fp32 rounding of x/s),
power-of-two equivariance, zero-padding invariance (DocSearch item 3), row
permutation equivariance, and the all-zero clamp.  weight_dequant (Admin
Guide 8.5.2) is pinned to torch's own float8 decode and bf16 cast, and to the
exact closed form for power-of-two scales.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import quant as Q

FL_1EM4 = Fraction(float(np.float32(1e-4)))


def rn32(x):
    """Exact round-to-nearest-even of a rational to fp32 (normal range)."""
    if x == 0:
        return Fraction(0)
    neg = x < 0
    a = -x if neg else x
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    sp = Fraction(2) ** (E - 23)
    q = a / sp
    lo = q.numerator // q.denominator
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2):
        lo += 1
    return -(lo * sp) if neg else lo * sp


def pow2_ceil_exact(s):
    p = Fraction(1)
    while p < s:
        p *= 2
    while p / 2 >= s:
        p /= 2
    return p


def act_quant_exact(x_bits, ue8m0):
    """Rational re-derivation of act_quant, element by element."""
    x = F.bf16_to_f32(x_bits)
    M, K = x.shape
    nb = (K + 127) // 128
    y = np.zeros((M, K), np.uint8)
    s = np.zeros((M, nb), np.float32)
    for m in range(M):
        for b in range(nb):
            cols = range(b * 128, min(K, b * 128 + 128))
            amax = max(abs(Fraction(float(x[m, k]))) for k in cols)
            sc = rn32(max(amax, FL_1EM4) / 448)
            if ue8m0:
                sc = pow2_ceil_exact(sc)
            s[m, b] = float(sc)
            for k in cols:
                q = rn32(Fraction(float(x[m, k])) / sc)
                y[m, k] = F.e4m3_encode_scalar(float(q)) if q != 0 else (0x80 if np.signbit(x[m, k]) else 0)
    return y, s


def bf16(v):
    return F.f32_to_bf16(np.asarray(v, np.float32))


def rand_x(shape, seed, spread=3.0):
    g = np.random.default_rng(seed)
    v = g.standard_normal(shape) * np.exp(g.uniform(-spread, spread, shape))
    return bf16(v)


def test_hand_worked_block():
    # amax = 56 = 448 / 8, so s = 1/8 exactly and y = 8x.
    x = np.zeros((1, 128), np.float32)
    x[0, :6] = [56.0, -28.0, 1.0, 0.0625, -0.0, 3.0]
    y, s = Q.act_quant(bf16(x))
    assert s[0, 0] == np.float32(0.125)
    # 448 -> 0x7E; -224 = -1.75*2^7 -> 0xF6; 8 = 2^3 -> 0x50; 0.5 -> 0x30;
    # -0 -> 0x80; 24 = 1.5*2^4 -> 0x5C; zeros -> 0x00
    assert list(y[0, :6]) == [0x7E, 0xF6, 0x50, 0x30, 0x80, 0x5C]
    assert np.all(y[0, 6:] == 0)


def test_matches_exact_rational_small():
    for seed, (M, K) in enumerate([(3, 128), (2, 300), (4, 1000), (1, 5)]):
        x = rand_x((M, K), 10 + seed)
        for ue in (False, True):
            y, s = Q.act_quant(x, ue8m0=ue)
            ye, se = act_quant_exact(x, ue)
            assert np.array_equal(s.view(np.uint32), se.view(np.uint32))
            assert np.array_equal(y, ye)


def test_block_max_encodes_to_448():
    x = rand_x((64, 1024), 20)
    y, s = Q.act_quant(x)
    xf = F.bf16_to_f32(x).reshape(64, 8, 128)
    yb = y.reshape(64, 8, 128)
    idx = np.argmax(np.abs(xf), axis=2)
    top = np.take_along_axis(yb, idx[..., None], axis=2)[..., 0]
    assert np.all(top & 0x7F == 0x7E)


def test_ue8m0_scale_is_power_of_two_and_max_in_range():
    x = rand_x((64, 512), 21)
    y, s = Q.act_quant(x, ue8m0=True)
    m, e = np.frexp(s.astype(np.float64))
    assert np.all(m == 0.5)
    _, s0 = Q.act_quant(x)
    assert np.all(s >= s0) and np.all(s < 2 * s0)
    mags = F.e4m3_decode(y.reshape(64, 4, 128) & 0x7F).max(axis=2)
    assert np.all((mags >= 224) & (mags <= 448))


def test_pow2_ceil_exact():
    g = np.random.default_rng(5)
    v = np.concatenate([
        np.exp(g.uniform(-30, 30, 5000)).astype(np.float32),
        np.ldexp(np.ones(40, np.float32), np.arange(-20, 20)),
        np.nextafter(np.ldexp(np.ones(40, np.float32), np.arange(-20, 20)), np.float32(np.inf)),
    ]).astype(np.float32)
    got = Q.pow2_ceil(v)
    for a, b in zip(v, got):
        assert Fraction(float(b)) == pow2_ceil_exact(Fraction(float(a)))


def test_roundtrip_within_half_ulp():
    x = rand_x((32, 640), 22)
    y, s = Q.act_quant(x)
    xf = F.bf16_to_f32(x).astype(np.float64)
    cols = np.arange(640) // 128
    sf = s.astype(np.float64)[:, cols]
    q = xf / sf
    aq = np.minimum(np.abs(q), 448.0)
    E = np.maximum(np.floor(np.log2(np.maximum(aq, 2.0 ** -30))), -6)
    half_ulp = np.ldexp(0.5, (E - 3).astype(int))
    err = np.abs(F.e4m3_decode(y) - q)
    assert np.all(err <= half_ulp + 2.0 ** -23 * np.abs(q) + 1e-300)


def test_power_of_two_equivariance():
    x = rand_x((16, 384), 23, spread=1.0)
    y, s = Q.act_quant(x)
    for j in (-8, -3, 1, 5, 20):
        xs = bf16(F.bf16_to_f32(x) * np.float32(2.0 ** j))
        y2, s2 = Q.act_quant(xs)
        assert np.array_equal(y2, y)
        assert np.array_equal(s2, (s * np.float32(2.0 ** j)).astype(np.float32))


def test_zero_padding_invariance():
    x = rand_x((20, 1000), 24)
    xp = np.zeros((20, 1024), np.uint16)
    xp[:, :1000] = x
    for ue in (False, True):
        y, s = Q.act_quant(x, ue8m0=ue)
        yp, sp = Q.act_quant(xp, ue8m0=ue)
        assert s.shape == (20, 8)
        assert np.array_equal(y, yp[:, :1000])
        assert np.array_equal(s, sp)


def test_row_permutation_equivariance():
    x = rand_x((50, 256), 25)
    perm = np.random.default_rng(0).permutation(50)
    y, s = Q.act_quant(x)
    yp, sp = Q.act_quant(x[perm])
    assert np.array_equal(yp, y[perm]) and np.array_equal(sp, s[perm])


def test_all_zero_block_clamps():
    x = np.zeros((2, 256), np.uint16)
    x[1, :] = 0x8000                      # -0.0
    y, s = Q.act_quant(x)
    assert np.all(s == np.float32(np.float32(1e-4) / np.float32(448.0)))
    assert np.all(y[0] == 0x00) and np.all(y[1] == 0x80)


def test_tiny_amax_below_clamp():
    x = bf16(np.full((1, 128), 3e-5, np.float32))
    y, s = Q.act_quant(x)
    assert s[0, 0] == np.float32(np.float32(1e-4) / np.float32(448.0))
    q = np.float32(F.bf16_to_f32(x)[0, 0]) / s[0, 0]
    assert np.all(y == F.e4m3_encode(np.array([q]))[0])


def test_empty_inputs():
    y, s = Q.act_quant(np.zeros((0, 256), np.uint16))
    assert y.shape == (0, 256) and s.shape == (0, 2)
    y, s = Q.act_quant(np.zeros((3, 0), np.uint16))
    assert y.shape == (3, 0) and s.shape == (3, 0)


# ---- weights -------------------------------------------------------------------

def test_weight_quant_block_max_and_padding():
    g = np.random.default_rng(30)
    w = (g.standard_normal((300, 260)) * 0.02).astype(np.float32)
    q, S = Q.weight_quant(w)
    assert S.shape == (3, 3)
    for i in range(3):
        for j in range(3):
            blk = w[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            qb = q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            r, c = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
            assert qb[r, c] & 0x7F == 0x7E
            assert S[i, j] == np.float32(np.max(np.abs(blk)) / np.float32(448))
    wp = np.zeros((384, 384), np.float32)
    wp[:300, :260] = w
    qp, Sp = Q.weight_quant(wp)
    assert np.array_equal(qp[:300, :260], q) and np.array_equal(Sp, S)


def test_weight_quant_rows_match_act_quant_on_one_block_row():
    # A 1-row weight is a 1x128 block per scale: the same arithmetic as
    # act_quant on an fp32 row that is exactly representable in bf16.
    x = rand_x((1, 512), 31)
    w = F.bf16_to_f32(x)
    q, S = Q.weight_quant(w)
    y, s = Q.act_quant(x)
    assert np.array_equal(q, y) and np.array_equal(S, s)


def test_weight_dequant_matches_torch():
    g = np.random.default_rng(32)
    w = (g.standard_normal((260, 300)) * 0.02).astype(np.float32)
    q, S = Q.weight_quant(w)
    out = Q.weight_dequant(q, S)
    qt = torch.from_numpy(q).view(torch.float8_e4m3fn).float()
    St = torch.from_numpy(Q.expand_block_scales(S, 260, 300))
    ref = (qt * St).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out, ref)


def test_weight_dequant_pow2_closed_form():
    g = np.random.default_rng(33)
    w = (g.standard_normal((256, 256)) * 0.02).astype(np.float32)
    q, S = Q.weight_quant(w, ue8m0=True)
    out = Q.weight_dequant(q, S)
    exact = F.e4m3_decode(q) * Q.expand_block_scales(S, 256, 256).astype(np.float64)
    # with a power-of-two scale the fp32 product is exact, so one rounding to bf16
    assert np.array_equal(out, F.f32_to_bf16(exact))
    assert np.array_equal(F.bf16_to_f32(out).astype(np.float64), exact)  # e4m3 * 2^k fits in bf16
