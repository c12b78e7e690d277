"""The quotient scheme of the quantisation kernels, checked exhaustively on the CPU.

The kernels divide each element by its block scale s as
    q = RN(x * r),  t = RN(q * s - x) (one fma),  result = RN(q - t * r) (one fma)
with r = RN(1 / s).  This test emulates those three roundings with exact
rational arithmetic and compares the result with the correctly rounded
quotient RN(x / s) that act_quant requires, for every pair of significands the
kernels can meet: x any bf16 significand (128), s any significand of
RN(max(amax, fl(1e-4)) / 448) with amax a bf16 value (128, plus the clamp
value), both signs and several relative binades.  Rounding of all three steps
is invariant under scaling x and s by powers of two while every intermediate
stays normal, which holds whenever the quotient is large enough (>= 2^-11) to
round to a non-zero e4m3 code; smaller quotients encode to a signed zero
either way.  For ue8m0 scales (powers of two) every step is exact.

The correction step is Markstein's (P. Markstein, IBM J. Res. Dev. 34(1),
1990); his theorem gives correct rounding under conditions on the
reciprocal and the first quotient, and this exhaustive rational check is
what establishes it on the domain above.  That domain is every use of the
scheme in the library: act_quant, act_quant of gathered rows and the SiLU
gate's quantisation (standalone and in the gated product's epilogue) all
divide a bf16 value by a scale derived from a bf16 block maximum.  The
weight quantiser, whose fp32 weights lie outside it, uses the correctly
rounded IEEE division instead.
"""

from fractions import Fraction

import numpy as np


def rn32(x):
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


def test_corrected_quotient_is_correctly_rounded():
    scales = {rn32(Fraction(128 + m, 128) / 448) for m in range(128)}
    scales.add(rn32(Fraction(float(np.float32(1e-4))) / 448))
    bad = []
    for s in scales:
        r = rn32(1 / s)
        for m in range(128):
            for sh in (-8, 0, 1, 5, 11):
                x = Fraction(128 + m, 128) * Fraction(2) ** (-sh)
                for xx in (x, -x):
                    q = rn32(xx * r)
                    t = rn32(q * s - xx)
                    q1 = rn32(q - t * r)
                    if q1 != rn32(xx / s):
                        bad.append((s, xx))
    assert not bad, bad[:5]


def _f32(x):
    """The fp32 value of a Fraction that is representable (checked)."""
    v = np.float32(float(x))
    assert Fraction(float(v)) == x
    return v


def _neighbours(y, k):
    """The fp32 values within k units in the last place of fp32 y (y > 0)."""
    out = [np.float32(y)]
    lo = hi = np.float32(y)
    for _ in range(k):
        lo = np.nextafter(lo, np.float32(0))
        hi = np.nextafter(hi, np.float32(np.inf))
        out += [lo, hi]
    return [Fraction(float(v)) for v in out]


# Every block maximum the quantisers meet is a bf16 value (the input, or the
# gate's bf16 output) or the clamp constant fl(1e-4); by scale invariance
# (every intermediate below stays normal for a >= 1e-4) one binade of bf16
# significands covers them all.
_AMAXES = [Fraction(128 + m, 128) for m in range(128)] + [Fraction(float(np.float32(1e-4)))]


def test_scale_by_reciprocal_and_correction():
    """s = RN(a / 448) computed as q = RN(a * r), t = RN(q * 448 - a) (fma,
    exact), s = RN(q - t * r) with r = RN(1 / 448)."""
    r = rn32(Fraction(1, 448))
    bad = []
    for a in _AMAXES:
        q = rn32(a * r)
        t = rn32(q * 448 - a)
        assert t == q * 448 - a          # the fma residual is exact
        s = rn32(q - t * r)
        if s != rn32(a / 448):
            bad.append(a)
    assert not bad, bad[:5]


def test_reciprocal_refinement():
    """RN(1 / s) for every scale s the quantisers can produce (fp32 scales
    RN(a / 448) and power-of-two scales), computed as r0 = the hardware
    reciprocal, e = RN(1 - s * r0) (fma), r = RN(r0 + r0 * e) (fma): correct
    for every r0 within two units in the last place of 1/s (the hardware
    reciprocal is specified to within one)."""
    scales = {rn32(a / 448) for a in _AMAXES} | {Fraction(1)}
    bad = []
    for s in scales:
        # scale to [1, 2): the refinement is invariant under powers of two
        while s >= 2:
            s /= 2
        while s < 1:
            s *= 2
        want = rn32(1 / s)
        for r0 in _neighbours(_f32(want), 2):
            e = rn32(1 - s * r0)
            r = rn32(r0 + r0 * e)
            if r != want:
                bad.append((s, r0))
    assert not bad, bad[:5]
