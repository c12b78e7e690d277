"""Number formats used by the FP8 linear layer: OCP e4m3 ("float8_e4m3fn") and bf16.

Oracle module -- test infrastructure only (see ``oracle/__init__.py``).

e4m3fn (Admin Guide "DeepSeek-V3 Administrator & Developer Guide" 8.5.1: the
quantised activations are cast to ``float8_e4m3fn`` and 448 is its largest
magnitude; DocSearch index of the DeepSeek-V3 README, item 10: ``fmt: e4m3``
means ``torch.float8_e4m3fn``).  A code is ``s eeee mmm``:

* e == 0            -> (-1)^s * 2^-6 * m/8           (subnormal, spacing 2^-9)
* 1 <= e <= 15      -> (-1)^s * 2^(e-7) * (1 + m/8)  except
* e == 15, m == 7   -> NaN (0x7F, 0xFF); there is no infinity.

Encoding is round-to-nearest-even with saturation to +-448; the sign of a zero
is kept (``-tiny`` encodes to 0x80) and subnormals are produced, not flushed.

bf16 is handled as raw ``uint16`` bit patterns: widening to fp32 is the exact
``bits << 16``; narrowing is round-to-nearest-even to 8 significant bits.

Two independent encoders are given for e4m3 and for bf16: a vectorised one
built from frexp / rint in float64 (all steps exact), and a scalar one that
searches the representable values with exact rational arithmetic.  The tests
pin both against each other and against torch's own casts.
"""

from fractions import Fraction

import numpy as np

E4M3_MAX = 448.0
_E4M3_MIN_NORMAL_EXP = -6      # smallest normal binade: 2^-6
_E4M3_MANT_BITS = 3


def e4m3_decode(codes):
    """Value of each e4m3fn code as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = np.ldexp(m.astype(np.float64) / 8.0, -6)
    nrm = np.ldexp(1.0 + m.astype(np.float64) / 8.0, e - 7)
    val = sign * np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (m == 7), np.nan, val)


def e4m3_encode(values):
    """Saturating round-to-nearest-even fp32 -> e4m3fn codes (uint8).

    Works in float64, where every step below is exact for fp32 inputs:
    ``E`` is the binade of |v| (clamped to the smallest normal binade, so that
    subnormals use the fixed spacing 2^-9), the quotient |v| / 2^(E-3) is
    rounded half-to-even by ``rint``, and the code is rebuilt from it.  A
    rounded quotient of 16 carries into the next binade through the same
    formula.  Codes above 0x7E (the value would be >= 480, or the NaN
    pattern) saturate to 0x7E = 448.
    """
    v = np.asarray(values, dtype=np.float32)
    if not np.all(np.isfinite(v)):
        raise ValueError("e4m3_encode: non-finite input is outside the contract")
    sign = (v.view(np.uint32) >> 31).astype(np.int64)
    a = np.abs(v.astype(np.float64))
    _, e2 = np.frexp(a)                      # a = f * 2^e2, f in [0.5, 1)
    E = np.where(a < 2.0 ** _E4M3_MIN_NORMAL_EXP, _E4M3_MIN_NORMAL_EXP, e2 - 1)
    q = np.ldexp(a, -(E - _E4M3_MANT_BITS))  # exact power-of-two scaling
    r = np.rint(q).astype(np.int64)          # ties to even
    code = (E + 7) * 8 + r - 8
    code = np.minimum(code, 0x7E)
    return (code | (sign << 7)).astype(np.uint8)


# --- scalar exact reference -------------------------------------------------

def e4m3_value_exact(code):
    """Exact rational value of a finite e4m3fn code (raises on NaN codes)."""
    code = int(code) & 0xFF
    s, e, m = code >> 7, (code >> 3) & 0xF, code & 7
    if e == 15 and m == 7:
        raise ValueError("NaN code")
    if e == 0:
        mag = Fraction(m, 8) * Fraction(1, 2 ** 6)
    else:
        mag = (1 + Fraction(m, 8)) * (Fraction(2) ** (e - 7))
    return -mag if s else mag


_POS = None


def e4m3_encode_scalar(value):
    """Nearest finite e4m3fn code by exhaustive search over exact values.

    Ties go to the even code (the code's parity is its mantissa's parity);
    magnitudes at or above 448 saturate to 0x7E; a zero result keeps the sign
    of the input.
    """
    global _POS
    if _POS is None:
        _POS = [(e4m3_value_exact(c), c) for c in range(0x7F)]
    f = np.float32(value)
    neg = bool(np.signbit(f))
    a = abs(Fraction(float(f)))
    if a >= 448:
        code = 0x7E
    else:
        best = None
        for val, c in _POS:
            d = abs(val - a)
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        code = best[1]
    return code | (0x80 if neg else 0)


# --- bf16 -------------------------------------------------------------------

def bf16_to_f32(bits):
    """Exact widening of bf16 bit patterns (uint16) to float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    return (b << 16).view(np.float32)


def f32_to_bf16(values):
    """Round float32 (or float64) values to bf16, nearest-even; returns uint16 bits.

    Same construction as ``e4m3_encode``: bf16 keeps 8 significant bits and
    fp32's exponent range, so the spacing in binade E is 2^(E-7), with a fixed
    spacing of 2^-133 below the smallest normal 2^-126.  Results that round to
    2^128 or beyond become infinity.  NaN inputs are outside the contract.
    """
    v = np.asarray(values, dtype=np.float64)
    if np.any(np.isnan(v)):
        raise ValueError("f32_to_bf16: NaN input is outside the contract")
    neg = np.signbit(v)
    a = np.abs(v)
    fin = np.isfinite(a)
    a0 = np.where(fin, a, 0.0)
    _, e2 = np.frexp(a0)
    E = np.where(a0 < 2.0 ** -126, -126, e2 - 1)
    q = np.ldexp(a0, -(E - 7))
    r = np.rint(q)
    mag = np.ldexp(r, E - 7)
    mag = np.where(fin & (mag < 2.0 ** 128), mag, np.inf)
    out = np.where(neg, -mag, mag).astype(np.float32)  # exact: mag is a bf16 value
    return (out.view(np.uint32) >> 16).astype(np.uint16)


def f32_to_bf16_scalar(value):
    """bf16 rounding of one finite value by exact rational arithmetic."""
    x = Fraction(float(value))
    neg = x < 0 or (x == 0 and np.signbit(np.float64(value)))
    a = abs(x)
    if a == 0:
        return 0x8000 if neg else 0
    # binade: 2^E <= a < 2^(E+1)
    E = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** E > a:
        E -= 1
    E = max(E, -126)
    spacing = Fraction(2) ** (E - 7)
    q = a / spacing
    lo = q.numerator // q.denominator
    rem = q - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    mag = lo * spacing
    if mag >= Fraction(2) ** 128:
        bits = 0x7F80
    else:
        bits = int(np.float32(float(mag)).view(np.uint32) >> 16)
    return bits | (0x8000 if neg else 0)
