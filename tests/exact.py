"""Exact-arithmetic helpers for pinning the oracle (tests only).

Rounding here is done the long way, independently of the oracle's C code:
the finite non-negative values of a binary format are enumerated in bit-pattern
order (which is also value order), the largest pattern not above the exact
value is found by binary search over exact ``Fraction`` values, and the exact
midpoint to the next pattern decides, ties going to the even pattern.
"""
import struct
from decimal import Decimal, getcontext
from fractions import Fraction

getcontext().prec = 80


def f32_value(bits: int) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<I", bits & 0xFFFFFFFF))[0])


def bf16_value(bits: int) -> Fraction:
    return f32_value((bits & 0xFFFF) << 16)


def _round_pattern(q: Fraction, value, max_finite: int, inf_bits: int, sign_bit: int) -> int:
    neg = q < 0
    a = -q if neg else q
    lo, hi = 0, max_finite  # value(lo) <= a is invariant once a >= 0
    if a >= value(max_finite):
        # beyond the largest finite value: overflow threshold is max + half a spacing
        top = value(max_finite)
        spacing = top - value(max_finite - 1)
        if a >= top + spacing / 2:
            return (sign_bit if neg else 0) | inf_bits
        p = max_finite
    else:
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if value(mid) <= a:
                lo = mid
            else:
                hi = mid
        p = lo
        if value(p) != a:
            mid_val = (value(p) + value(p + 1)) / 2
            if a > mid_val or (a == mid_val and (p & 1)):
                p += 1
    return (sign_bit if neg else 0) | p


def round_bf16_exact(q) -> int:
    """Nearest-even bf16 bit pattern of an exact rational (or Decimal)."""
    q = Fraction(q)
    return _round_pattern(q, bf16_value, 0x7F7F, 0x7F80, 0x8000)


def round_f32_exact(q) -> int:
    q = Fraction(q)
    return _round_pattern(q, f32_value, 0x7F7FFFFF, 0x7F800000, 0x80000000)


def f32_bits(v: float) -> int:
    return struct.unpack("<I", struct.pack("<f", v))[0]


def ulp_distance_bf16(a: int, b: int) -> int:
    """Distance between two bf16 patterns on the monotone integer line (+0 == -0)."""
    def key(u):
        u &= 0xFFFF
        return -(u & 0x7FFF) if u & 0x8000 else u
    return abs(key(a) - key(b))


def near_midpoint(q: Fraction, rounded_value: Fraction, spacing: Fraction, rel: float) -> bool:
    """True if the exact value q lies within ``rel`` (relative) of a rounding midpoint."""
    d = abs(abs(q) - abs(rounded_value))
    return abs(d - spacing / 2) <= Fraction(rel) * abs(q)


def rmsnorm_decimal(v, w, eps32: float):
    """RMSNorm of one row in 80-digit decimal arithmetic (Decimal sqrt), exact inputs.

    Used only as a high-precision brute force for tiny rows."""
    dv = [Decimal(Fraction(a).numerator) / Decimal(Fraction(a).denominator) for a in v]
    dw = [Decimal(Fraction(a).numerator) / Decimal(Fraction(a).denominator) for a in w]
    de = Decimal(Fraction(eps32).numerator) / Decimal(Fraction(eps32).denominator)
    s = sum(a * a for a in dv)
    r = 1 / (s / len(dv) + de).sqrt()
    return [a * r * b for a, b in zip(dv, dw)]


def e4m3_value(code: int) -> Fraction:
    """Exact value of an fp8 e4m3fn code (1 sign, 4 exponent bits bias 7, 3
    mantissa bits; 0x7F / 0xFF are NaN and not valid here)."""
    sign = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0:
        return sign * Fraction(m, 8) * Fraction(1, 64)
    return sign * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def round_e4m3_exact(q) -> int:
    """Nearest-even e4m3fn code of an exact rational, saturating at +-448."""
    q = Fraction(q)
    neg = q < 0
    a = -q if neg else q
    if a >= 448:
        p = 0x7E
    else:
        lo, hi = 0, 0x7E  # value(lo) <= a < value(hi)
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if e4m3_value(mid) <= a:
                lo = mid
            else:
                hi = mid
        p = lo
        if e4m3_value(p) != a:
            mid_val = (e4m3_value(p) + e4m3_value(p + 1)) / 2
            if a > mid_val or (a == mid_val and (p & 1)):
                p += 1
    return (0x80 if neg else 0) | p


def round_half_even(q) -> int:
    """Nearest integer to an exact rational, ties to even."""
    q = Fraction(q)
    fl = q.numerator // q.denominator
    frac = q - fl
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and fl % 2):
        return fl + 1
    return fl
