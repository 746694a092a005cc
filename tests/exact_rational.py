"""Exact-rational models of the two roundings of the cache writer, for pins.

Everything here works on ``fractions.Fraction`` values, with no floating
point anywhere: ``round_f32`` rounds an exact rational to the nearest IEEE
binary32 value (ties to even mantissa), and ``e4m3_code`` rounds an exact
rational to the nearest OCP e4m3fn value (ties to even mantissa, saturating
at 448) and returns its byte.  Tests use them to derive, from first
principles, the codes a quantizer must produce; they share nothing with the
oracle or the library.
"""

from fractions import Fraction

F = Fraction


def _floor_log2(a: Fraction) -> int:
    """floor(log2(a)) for a > 0, exactly."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(m: Fraction) -> int:
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > F(1, 2) or (rem == F(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def round_f32(q: Fraction) -> Fraction:
    """Nearest binary32 value to q (24-bit significand, subnormals below
    2^-126 with spacing 2^-149), ties to even.  No overflow handling: the
    callers stay far below 2^128."""
    q = F(q)
    if q == 0:
        return F(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(_floor_log2(a), -126)
    ulp = F(2) ** (e - 23)
    return sign * _round_half_even(a / ulp) * ulp


def e4m3_code(y: Fraction) -> int:
    """OCP e4m3fn byte of the value nearest to y: 3 mantissa bits, exponent
    bias 7, subnormal spacing 2^-9 below 2^-6, ties to even mantissa,
    magnitudes that round above 448 saturate to 448 (byte 0x7E)."""
    y = F(y)
    sign = 0x80 if y < 0 else 0
    a = abs(y)
    if a == 0:
        return sign
    e = max(_floor_log2(a), -6)
    ulp = F(2) ** (e - 3)
    m = _round_half_even(a / ulp)           # significand in units of ulp: 8..16 (normal)
    val = m * ulp
    if val >= 448:
        return sign | 0x7E
    if val < F(2) ** -6:                     # subnormal: m in 0..7 counts 2^-9
        return sign | m
    e2 = _floor_log2(val)                    # may have carried to the next binade
    mant = val / F(2) ** e2 * 8 - 8          # 0..7
    assert mant.denominator == 1 and 0 <= mant < 8
    return sign | ((e2 + 7) << 3) | int(mant)


def quantize_exact(x: Fraction, amax: Fraction):
    """(scale, code) of one element under the writer's reading: scale =
    round_f32(amax / 448), y = round_f32(x / scale), code = e4m3_code(y)."""
    s = round_f32(F(amax) / 448)
    return s, e4m3_code(round_f32(F(x) / s))


def quantize_by_reciprocal(x: Fraction, amax: Fraction):
    """The same with x * round_f32(1 / scale) in place of the division: the
    alternative reading the pins must tell apart."""
    s = round_f32(F(amax) / 448)
    r = round_f32(1 / s)
    return s, e4m3_code(round_f32(F(x) * r))


def _next_f32(r: Fraction, up: bool) -> Fraction:
    """The binary32 neighbour of a positive binary32 value r."""
    e = max(_floor_log2(r), -126)
    ulp = F(2) ** (e - 23)
    if up:
        return r + ulp
    # stepping down from a power of two halves the spacing
    if r == F(2) ** e and e > -126:
        return r - ulp / 2
    return r - ulp


def sqrt_f32(v: Fraction) -> Fraction:
    """The binary32 value nearest to sqrt(v) for v >= 0, decided exactly:
    r is nearest when v lies between the squares of the midpoints to its
    neighbours (a square root never falls on such a midpoint)."""
    import math
    v = F(v)
    if v == 0:
        return F(0)
    r = round_f32(F(math.sqrt(v.numerator / v.denominator)))
    while True:
        up = _next_f32(r, True)
        if v >= ((r + up) / 2) ** 2:
            r = up
            continue
        dn = _next_f32(r, False)
        if v < ((r + dn) / 2) ** 2:
            r = dn
            continue
        return r
