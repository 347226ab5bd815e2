"""Brute-force helpers for pinning the oracle: exact rational FP8 values from the OCP bit-field
definitions and nearest-value search over every finite code.  Pure Python, deliberately naive."""
from fractions import Fraction


def fp8_value(code: int, fmt: int):
    """Exact value of an FP8 code as a Fraction, or 'nan' / 'inf' / '-inf'."""
    sign = -1 if code & 0x80 else 1
    if fmt == 0:      # E4M3: 4 exponent bits, bias 7, 3 mantissa bits; S.1111.111 is NaN
        e, m = (code >> 3) & 0xF, code & 0x7
        if e == 0xF and m == 0x7:
            return "nan"
        mag = Fraction(m, 8) * Fraction(2) ** (1 - 7) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    else:             # E5M2: 5 exponent bits, bias 15, 2 mantissa bits; exponent 31 is Inf/NaN
        e, m = (code >> 2) & 0x1F, code & 0x3
        if e == 0x1F:
            return "nan" if m else ("inf" if sign > 0 else "-inf")
        mag = Fraction(m, 4) * Fraction(2) ** (1 - 15) if e == 0 else (1 + Fraction(m, 4)) * Fraction(2) ** (e - 15)
    return sign * mag


def finite_codes(fmt: int):
    return [c for c in range(256) if isinstance(fp8_value(c, fmt), Fraction)]


def nearest_code(v: float, fmt: int) -> int:
    """Nearest finite code to v (|v| <= MAX) by exhaustive search; ties go to the even code
    (mantissa LSB 0).  Sign follows v, so -0.0 and tiny negatives give 0x80."""
    import math
    x = Fraction(v)
    neg = math.copysign(1.0, v) < 0
    best = None
    for c in finite_codes(fmt):
        if (c & 0x80) != (0x80 if neg else 0):
            continue
        d = abs(fp8_value(c, fmt) - x)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return best[1]
