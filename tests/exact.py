"""Exact rational arithmetic helpers for the oracle's pins (CPU only).

Written independently of ``oracle/``: round-to-nearest-even of an exact
rational number to a binary format with ``sig_bits`` significant bits and
minimum normal exponent ``emin`` (IEEE-754 definition).
"""

from fractions import Fraction


def floor_log2(a: Fraction) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def rne(q: Fraction, sig_bits: int, emin: int) -> Fraction:
    if q == 0:
        return Fraction(0)
    sign = -1 if q < 0 else 1
    a = abs(q)
    e = max(floor_log2(a), emin)
    quantum = Fraction(2) ** (e - sig_bits + 1)
    n = a / quantum
    fl = n.numerator // n.denominator
    rem = n - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return sign * fl * quantum


def rne_f32(q):
    return rne(Fraction(q), 24, -126)


def rne_bf16(q):
    return rne(Fraction(q), 8, -126)


def e4m3_exact(code: int) -> Fraction:
    """E4M3FN code -> exact value (OCP definition; NaN codes not allowed)."""
    s, e, m = code >> 7, (code >> 3) & 15, code & 7
    assert not (e == 15 and m == 7)
    if e == 0:
        v = Fraction(m, 8) * Fraction(2) ** (1 - 7)
    else:
        v = (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if s else v
