"""Exact-arithmetic helpers for pinning the oracle (rational numbers and 60-digit decimals).

These re-derive roundings from first principles with Python's Fraction and
Decimal types; they share nothing with the oracle's numpy code.
"""

from decimal import Decimal, localcontext
from fractions import Fraction
import math
import struct


def frac_of_f32(v: float) -> Fraction:
    return Fraction(struct.unpack("<f", struct.pack("<f", v))[0])


def frac_of_bf16(bits: int) -> Fraction:
    v = struct.unpack("<f", struct.pack("<I", (bits & 0xFFFF) << 16))[0]
    if math.isnan(v) or math.isinf(v):
        raise ValueError("not finite")
    return Fraction(v)


def _binade(a: Fraction) -> int:
    """e with 2^e <= a < 2^(e+1), for a > 0."""
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    return e


def _round_half_even(n: Fraction) -> int:
    fl = n.numerator // n.denominator
    r = n - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def rne_bf16_bits(x) -> int:
    """Exact round-to-nearest-even of a rational (or Decimal) to bf16 bits."""
    x = Fraction(x)
    sign = 0x8000 if x < 0 else 0
    a = abs(x)
    if a == 0:
        return sign
    e = max(_binade(a), -126)
    n = _round_half_even(a / Fraction(2) ** (e - 7))
    if n == 256:
        e, n = e + 1, 128
    if e > 127:
        return sign | 0x7F80
    if n < 128:  # subnormal (only possible at e == -126)
        return sign | n
    return sign | ((e + 127) << 7) | (n - 128)


def rne_f32(x) -> float:
    """Exact round-to-nearest-even of a rational to fp32 (returned as a Python float)."""
    x = Fraction(x)
    sign = -1 if x < 0 else 1
    a = abs(x)
    if a == 0:
        return 0.0 * sign
    e = max(_binade(a), -126)
    n = _round_half_even(a / Fraction(2) ** (e - 23))
    v = Fraction(n) * Fraction(2) ** (e - 23)
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)


def dec(x) -> Decimal:
    f = Fraction(x)
    return Decimal(f.numerator) / Decimal(f.denominator)


def sigmoid_dec(x) -> Decimal:
    """sigmoid in 60-digit decimal arithmetic (x rational)."""
    with localcontext() as ctx:
        ctx.prec = 60
        d = dec(x)
        if d >= 0:
            return Decimal(1) / (Decimal(1) + (-d).exp())
        ed = d.exp()
        return ed / (Decimal(1) + ed)


def silu_dec(x) -> Decimal:
    with localcontext() as ctx:
        ctx.prec = 60
        return dec(x) * sigmoid_dec(x)


def softmax_picks_dec(logits):
    """exp(l_i - l_0) / sum_j exp(l_j - l_0) for a list of rationals, 60 digits."""
    with localcontext() as ctx:
        ctx.prec = 60
        l0 = dec(logits[0])
        ex = [(dec(l) - l0).exp() for l in logits]
        s = sum(ex, Decimal(0))
        return [v / s for v in ex]


def unpack_int4_row(row_bytes):
    """Element 2j is the low nibble of byte j, element 2j+1 the high nibble."""
    out = []
    for b in row_bytes:
        out.append(int(b) & 0xF)
        out.append(int(b) >> 4)
    return out


def rne_e4m3(x) -> Fraction:
    """Exact round-to-nearest-even of a rational to an OCP FP8 E4M3 value: 3 mantissa
    bits, least normal magnitude 2^-6, subnormal step 2^-9, largest finite 448
    (beyond it: ValueError). Zero keeps no sign here."""
    x = Fraction(x)
    sign = -1 if x < 0 else 1
    a = abs(x)
    if a < Fraction(1, 64):
        return sign * Fraction(_round_half_even(a * 512), 512)
    e = _binade(a)
    v = _round_half_even(a / Fraction(2) ** (e - 3)) * Fraction(2) ** (e - 3)
    if v > 448:
        raise ValueError("beyond E4M3")
    return sign * v


def fp8_row_exact(vals):
    """One row quantised with its power-of-two scale: e = floor(log2 max|v|) - 7
    (0 for an all-zero row), each value replaced by rne_e4m3(v 2^-e) 2^e.
    Returns (values, e)."""
    vals = [Fraction(v) for v in vals]
    amax = max(abs(v) for v in vals)
    e = _binade(amax) - 7 if amax > 0 else 0
    s = Fraction(2) ** e
    return [rne_e4m3(v / s) * s for v in vals], e
