"""Exact rational helpers for the oracle pins: round an exact value to binary32."""
from fractions import Fraction
import math
import struct


def f32_bits(x: float) -> int:
    return struct.unpack("<I", struct.pack("<f", x))[0]


def f32_from_bits(u: int) -> float:
    return struct.unpack("<f", struct.pack("<I", u))[0]


def round_half_even(q: Fraction) -> int:
    fl = math.floor(q)
    rem = q - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        return fl + 1
    return fl


def to_f32(q: Fraction) -> float:
    """The binary32 value nearest to the exact rational q (ties to even); overflow -> inf."""
    if q == 0:
        return 0.0
    sign = -1.0 if q < 0 else 1.0
    a = abs(q)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    # a in [2^e, 2^(e+1)); 24 significant bits, or the fixed subnormal quantum 2^-149
    quantum_exp = max(e - 23, -149)
    n = round_half_even(a / Fraction(2) ** quantum_exp)
    v = n * Fraction(2) ** quantum_exp
    if v >= Fraction(2) ** 128:
        return sign * math.inf
    return sign * float(v)   # exact: v has <= 24 significant bits and is in double range
