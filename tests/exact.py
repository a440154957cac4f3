"""Exact rational rounding helpers for pinning the oracle.

Written independently of the oracle: they work on fractions.Fraction and round
by integer arithmetic, so they share no float trick with the code they check.
"""

from fractions import Fraction as F
import struct


def _round_to_grid(a: F, ulp: F) -> F:
    """Nearest multiple of ulp to a >= 0, ties to the even multiple."""
    q = a / ulp
    n = q.numerator // q.denominator
    r = q - n
    if r > F(1, 2) or (r == F(1, 2) and n % 2 == 1):
        n += 1
    return n * ulp


def _floor_log2(a: F) -> int:
    e = a.numerator.bit_length() - a.denominator.bit_length()
    while F(2) ** e > a:
        e -= 1
    while F(2) ** (e + 1) <= a:
        e += 1
    return e


def round_binary(x: F, sig_bits: int, emin: int) -> F:
    """Round x to a binary format with sig_bits significant bits (implicit bit
    included) whose smallest normal exponent is emin (subnormals below), nearest
    even.  No overflow handling."""
    if x == 0:
        return F(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), emin)
    ulp = F(2) ** (e - (sig_bits - 1))
    return s * _round_to_grid(a, ulp)


def rn_f32(x: F) -> F:
    return round_binary(x, 24, -126)


def rn_bf16(x: F) -> F:
    return round_binary(x, 8, -126)


def f32_bits(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def bf16_bits_of(v) -> int:
    """bf16 pattern of a value that is exactly representable in bf16."""
    b = f32_bits(v)
    assert b & 0xFFFF == 0, "value is not a bf16"
    return b >> 16


def rint_half_even(x: F) -> int:
    s = -1 if x < 0 else 1
    return s * int(_round_to_grid(abs(x), F(1)))
