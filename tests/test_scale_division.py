"""The fused decode kernel derives the per-token scale s = RN(absmax/127) of bf16 rows without
a division: m = RN(a * c) with c = RN(1/127), then s = fma(fma(-127, m, a), c, m).  This
checks, with exact rational arithmetic, that the formula equals the correctly rounded
quotient for every non-negative finite bf16 value a (the kernel's absmax is one of the row's
bf16 values).  Test of an arithmetic identity the kernel relies on; it uses no kernel code."""

from fractions import Fraction

import numpy as np


def _rn32(x: Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even."""
    if x == 0:
        return np.float32(0.0)
    f = np.float32(float(x))  # within one ulp of the answer
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.int32)) & 1))


def test_div127_formula_is_the_correctly_rounded_quotient_for_every_bf16():
    c = np.float32(1.0) / np.float32(127.0)
    fc = Fraction(float(c))
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # +0, subnormals, normals below inf
    a_all = (bits << 16).view(np.float32)
    want = a_all / np.float32(127.0)  # IEEE float32 division: correctly rounded
    m_all = a_all * c                 # IEEE float32 product: correctly rounded
    for a, m, q in zip(a_all, m_all, want):
        fa, fm = Fraction(float(a)), Fraction(float(m))
        r = _rn32(fa - 127 * fm)             # fma(-127, m, a)
        s = _rn32(Fraction(float(r)) * fc + fm)  # fma(r, c, m)
        assert s == q, (hex(int(np.float32(a).view(np.uint32))), float(s), float(q))


def test_plain_product_is_not_enough():
    """Without the correction step the product misses the quotient for some bf16 values,
    so the step is needed."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    a = (bits << 16).view(np.float32)
    assert np.any(a * (np.float32(1.0) / np.float32(127.0)) != a / np.float32(127.0))
