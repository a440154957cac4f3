"""Two kernels divide a bf16 absmax a by a constant d without a division instruction:
m = RN(a * c) with c = RN(1/d), then q = fma(fma(-d, m, a), c, m).  The fused decode kernel
takes the per-token INT8 scale RN(a/127) this way, the FP8 group quant the UE8M0 exponent's
quotient RN(a/448).  This checks, with exact rational arithmetic, that the formula equals
the correctly rounded quotient for every non-negative finite bf16 value a (the absmax is
one of the bf16 inputs).  Test of an arithmetic identity the kernels rely on; it uses no
kernel code."""

from fractions import Fraction

import numpy as np
import pytest


def _rn32(x: Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even."""
    if x == 0:
        return np.float32(0.0)
    f = np.float32(float(x))  # within one ulp of the answer
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.int32)) & 1))


@pytest.mark.parametrize("d", [127, 448])
def test_corrected_product_is_the_correctly_rounded_quotient_for_every_bf16(d):
    c = np.float32(1.0) / np.float32(d)
    fc = Fraction(float(c))
    bits = np.arange(0, 0x7F80, dtype=np.uint32)  # +0, subnormals, normals below inf
    a_all = (bits << 16).view(np.float32)
    want = a_all / np.float32(d)  # IEEE float32 division: correctly rounded
    m_all = a_all * c             # IEEE float32 product: correctly rounded
    for a, m, q in zip(a_all, m_all, want):
        fa, fm = Fraction(float(a)), Fraction(float(m))
        r = _rn32(fa - d * fm)                   # fma(-d, m, a)
        s = _rn32(Fraction(float(r)) * fc + fm)  # fma(r, c, m)
        assert s == q, (d, hex(int(np.float32(a).view(np.uint32))), float(s), float(q))


@pytest.mark.parametrize("d", [127, 448])
def test_plain_product_is_not_enough(d):
    """Without the correction step the product misses the quotient for some bf16 values,
    so the step is needed."""
    bits = np.arange(0, 0x7F80, dtype=np.uint32)
    a = (bits << 16).view(np.float32)
    assert np.any(a * (np.float32(1.0) / np.float32(d)) != a / np.float32(d))


def test_the_kernel_constant_is_the_rounded_reciprocal():
    """The FP8 group quant's literal for RN(1/448) is that float32 (bits 0x3B124925)."""
    assert int((np.float32(1.0) / np.float32(448)).view(np.uint32)) == 0x3B124925
