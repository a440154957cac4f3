"""The fused decode kernel quantises a value v of a row with scale s (a normal f32, s = RN(a/127)
for the row's absmax a) by one fma, b = RN(v * inv + 384) with inv ~ 1/s, and reads the
INT8 code and a near-tie flag from b's bit pattern: w = (bits(b) + 2^14 - 128 * 2^15) << 1
holds the code in byte 2 (two's complement) and, in its low 16 bits, twice the index of
b's fraction; a zero there flags a possible near-tie, which the kernel then redoes with the
correctly rounded division.  This restates that rule on the host in exact rational
arithmetic and checks that every unflagged code equals clamp(rint(RN(v / s)), -127, 127)
(rint to even) for values on and next to every rounding tie (k + 1/2) s, at bf16 absmaxes
spread over the whole exponent range and at f32 absmaxes (rows after RMSNorm), with inv
either RN(1/s) or the Newton-refined reciprocal of an rcp one ulp either side of RN(1/s).
It uses no kernel code."""

from fractions import Fraction

import numpy as np
import pytest

_F32_TINY = np.float32(np.finfo(np.float32).tiny)


def _rn32(x: Fraction) -> np.float32:
    """Round a rational to the nearest float32, ties to even."""
    if x == 0:
        return np.float32(0.0)
    f = np.float32(float(x))  # within one ulp of the answer
    cands = [np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))]
    return min(cands, key=lambda c: (abs(Fraction(float(c)) - x), int(np.float32(c).view(np.int32)) & 1))


def _rint_even(x: Fraction) -> int:
    fl = x.numerator // x.denominator
    rem = x - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return fl


def _exact_code(v: np.float32, s: np.float32) -> int:
    """clamp(rint(RN(v / s)), -127, 127) with RN to float32 and rint to even."""
    q = _rn32(Fraction(float(v)) / Fraction(float(s)))
    return max(-127, min(127, _rint_even(Fraction(float(q)))))


def _fast_rule(v: np.float32, inv: np.float32, adj: int = 0x4000 - 0x400000):
    """(flagged, code) of the one-fma rule.  b = RN(v inv + 384) lies in [256, 512], where
    float32 has the unit 2^-15, so its pattern is 0x43800000 + round((x - 256) 2^15)."""
    x = Fraction(float(v)) * Fraction(float(inv)) + 384
    assert Fraction(256) < x < Fraction(512)
    bits = 0x43800000 + _rint_even(x * 2**15) - 256 * 2**15
    w = ((bits + adj) << 1) & 0xFFFFFFFF
    code = (w >> 16) & 0xFF
    return (w & 0xFFFF) == 0, code - 256 if code >= 128 else code


def _reciprocals(s: np.float32):
    """RN(1/s) and the Newton step r0 + r0 (1 - s r0) (two fmas) from r0 = RN(1/s) and its two
    neighbours (a one-ulp rcp)."""
    rn = np.float32(1.0) / s
    out = {float(rn)}
    for r0 in (np.nextafter(rn, np.float32(0)), rn, np.nextafter(rn, np.float32(np.inf))):
        e = _rn32(1 - Fraction(float(s)) * Fraction(float(r0)))
        out.add(float(_rn32(Fraction(float(r0)) * Fraction(float(e)) + Fraction(float(r0)))))
    return [np.float32(r) for r in sorted(out)]


def _bf16(x: float) -> np.float32:
    b = int(np.array([x], dtype=np.float32).view(np.uint32)[0])
    b = (b + 0x7FFF + ((b >> 16) & 1)) & 0xFFFF0000  # round to nearest even bf16
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def _step(t: np.float32, d: int, bf16_values: bool) -> np.float32:
    """The value d representable steps (bf16 or float32) away from a positive t."""
    b = int(np.array([t], dtype=np.float32).view(np.uint32)[0])
    b = max(0, b + (d << 16 if bf16_values else d))
    return np.array([b], dtype=np.uint32).view(np.float32)[0]


def _cases(a: np.float32, bf16_values: bool, rng):
    s = _rn32(Fraction(float(a)) / 127)
    ks = sorted(set(rng.integers(0, 127, size=10).tolist()) | {0, 1, 126})
    vals = [a, np.float32(0.0)]
    for k in ks:
        c = float(Fraction(2 * k + 1, 2) * Fraction(float(s)))
        base = _bf16(c) if bf16_values else np.float32(c)
        for d in range(-2, 3):
            v = _step(base, d, bf16_values)
            if 0 < v <= a:
                vals.append(v)
        # values whose quotient sits at the edges of the flag window (about 2^-15 from the tie)
        for e in (-2**-14, -2**-15, -1.5 * 2**-16, -2**-16, -2**-17, 2**-17, 2**-16, 1.5 * 2**-16, 2**-15, 2**-14):
            v = _rn32((Fraction(2 * k + 1, 2) + Fraction(e)) * Fraction(float(s)))
            if 0 < v <= a:
                vals.append(v)
    vals += [np.float32(x) for x in (rng.uniform(-1, 1, 6) * float(a)).astype(np.float32)]
    if bf16_values:
        vals = [_bf16(float(v)) for v in vals]
    vals = [v for v in vals if abs(v) <= a]
    return s, vals + [np.float32(-v) for v in vals]


def _absmaxes(bf16_rows: bool):
    bits = np.arange(0x0080, 0x7F80, 1531, dtype=np.uint32)  # normal bf16 values, every exponent range
    a = (bits << 16).view(np.float32)
    if not bf16_rows:
        a = a * np.float32(1.0 + 2.0**-7 + 2.0**-19)  # f32 absmaxes with low mantissa bits
    return [x for x in a if np.isfinite(x)]


@pytest.mark.parametrize("bf16_rows", [True, False])
def test_unflagged_codes_equal_the_correctly_rounded_codes(bf16_rows):
    rng = np.random.default_rng(20 + bf16_rows)
    checked = flagged = 0
    for a in _absmaxes(bf16_rows):
        s, vals = _cases(a, bf16_rows, rng)
        if not s >= _F32_TINY:
            continue  # the kernel sends a zero or subnormal scale to the exact path whole
        for inv in _reciprocals(s):
            for v in vals:
                flag, code = _fast_rule(v, inv)
                if flag:
                    flagged += 1
                    # a flag sits within 2^-14 of a rounding tie of v / s: the rule is not
                    # sending ordinary values to the slow path
                    q = Fraction(float(v)) / Fraction(float(s))
                    assert abs(abs(q) - abs(q).numerator // abs(q).denominator - Fraction(1, 2)) < Fraction(1, 2**14)
                    continue
                checked += 1
                assert code == _exact_code(v, s), (float(a), float(v), float(inv), code, _exact_code(v, s))
    # bf16 values meet the flag only at exact ties (an absmax with mantissa 0x7E) and tiny
    # quotients; the f32 values near the ties are flagged in bulk
    assert checked > 2000 and flagged > (0 if bf16_rows else 200), (checked, flagged)


def test_exact_ties_are_flagged():
    """Where v / s is exactly a half-integer (an absmax with mantissa 0x7E makes (k + 1/2) s a
    bf16 value), RN(v / s) is that half-integer and the code depends on rint's tie rule: the
    rule must not decide it."""
    a = np.float32(1.984375 * 2.0**3)  # mantissa 0x7E
    s = _rn32(Fraction(float(a)) / 127)
    hits = 0
    for k in range(127):
        v = Fraction(2 * k + 1, 2) * Fraction(float(s))
        if Fraction(float(_bf16(float(v)))) != v:
            continue
        for inv in _reciprocals(s):
            assert _fast_rule(np.float32(float(v)), inv)[0]
            hits += 1
    assert hits > 20


def test_a_rule_without_the_rounding_offset_fails():
    """Planted mistake: dropping the + 2^14 (so byte 2 holds floor instead of the nearest
    integer) must disagree with the exact codes on these cases."""
    rng = np.random.default_rng(7)
    wrong = 0
    for a in _absmaxes(True)[::4]:
        s, vals = _cases(a, True, rng)
        if not s >= _F32_TINY:
            continue
        inv = np.float32(1.0) / s
        for v in vals:
            flag, code = _fast_rule(v, inv, adj=-0x400000)
            wrong += (not flag) and code != _exact_code(v, s)
    assert wrong > 0
