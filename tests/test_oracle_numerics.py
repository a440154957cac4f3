"""Pins for oracle/numerics.py: bf16 rounding, E4M3FN, UE8M0 exponent, fixed exp.

Each check compares the oracle with an independent computation (exact
fractions, brute-force nearest-value search, or closed forms).
"""

import bisect
import math
from fractions import Fraction as F

import numpy as np
import pytest

from exact import rn_bf16, f32_bits
from oracle import numerics as nm


def _all_finite_bf16_positive():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)  # +subnormals .. largest finite
    return bits, nm.bf16_to_f32(bits)


def test_bf16_decode_is_high_half():
    assert nm.bf16_to_f32(np.array([0x3F80], np.uint16))[0] == 1.0
    assert nm.bf16_to_f32(np.array([0xC040], np.uint16))[0] == -3.0
    assert nm.bf16_to_f32(np.array([0x0001], np.uint16))[0] == 2.0 ** -133
    assert np.isinf(nm.bf16_to_f32(np.array([0x7F80], np.uint16))[0])


def test_bf16_rn_against_exact_fractions():
    rng = np.random.default_rng(0)
    vals = list(rng.standard_normal(2000) * np.exp2(rng.integers(-140, 120, 2000)))
    # exact midpoints between neighbouring bf16 values (ties) and near-ties
    _, pos = _all_finite_bf16_positive()
    idx = rng.integers(0, len(pos) - 1, 500)
    for i in idx:
        lo, hi = float(pos[i]), float(pos[i + 1])
        mid = (lo + hi) / 2.0  # exact in float64
        vals += [mid, -mid, np.nextafter(mid, 0.0), np.nextafter(mid, np.inf)]
    vals += [0.0, 2.0 ** -134, 2.0 ** -133 * 1.5, 2.0 ** -126 * (1 - 2.0 ** -9), 1.0, -1.0]
    vals = np.array(vals, np.float64)
    got = nm.f64_to_bf16_rn(vals)
    for v, g in zip(vals, got):
        want = rn_bf16(F(float(v)))
        w_bits = f32_bits(float(want)) >> 16
        if want == 0:
            w_bits = 0x8000 if math.copysign(1.0, v) < 0 else 0
        assert int(g) == w_bits, (v, hex(int(g)), hex(w_bits))


def test_bf16_ulp_distance():
    a = np.array([0x3F80, 0x3F80, 0x0000, 0x8000, 0x8001], np.uint16)
    b = np.array([0x3F81, 0x3F7F, 0x8000, 0x0001, 0x0001], np.uint16)
    assert list(nm.bf16_ulp_distance(a, b)) == [1, 1, 0, 1, 2]


# ---------------------------------------------------------------- E4M3FN


def test_e4m3_decode_format_definition():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
             0x3C: 1.5, 0x7E: 448.0, 0x77: 240.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in table.items():
        assert nm.e4m3_decode(np.array([c]))[0] == v
    d = nm.e4m3_decode(np.array([0x80]))[0]
    assert d == 0.0 and math.copysign(1.0, d) < 0
    assert np.isnan(nm.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    # the 127 non-negative finite codes are strictly increasing
    vals = nm.e4m3_decode(np.arange(0, 0x7F))
    assert np.all(np.diff(vals) > 0)


def _reachable_encoder_inputs():
    """Every value x * 2^-e with x bf16 and |.| <= 448, down to 2^-24 (far below
    the smallest subnormal 2^-9): significand 128..255 times a power of two."""
    out = []
    for m in range(128, 256):
        for k in range(-31, 2):
            v = m * 2.0 ** k
            if v <= 448.0:
                out.append(v)
    out += [2.0 ** -40, 3 * 2.0 ** -30]
    v = np.array(sorted(set(out)), np.float64)
    return np.concatenate([v, -v, [0.0, -0.0]])


def test_e4m3_encoder_exhaustive_against_nearest_code():
    codes = np.arange(0, 0x7F)
    cvals = [F(float(x)) for x in nm.e4m3_decode(codes)]  # increasing
    inputs = _reachable_encoder_inputs()
    got = nm.e4m3_encode_rn(inputs)
    for v, g in zip(inputs, got):
        a = F(abs(float(v)))
        i = bisect.bisect_left(cvals, a)
        if i < len(cvals) and cvals[i] == a:
            c = i
        else:
            lo, hi = i - 1, i
            dlo, dhi = a - cvals[lo], cvals[hi] - a
            c = lo if dlo < dhi else hi if dhi < dlo else (lo if lo % 2 == 0 else hi)
        want = c | (0x80 if math.copysign(1.0, v) < 0 else 0)
        assert int(g) == want, (v, hex(int(g)), hex(want))


def test_e4m3_encoder_rejects_out_of_range():
    with pytest.raises(ValueError):
        nm.e4m3_encode_rn(np.array([449.0]))


# ---------------------------------------------------------------- UE8M0


def test_ue8m0_exponent_exhaustive_bf16():
    """Every positive finite bf16 absmax against the exact definition, and against
    the f32-division route RN_f32(a/448) -> ceil(log2) taken from the bits."""
    bits, a = _all_finite_bf16_positive()
    e = nm.ue8m0_exponent(a.astype(np.float64))
    # exact definition with fractions on a strided subset (all values is slow)
    for i in range(0, len(a), 37):
        av = F(float(a[i]))
        k = -140
        while F(2) ** k * 448 < av:
            k += 1
        assert max(k, -127) == e[i], (float(a[i]), e[i], k)
    # bit route in f32
    r = (a / np.float32(448.0)).astype(np.float32)
    rb = r.view(np.uint32).astype(np.int64)
    ef = (rb >> 23) & 0xFF
    fr = rb & 0x7FFFFF
    normal = ef > 0
    ceil_norm = ef - 127 + (fr != 0)
    # subnormal r = fr * 2^-149: ceil(log2) = bit_length(fr - 1) - 149
    ceil_sub = np.array([int(int(f) - 1).bit_length() - 149 for f in fr])
    e_bits = np.maximum(np.where(normal, ceil_norm, ceil_sub), -127)
    assert np.array_equal(e_bits, e)
    # invariants: 2^e >= a/448 > 2^(e-1) unless clamped
    assert np.all(np.ldexp(448.0, e) >= a)
    unclamped = e > -127
    assert np.all(np.ldexp(448.0, e[unclamped] - 1) < a[unclamped])


def test_ue8m0_zero_clamps():
    assert nm.ue8m0_exponent(np.array([0.0]))[0] == -127


# ---------------------------------------------------------------- exp


def test_exp_fixed_within_two_ulp_of_libm():
    x = np.linspace(-87.0, 88.0, 200001).astype(np.float32)
    x = np.concatenate([x, np.array([0.0, -0.0, 1.0, -1.0, 0.5, 1e-6, -1e-6], np.float32)])
    y = nm.exp_f32_fixed(x)
    ref = np.exp(x.astype(np.float64))
    ulp = np.spacing(ref.astype(np.float32)).astype(np.float64)
    err = np.abs(y.astype(np.float64) - ref) / ulp
    assert err.max() <= 2.0, err.max()
    assert nm.exp_f32_fixed(np.array([0.0], np.float32))[0] == 1.0


def test_exp_fixed_overflow_underflow():
    assert np.isinf(nm.exp_f32_fixed(np.array([89.0, 200.0], np.float32))).all()
    assert (nm.exp_f32_fixed(np.array([-110.0, -1e4], np.float32)) == 0.0).all()
    sub = nm.exp_f32_fixed(np.array([-100.0], np.float32))[0]
    assert 0 < sub < 2.0 ** -126 and abs(float(sub) - np.exp(-100.0)) <= 2.0 ** -149  # subnormal grid
