"""Number formats used by the W8A8 / FP8 hot path, written from their definitions.

TEST INFRASTRUCTURE ONLY (see the package docstring).  No HIP code shares
anything with this module.

bfloat16
    1 sign bit, 8 exponent bits (bias 127), 7 fraction bits: the top half of an
    IEEE binary32.  Decoding is a 16-bit shift; encoding rounds to nearest, ties
    to even, from the exact value.

E4M3FN (OCP 8-bit float, the ``float8_e4m3fn`` the SGLang wrapper allocates in
PR #34277's fp8_wo_a.py snippet)
    1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent field 0 holds
    subnormals k * 2^-9; no infinities; S.1111.111 is NaN, so the largest finite
    magnitude is 1.75 * 2^8 = 448.

UE8M0
    An unsigned 8-bit biased exponent (bias 127) that stands for the power of
    two 2^(byte-127).  PR #34277 (实现拆解 item 1) writes one such byte per
    128-wide hidden group.

exp
    SiLU needs exp.  Library exp functions differ between the host libm and the
    device by an ulp now and then, which would flip INT8 requantisation codes, so
    the method's exp is read as one fixed f32 operation sequence: Cody-Waite
    reduction x = n*ln2 + r with ln2 split into a 9-bit head and a tail, a
    degree-7 Taylor polynomial for e^r in Horner form, then scaling by 2^n.  Every
    step is one correctly rounded f32 operation, with no fused multiply-add.
"""

from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------
# bfloat16
# ----------------------------------------------------------------------------


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact bf16 -> f32: the 16 stored bits are the high half of the f32."""
    b = np.asarray(bits).astype(np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def f64_to_bf16_rn(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bfloat16 (nearest, ties to even); returns uint16 bits.

    Normal range (|x| >= 2^-126): keep 8 significant bits.  Below it the grid is
    the subnormal step 2^-133.  Values that round past the largest finite bf16
    become infinity.  The sign of zero is kept.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)  # x = m * 2^e, 0.5 <= |m| < 1
    normal = np.abs(x) >= 2.0 ** -126
    # normal: round m * 2^8 (an exact float64) to an integer, ties to even
    r_norm = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    # subnormal grid 2^-133
    r_sub = np.ldexp(np.rint(np.ldexp(x, 133)), -133)
    r = np.where(normal, r_norm, r_sub)
    r = np.copysign(r, x)  # rint keeps the sign of zero; copysign makes it explicit
    with np.errstate(over="ignore"):
        f = r.astype(np.float32)  # exact: r is on the bf16 grid, or overflows to inf
    return (f.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def bf16_ulp_distance(a_bits: np.ndarray, b_bits: np.ndarray) -> np.ndarray:
    """Distance between two bf16 bit patterns in units in the last place.

    Maps the sign-magnitude patterns onto a monotonic integer line (so +0 and -0
    are both 0) and subtracts.
    """

    def line(b):
        b = np.asarray(b).astype(np.int64)
        mag = b & 0x7FFF
        return np.where(b & 0x8000, -mag, mag)

    return np.abs(line(a_bits) - line(b_bits))


# ----------------------------------------------------------------------------
# E4M3FN
# ----------------------------------------------------------------------------

E4M3_MAX = 448.0
E4M3_BIAS = 7


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """E4M3FN byte -> float64 value (NaN for S.1111.111)."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    ef = (c >> 3) & 0xF
    fr = c & 0x7
    val = np.where(
        ef == 0,
        np.ldexp(fr.astype(np.float64), -9),  # subnormal: fr * 2^-9
        np.ldexp((8 + fr).astype(np.float64), ef - E4M3_BIAS - 3),  # (1 + fr/8) * 2^(ef-7)
    )
    val = np.where((ef == 0xF) & (fr == 0x7), np.nan, val)
    return sign * val


def e4m3_encode_rn(v: np.ndarray) -> np.ndarray:
    """Encode finite values with |v| <= 448 to E4M3FN, nearest, ties to even.

    The caller guarantees the range (the group scale makes |x * 2^-e| <= 448), so
    saturation never comes into play; larger inputs raise.
    """
    v = np.asarray(v, dtype=np.float64)
    if np.any(~np.isfinite(v)) or np.any(np.abs(v) > E4M3_MAX):
        raise ValueError("E4M3 encoder input out of range")
    sign = np.signbit(v).astype(np.int64) << 7
    a = np.abs(v)
    m, e = np.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    E = e - 1  # a = (2m) * 2^E with 2m in [1, 2)
    normal = a >= 2.0 ** -6
    # normal: 3 fraction bits -> round (2m) * 8 in [8, 16]
    r = np.rint(np.ldexp(m, 4)).astype(np.int64)  # (2m)*8 = m*16
    carry = r == 16
    E = np.where(carry, E + 1, E)
    r = np.where(carry, 8, r)
    code_norm = ((E + E4M3_BIAS) << 3) | (r - 8)
    # subnormal: multiples of 2^-9; a result of 8 is the smallest normal 0x08
    code_sub = np.rint(np.ldexp(a, 9)).astype(np.int64)
    code = np.where(normal, code_norm, code_sub)
    if np.any((code & 0x7F) == 0x7F):
        raise ValueError("E4M3 encoder produced NaN code")
    return (code | sign).astype(np.uint8)


# ----------------------------------------------------------------------------
# UE8M0 group exponent
# ----------------------------------------------------------------------------

UE8M0_MIN_EXP = -127


def ue8m0_exponent(absmax: np.ndarray) -> np.ndarray:
    """Smallest integer e with 2^e >= absmax / 448, clamped below at -127.

    This is the power-of-two group scale: x * 2^-e then lies within the E4M3
    range.  Computed with exact float64 comparisons (448 * 2^e is exact), never
    with a log.  absmax = 0 gives the clamp value -127 (byte 0).
    """
    a = np.asarray(absmax, dtype=np.float64)
    if np.any(a < 0) or np.any(~np.isfinite(a)):
        raise ValueError("absmax must be finite and >= 0")
    pos = a > 0
    safe = np.where(pos, a, 1.0)
    _, ea = np.frexp(safe)  # safe in [2^(ea-1), 2^ea)
    e = ea - 9  # first guess: 448 < 2^9
    # adjust with exact comparisons until 448*2^(e-1) < a <= 448*2^e
    for _ in range(4):
        too_small = np.ldexp(448.0, e) < safe
        e = np.where(too_small, e + 1, e)
    for _ in range(4):
        too_big = np.ldexp(448.0, e - 1) >= safe
        e = np.where(too_big, e - 1, e)
    assert np.all(np.ldexp(448.0, e) >= safe) and np.all(np.ldexp(448.0, e - 1) < safe)
    e = np.where(pos, e, UE8M0_MIN_EXP)
    return np.maximum(e, UE8M0_MIN_EXP).astype(np.int64)


# ----------------------------------------------------------------------------
# The fixed-sequence f32 exp used inside SiLU
# ----------------------------------------------------------------------------

_F = np.float32
LOG2E_F = _F(1.4426950408889634)
LN2_HI_F = _F(0.693359375)  # 355/512: 9 significant bits, so n*LN2_HI is exact for |n| <= 2^15
LN2_LO_F = _F(0.6931471805599453 - 0.693359375)
# 1/k! for k = 0..7, each rounded to f32
EXP_POLY_F = [_F(1.0), _F(1.0), _F(0.5), _F(1.0 / 6.0), _F(1.0 / 24.0), _F(1.0 / 120.0),
              _F(1.0 / 720.0), _F(1.0 / 5040.0)]


def exp_f32_fixed(x: np.ndarray) -> np.ndarray:
    """exp(x) for f32 x by one fixed sequence of correctly rounded f32 operations.

    n = rint(x * log2e); if n > 128 the result is +inf, if n < -151 it is +0.
    r = (x - n*LN2_HI) - n*LN2_LO; p = Horner(1/7!, ..., 1/1!, 1/0!) at r;
    result = p * 2^n rounded once (ldexp).
    """
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        t = (x * LOG2E_F).astype(np.float32)
        n = np.rint(t).astype(np.float32)
        hi = (n * LN2_HI_F).astype(np.float32)
        lo = (n * LN2_LO_F).astype(np.float32)
        r = ((x - hi).astype(np.float32) - lo).astype(np.float32)
        p = EXP_POLY_F[7]
        for k in range(6, -1, -1):
            p = ((p * r).astype(np.float32) + EXP_POLY_F[k]).astype(np.float32)
        ni = np.clip(n, -200, 200).astype(np.int32)
        y = np.ldexp(p, ni).astype(np.float32)
        y = np.where(n > 128, np.float32(np.inf), y)
        y = np.where(n < -151, np.float32(0.0), y)
    return y.astype(np.float32)
