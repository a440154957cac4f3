"""Pins for oracle/int8_linear.py.

Hand-worked rows (tests/golden/int8_rows.txt), exact-fraction recomputation of
the f32 quant decision, invariants, brute-force integer GEMMs, closed forms, and
the epilogue against exactly rounded products.
"""

import os
from fractions import Fraction as F

import numpy as np
import pytest

import synthetic as syn
from exact import bf16_bits_of, f32_bits, rint_half_even, rn_bf16, rn_f32
from oracle import int8_linear as il
from oracle import numerics as nm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows():
    out = []
    for line in open(os.path.join(GOLDEN, "int8_rows.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, xs, sb, qs = [p.strip() for p in line.split("|")]
        out.append((name, [float(v) for v in xs.split()], int(sb, 16), [int(v) for v in qs.split()]))
    return out


@pytest.mark.parametrize("row", _rows(), ids=lambda r: r[0])
def test_hand_rows(row):
    name, xs, s_bits, q_want = row
    x = np.array([[bf16_bits_of(v) for v in xs]], np.uint16)
    q, s = il.quant_int8_per_token(x)
    assert int(s.view(np.uint32)[0]) == s_bits
    assert q[0].tolist() == q_want


def _exact_quant_row(xvals):
    """Quant of one row in exact rational arithmetic with explicit f32 roundings."""
    a = max(abs(F(v)) for v in xvals)
    s = rn_f32(a / 127)
    if s == 0:
        return 0, [0] * len(xvals)
    q = [max(-127, min(127, rint_half_even(rn_f32(F(v) / s)))) for v in xvals]
    return s, q


def test_quant_matches_exact_fractions_on_outlier_rows():
    x, _, _ = syn.tiny_linear()
    x2 = syn.activations((99, 1), 3, 512, outlier_frac=0.05, outlier_mul=1000.0)
    for xb in (x, x2):
        q, s = il.quant_int8_per_token(xb)
        xf = nm.bf16_to_f32(xb)
        for m in range(xb.shape[0]):
            s_ex, q_ex = _exact_quant_row([float(v) for v in xf[m]])
            assert int(s.view(np.uint32)[m]) == f32_bits(float(s_ex))
            assert q[m].tolist() == q_ex


def test_quant_invariants():
    for M in (1, 7, 64):
        x, _, _ = syn.wq_a_linear(M)
        q, s = il.quant_int8_per_token(x)
        xf = nm.bf16_to_f32(x).astype(np.float64)
        assert q.dtype == np.int8 and np.abs(q.astype(int)).max() <= 127
        assert (q != -128).all()
        a = np.abs(xf).max(axis=1)
        assert np.array_equal(s, (a.astype(np.float32) / np.float32(127)).astype(np.float32))
        # the absmax element maps to +-127 in every non-zero row
        assert (np.abs(q.astype(int)).max(axis=1)[a > 0] == 127).all()
        # sign agreement and |q - x/s| <= 1/2 (up to the f32 rounding of x/s)
        r = xf / s.astype(np.float64)[:, None]
        assert (np.sign(q) * np.sign(xf) >= 0).all()
        assert np.abs(q - r).max() <= 0.5 + 1e-5


def test_zero_row_and_mixed_rows():
    x = np.zeros((3, 64), np.uint16)
    x[1, 5] = bf16_bits_of(-4.0)
    q, s = il.quant_int8_per_token(x)
    assert s[0] == 0 and s[2] == 0 and (q[0] == 0).all() and (q[2] == 0).all()
    assert q[1, 5] == -127 and (np.delete(q[1], 5) == 0).all()


def test_half_away_rounding_would_fail_hand_row():
    # a mistake planted on the CPU: round half away from zero instead of to even
    xs = [1.0, -2.5, 0.5, 127.0]
    away = [int(np.sign(v) * np.floor(abs(v) + 0.5)) for v in xs]
    q, _ = il.quant_int8_per_token(np.array([[bf16_bits_of(v) for v in xs]], np.uint16))
    assert away != q[0].tolist()


# ---------------------------------------------------------------- GEMM


def test_gemm_bruteforce_python_ints():
    g = np.random.default_rng(3)
    for M, K, N in [(1, 16, 1), (3, 32, 5), (8, 64, 16), (5, 48, 7)]:
        q = g.integers(-127, 128, (M, K)).astype(np.int8)
        w = g.integers(-127, 128, (N, K)).astype(np.int8)
        acc = il.gemm_int8_int32(q, w)
        for m in range(M):
            for n in range(N):
                assert acc[m, n] == sum(int(q[m, k]) * int(w[n, k]) for k in range(K))


def test_gemm_closed_forms():
    K = 4096
    q = np.full((2, K), 127, np.int8)
    w = np.full((3, K), 127, np.int8)
    assert (il.gemm_int8_int32(q, w) == 16129 * K).all()
    q = np.full((1, K), -127, np.int8)
    assert (il.gemm_int8_int32(q, w) == -16129 * K).all()
    # one-hot weight columns copy a q column
    g = np.random.default_rng(4)
    q = g.integers(-127, 128, (5, 64)).astype(np.int8)
    cols = [3, 0, 63, 17]
    w = np.zeros((4, 64), np.int8)
    for n, c in enumerate(cols):
        w[n, c] = 1
    assert np.array_equal(il.gemm_int8_int32(q, w), q[:, cols].astype(np.int32))


def test_gemm_int32_bound_at_long_k():
    K = 131072
    q = np.full((1, K), 127, np.int8)
    w = np.full((1, K), 127, np.int8)
    assert il.gemm_int8_int32(q, w)[0, 0] == 16129 * K < 2 ** 31


# ---------------------------------------------------------------- epilogue


def test_epilogue_against_exact_products():
    g = np.random.default_rng(5)
    acc = g.integers(-2 ** 26, 2 ** 26, (4, 33)).astype(np.int32)
    acc[0, 0] = 0
    s = g.uniform(1e-4, 1.0, 4).astype(np.float32)
    sw = g.uniform(1e-3, 1e-2, 33).astype(np.float32)
    y = il.epilogue_bf16(acc, s, sw)
    for m in range(4):
        for n in range(33):
            want = rn_bf16(F(int(acc[m, n])) * F(float(s[m])) * F(float(sw[n])))
            wb = 0 if want == 0 else f32_bits(float(want)) >> 16
            assert int(y[m, n]) == wb, (m, n)


def test_linear_composition_and_tuple_path():
    x, w, sw = syn.tiny_linear()
    r = il.linear_w8a8(x, w, sw)
    assert r["q"].shape == (4, 256) and r["acc"].shape == (4, 512) and r["y"].shape == (4, 512)
    r2 = il.matmul_from_tuple(r["q"], r["s"], w, sw)
    assert np.array_equal(r2["acc"], r["acc"]) and np.array_equal(r2["y"], r["y"])
    # dequantised result approximates the bf16 float product
    xf = nm.bf16_to_f32(x).astype(np.float64)
    ref = xf @ (w.astype(np.float64) * sw[:, None]).T
    yf = nm.bf16_to_f32(r["y"]).astype(np.float64)
    rel = np.linalg.norm(yf - ref) / np.linalg.norm(ref)
    assert rel < 0.05
