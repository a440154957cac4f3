"""Oracle for the INT8 W8A8 dynamic linear  Y = dequant(quant(X) . W).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows "DeepSeek-V4 W8A8 性能分析" section 一: a dense linear Y = X W with
X [M, K], W [K, N], Y [M, N]; the W8A8_DYNAMIC chain turns BF16 X into an INT8
payload plus a per-token scale (npu_dynamic_quant), runs the quant matmul, and
returns BF16 Y; a Linear may instead receive the (INT8 payload, scale) tuple
from an upstream fused producer and skip its own quantisation.

Readings where the page is silent (each listed in the design doc):
* scale s_m = RN_f32(absmax_m / 127), stored as f32; the page fixes an fp32
  per-token scale, so the code decision q = rint(x / s) is taken in f32 with a
  correctly rounded division and round-to-nearest-even;
* codes are symmetric, clamped to [-127, 127];
* an all-zero row gives s = 0 and q = 0;
* weights arrive pre-quantised: int8 stored [N, K] (K contiguous) with one f32
  scale per output channel n; there is no bias;
* the epilogue value acc * s_m * sw_n is rounded once to BF16.
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32, f64_to_bf16_rn

QMAX = 127


def quant_int8_per_token(x: np.ndarray, *, is_bf16_bits: bool = True):
    """Per-token dynamic INT8 quantisation.

    x: [M, K] bf16 bit patterns (uint16), or f32 values when is_bf16_bits=False.
    Returns (q int8 [M, K], s f32 [M]).

    a_m = max_k |x[m, k]|          (exact in f32)
    s_m = RN_f32(a_m / 127)
    q   = clamp(rint(RN_f32(x / s_m)), -127, 127), or 0 when a_m = 0
    """
    xf = bf16_to_f32(x) if is_bf16_bits else np.asarray(x, dtype=np.float32)
    if xf.ndim != 2:
        raise ValueError("x must be 2-D [M, K]")
    M, K = xf.shape
    a = np.max(np.abs(xf), axis=1) if K > 0 else np.zeros(M, np.float32)
    a = a.astype(np.float32)
    s = (a / np.float32(QMAX)).astype(np.float32)
    safe = np.where(s > 0, s, np.float32(1.0)).astype(np.float32)
    ratio = (xf / safe[:, None]).astype(np.float32)  # f32 division, correctly rounded
    q = np.clip(np.rint(ratio), -QMAX, QMAX)
    q = np.where((s > 0)[:, None], q, 0.0)
    return q.astype(np.int8), s


def gemm_int8_int32(q: np.ndarray, w_nk: np.ndarray) -> np.ndarray:
    """acc[m, n] = sum_k q[m, k] * W[k, n] with W stored as w_nk[n, k].

    Every product and partial sum is an integer below 2^53 in magnitude
    (|acc| <= K * 127 * 127 and K <= 131072), so the float64 matrix product is
    exact whatever order it sums in.  The result must fit int32.
    """
    q = np.asarray(q)
    w_nk = np.asarray(w_nk)
    K = q.shape[1]
    if w_nk.shape[1] != K:
        raise ValueError("K mismatch")
    if K > 131072:
        raise ValueError("K above the exact-int32 bound")
    acc = q.astype(np.float64) @ w_nk.astype(np.float64).T
    acc_i = acc.astype(np.int64)
    assert np.all(acc_i == acc)
    assert np.all(np.abs(acc_i) < 2 ** 31)
    return acc_i.astype(np.int32)


def epilogue_bf16(acc: np.ndarray, s: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """y[m, n] = RN_bf16(acc[m, n] * s_m * sw_n); returns bf16 bit patterns.

    For K <= 8192, |acc| < 2^27 and acc * s_m (s has 24 significant bits) is
    exact in float64, so only the second product rounds before the bf16
    rounding; for longer K each float64 rounding adds at most 2^-53 relative,
    far below the 2^-9 half-ulp of bf16.
    """
    acc = np.asarray(acc, dtype=np.float64)
    v = (acc * np.asarray(s, np.float64)[:, None]) * np.asarray(sw, np.float64)[None, :]
    return f64_to_bf16_rn(v)


def linear_w8a8(x_bits: np.ndarray, w_nk: np.ndarray, w_scale: np.ndarray):
    """The whole chain: BF16 X -> (q, s) -> acc -> BF16 Y.

    Returns a dict with q, s, acc and y (bf16 bits), so every intermediate can be
    compared bit for bit.
    """
    q, s = quant_int8_per_token(x_bits)
    acc = gemm_int8_int32(q, w_nk)
    y = epilogue_bf16(acc, s, w_scale)
    return {"q": q, "s": s, "acc": acc, "y": y}


def matmul_from_tuple(q: np.ndarray, s: np.ndarray, w_nk: np.ndarray, w_scale: np.ndarray):
    """The tuple-reuse path: an upstream producer already gave (q, s)."""
    acc = gemm_int8_int32(q, w_nk)
    return {"acc": acc, "y": epilogue_bf16(acc, s, w_scale)}
