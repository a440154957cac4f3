"""Oracle for the W8A8 MoE expert block.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows:
* "DeepSeek-V4 W8A8 性能分析" section 五: each expert e has its own weights and
  its own row count M_e; expert_tokens goes to the grouped matmul as
  group_list; DeepSeek-V4-Flash expert shapes W13 K=4096 N=4096 (gate and up)
  and W2 K=2048 N=4096;
* "DeepSeek V4 950 低精度优化全复盘" section 2.3 (RMSNorm fused with quant in
  registers, written back in low precision; SwiGLU fused with quant so the
  activation is not written back in high precision) and section 3.2 (sort the
  tokens by expert id before dispatch so each expert's rows are contiguous).

Readings where the pages are silent (listed in the design doc):
* sort: stable by expert id over the flattened (token, slot) pairs, so ties keep
  token-then-slot order; offsets is the exclusive prefix sum of per-expert counts;
* RMSNorm: v = (x * inv) * gamma with inv = 1 / sqrt(mean(x^2) + eps), eps = 1e-6,
  gamma bf16; the sum of squares is taken in float64 (exactly rounded here),
  mean and eps in f32, sqrt and the division correctly rounded in f32, v is not
  rounded to bf16 before the per-token INT8 quant.  The page fixes no summation
  order, so a row whose f32 mean square another float64 order could round to the
  neighbouring f32 value is flagged, and both readings are accepted for it;
* gate = first half of W13's output columns, up = second half;
  g = (f32(acc) * s) * sw and likewise u, silu(g) = g / (1 + exp(-g)) with the
  fixed-sequence f32 exp, h = silu(g) * u in f32 (not rounded to bf16), then the
  per-token INT8 quant of h and the W2 GEMM with the bf16 epilogue;
* the block returns the rows in sorted order plus the permutation; the combine
  back to token order is a separate step.
"""

from __future__ import annotations

import math

import numpy as np

from .int8_linear import epilogue_bf16, gemm_int8_int32, quant_int8_per_token
from .numerics import bf16_to_f32, exp_f32_fixed

RMS_EPS = np.float32(1e-6)


def expert_sort(topk_ids: np.ndarray, num_experts: int, drop_invalid: bool = False):
    """(perm, offsets): perm[r] = flattened pair index t*TOPK + slot of sorted row r;
    rows of expert e are perm[offsets[e]:offsets[e+1]].  With drop_invalid, pairs whose id
    is outside [0, E) take no row (offsets[E] counts the kept pairs and perm holds only
    them); without it such an id is an error."""
    ids = np.asarray(topk_ids).reshape(-1).astype(np.int64)
    ok = (ids >= 0) & (ids < num_experts)
    if not drop_invalid and not ok.all():
        raise ValueError("expert id out of range")
    kept = np.flatnonzero(ok)
    perm = kept[np.argsort(ids[kept], kind="stable")].astype(np.int32)
    counts = np.bincount(ids[kept], minlength=num_experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return perm, offsets


def _mean_square_f32(ss: float, K: int) -> np.float32:
    return np.float32(ss / K)


def rmsnorm_mean_squares(x_bits: np.ndarray):
    """Per row: (ms, ms_other, flagged).

    ms = f32(ss / K) with ss the exactly rounded float64 sum of the squares.  A kernel that
    sums the same float64 squares in another order lands within K 2^-53 ss of the exact sum
    (all terms are positive: the error of a recursive or pairwise sum of n positive terms is at
    most (n - 1) u times the sum), and its own f64 division by K adds one more rounding.  When
    the f32 mean square of some value in that interval differs from ms, the row is flagged and
    ms_other is that other f32 neighbour (else ms_other = ms): both are correct readings of a
    float64 sum of squares."""
    xf = bf16_to_f32(x_bits)
    M, K = xf.shape
    ms = np.empty(M, np.float32)
    other = np.empty(M, np.float32)
    delta = (K + 2) * 2.0 ** -53
    for m in range(M):
        ss = math.fsum(float(v) * float(v) for v in xf[m])  # exactly rounded float64 sum
        ms[m] = _mean_square_f32(ss, K)
        lo = _mean_square_f32(ss * (1.0 - delta), K)
        hi = _mean_square_f32(ss * (1.0 + delta), K)
        other[m] = lo if lo != ms[m] else hi
    return ms, other, other != ms


def _rmsnorm_from_ms(xf, gf, ms, eps):
    d = (ms + np.float32(eps)).astype(np.float32)
    r = np.sqrt(d).astype(np.float32)  # correctly rounded f32 sqrt
    inv = (np.float32(1.0) / r).astype(np.float32)
    v = (xf * inv[:, None]).astype(np.float32)
    return (v * gf[None, :]).astype(np.float32)


def rmsnorm_f32(x_bits: np.ndarray, gamma_bits: np.ndarray, eps=RMS_EPS, alternates: bool = False):
    """v = (x * inv) * gamma in f32 with inv = 1 / sqrt(f32(ss / K) + eps), per row.

    With alternates=True returns (v, v_other, flagged): v_other recomputes the flagged rows
    (rmsnorm_mean_squares) with the other f32 mean square, and equals v elsewhere."""
    xf = bf16_to_f32(x_bits)
    gf = bf16_to_f32(gamma_bits)
    ms, other, flagged = rmsnorm_mean_squares(x_bits)
    v = _rmsnorm_from_ms(xf, gf, ms, eps)
    if not alternates:
        return v
    return v, _rmsnorm_from_ms(xf, gf, other, eps), flagged


def silu_mul_f32(acc: np.ndarray, s: np.ndarray, sw: np.ndarray) -> np.ndarray:
    """h = silu(g) * u from the gate/up accumulators of one or more rows.

    acc [R, 2I] int32, s [R] f32, sw [R, 2I] f32 (the row's expert's channel
    scales).  g, u = (f32(acc) * s) * sw split at I; silu(g) = g / (1 + exp(-g)).
    """
    R, N2 = acc.shape
    I = N2 // 2
    af = acc.astype(np.float32)  # int32 -> f32, nearest
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        val = ((af * s[:, None].astype(np.float32)).astype(np.float32) * sw.astype(np.float32)).astype(np.float32)
        g, u = val[:, :I], val[:, I:]
        e = exp_f32_fixed((-g).astype(np.float32))
        den = (np.float32(1.0) + e).astype(np.float32)
        sg = (g / den).astype(np.float32)
        return (sg * u).astype(np.float32)


def moe_block(h_bits, gamma_bits, topk_ids, w13, sw13, w2, sw2, *, eps=RMS_EPS, keep=False, v_rows=None):
    """The whole block.  Shapes: h [T, H] bf16 bits; gamma [H]; topk_ids [T, TOPK];
    w13 int8 [E, 2I, H] (rows = output channels); sw13 f32 [E, 2I]; w2 int8 [E, H, I];
    sw2 f32 [E, H].  Returns a dict with perm, offsets, y (bf16 bits [T*TOPK, H],
    sorted rows) and, with keep=True, every intermediate.  v_rows, when given, replaces
    the RMSNorm output per token (the other reading of a flagged row)."""
    T, H = h_bits.shape
    E = w13.shape[0]
    TOPK = topk_ids.shape[1]
    perm, offsets = expert_sort(topk_ids, E)
    tok = perm // TOPK
    v = rmsnorm_f32(h_bits, gamma_bits, eps) if v_rows is None else v_rows  # per token; row r uses token tok[r]
    q1, s1 = quant_int8_per_token(v[tok], is_bf16_bits=False)
    R = T * TOPK
    I = w13.shape[1] // 2
    acc13 = np.zeros((R, 2 * I), np.int32)
    hmid = np.zeros((R, I), np.float32)
    y = np.zeros((R, w2.shape[1]), np.uint16)
    q2 = np.zeros((R, I), np.int8)
    s2 = np.zeros(R, np.float32)
    acc2 = np.zeros((R, w2.shape[1]), np.int32)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        acc13[lo:hi] = gemm_int8_int32(q1[lo:hi], w13[e])
        hmid[lo:hi] = silu_mul_f32(acc13[lo:hi], s1[lo:hi], np.broadcast_to(sw13[e], (hi - lo, 2 * I)))
    q2[:], s2[:] = quant_int8_per_token(hmid, is_bf16_bits=False)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        acc2[lo:hi] = gemm_int8_int32(q2[lo:hi], w2[e])
        y[lo:hi] = epilogue_bf16(acc2[lo:hi], s2[lo:hi], sw2[e])
    out = {"perm": perm, "offsets": offsets, "y": y}
    if keep:
        out.update(q1=q1, s1=s1, acc13=acc13, h=hmid, q2=q2, s2=s2, acc2=acc2, v=v)
    return out
