"""Oracle for the per-token-group FP8 quant, its packed UE8M0 scales, and the
grouped FP8 contraction that consumes them.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Follows the SGLang PR #34277 summary (prhub.com.cn):
* 功能与动机: the DSV4 wo_a quant kernel emits the packed UE8M0 int32 scale
  layout the downstream FP8 einsum reads, instead of fp32 scales that a
  separate transpose-and-pack kernel converts before every einsum;
* 实现拆解 item 1 and the kernel write-logic snippet: 4 UE8M0 bytes per int32;
  hidden group h goes to pack h // 4, byte h % 4; the physical layout is
  [outer group g, packed hidden, aligned token] with the token index contiguous
  and padded to a multiple of 4, word offset (g * PH + h // 4) * TA + t; when the
  last hidden group is written, the rest of its pack is zeroed;
* 实现拆解 item 2 and the wrapper snippet: x [T, G, D], hidden groups D / 128,
  PH = ceil((D / 128) / 4), TA = ceil(T / 4) * 4, payload float8_e4m3fn shaped
  like x, int32 storage [G, PH, TA], a launch only when x has elements, and the
  logical view [T, G, PH] obtained by two transposes and a token slice;
* 实现拆解 item 3: packed and fp32 scales must give bit-identical einsum output.

Readings where the page is silent (listed in the design doc):
* the group exponent is the smallest e with 2^e >= absmax / 448 (the E4M3
  maximum), clamped below at -127; the UE8M0 byte is e + 127;
* the payload is E4M3FN(x * 2^-e), nearest, ties to even; the sign of zero is kept;
* the token-padding words t in [T, TA) are zero (the page leaves them
  uninitialised and hides them behind the slice; zeroing makes the whole storage
  comparable);
* D must be a multiple of 128;
* the contraction out[t, g, n] = sum_k x[t, g, k] * W_g[n, k] uses per-(t, g, 128-k
  block) activation scales and per-(g, 128-n block, 128-k block) power-of-two
  weight scales, accumulates in float and rounds once to bf16.

The MX-like variant follows "重塑大模型推理数据流：DeepSeek V4 950 低精度优化全复盘",
section 2.1: every 32 consecutive elements share one 8-bit (UE8M0) scale, with E4M3
values.  Readings (listed in the design doc): the per-block exponent is the same rule as
above with 32-element groups; the bytes use the same packed layout (hidden groups
D / 32); the weights carry one power-of-two scale per (output column, 32-deep K
block); the contraction scales each 32-term block sum by both scales.
"""

from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f32, e4m3_decode, e4m3_encode_rn, f64_to_bf16_rn, ue8m0_exponent

GROUP = 128  # elements sharing one UE8M0 exponent (the wo_a quant of the PR)
MX_GROUP = 32  # elements sharing one scale in the MX-like block scaling
PER_PACK = 4  # UE8M0 bytes per int32 word


def layout_dims(T: int, D: int, group: int = GROUP):
    """(HG, PH, TA): hidden groups, packed hidden words, 4-aligned token count."""
    if D % group:
        raise ValueError(f"D must be a multiple of {group}")
    HG = D // group
    PH = (HG + PER_PACK - 1) // PER_PACK
    TA = (T + PER_PACK - 1) // PER_PACK * PER_PACK
    return HG, PH, TA


def group_quant_fp8(x_bits: np.ndarray, group: int = GROUP):
    """x [T, G, D] bf16 bits -> (payload uint8 E4M3FN [T, G, D], exponent bytes uint8 [T, G, HG]),
    one exponent per `group` consecutive elements (128, or 32 for the MX-like blocks)."""
    x_bits = np.asarray(x_bits)
    T, G, D = x_bits.shape
    HG, _, _ = layout_dims(T, D, group)
    xf = bf16_to_f32(x_bits).astype(np.float64).reshape(T, G, HG, group)
    a = np.max(np.abs(xf), axis=-1) if T > 0 else np.zeros((0, G, HG))
    e = ue8m0_exponent(a)  # [T, G, HG]
    scaled = np.ldexp(xf, -e[..., None])  # exact power-of-two scaling in float64
    payload = e4m3_encode_rn(scaled).reshape(T, G, D)
    ebyte = (e + 127).astype(np.uint8)
    return payload, ebyte


def pack_ue8m0(ebyte: np.ndarray) -> np.ndarray:
    """Exponent bytes [T, G, HG] -> int32 storage [G, PH, TA].

    Byte h of token t, outer group g lands at byte h % 4 of word
    (g * PH + h // 4) * TA + t (little-endian: byte j is bits 8j..8j+7).  Every
    byte not written this way is zero.
    """
    T, G, HG = ebyte.shape
    PH = (HG + PER_PACK - 1) // PER_PACK
    TA = (T + PER_PACK - 1) // PER_PACK * PER_PACK
    flat = np.zeros(G * PH * TA * PER_PACK, dtype=np.uint8)
    t, g, h = np.meshgrid(np.arange(T), np.arange(G), np.arange(HG), indexing="ij")
    word = (g * PH + h // PER_PACK) * TA + t
    flat[word * PER_PACK + h % PER_PACK] = ebyte[t, g, h]
    return flat.view("<i4").reshape(G, PH, TA)


def logical_view(storage: np.ndarray, T: int) -> np.ndarray:
    """The [T, G, PH] view of storage [G, PH, TA]: transpose, slice, transpose."""
    return storage.transpose(0, 2, 1)[:, :T, :].transpose(1, 0, 2)


def unpack_ue8m0(storage: np.ndarray, T: int, HG: int) -> np.ndarray:
    """Inverse of pack_ue8m0 on the valid region: storage -> exponent bytes [T, G, HG]."""
    G, PH, TA = storage.shape
    b = np.ascontiguousarray(storage).view(np.uint8).reshape(G, PH, TA, PER_PACK)
    out = np.zeros((T, G, HG), dtype=np.uint8)
    for h in range(HG):
        out[:, :, h] = b[:, h // PER_PACK, :T, h % PER_PACK].T
    return out


def group_quant_fp8_packed(x_bits: np.ndarray, group: int = GROUP):
    """The whole producer: payload [T, G, D] and packed int32 storage [G, PH, TA]."""
    payload, ebyte = group_quant_fp8(x_bits, group)
    return payload, pack_ue8m0(ebyte), ebyte


def fp8_grouped_contraction(xq: np.ndarray, x_scale_f: np.ndarray, wq: np.ndarray, w_scale: np.ndarray,
                            *, return_abs: bool = False):
    """out[t, g, n] = sum over 128-wide k blocks kb of
         x_scale_f[t, g, kb] * w_scale[g, n // 128, kb] * sum_{k in kb} x[t, g, k] * W_g[n, k]

    xq: E4M3FN codes [T, G, D]; x_scale_f: float scales [T, G, D/128]
    (powers of two); wq: E4M3FN codes [G, N, D]; w_scale: f32 [G, N/128, D/128].

    Each 128-term block sum of E4M3 x E4M3 products is exact in float64 (each
    product has at most 8 significant bits, magnitudes within [2^-18, 2^18), so
    a 128-term sum needs at most 44 bits).  The 32 scaled block sums are added in
    float64 in block order and rounded once to bf16.  With return_abs, also
    returns S = sum of |scaled products| per output, the scale of the f32
    accumulation error the GPU may add.
    """
    T, G, D = xq.shape
    Gw, N, Dw = wq.shape
    assert Gw == G and Dw == D and D % GROUP == 0 and N % GROUP == 0
    HG = D // GROUP
    xv = e4m3_decode(xq).reshape(T, G, HG, GROUP)
    wv = e4m3_decode(wq).reshape(G, N, HG, GROUP)
    out = np.zeros((T, G, N), dtype=np.float64)
    sabs = np.zeros((T, G, N), dtype=np.float64)
    wsc = np.repeat(np.asarray(w_scale, np.float64), GROUP, axis=1)  # [G, N, HG]
    for g in range(G):
        for kb in range(HG):
            blk = xv[:, g, kb, :] @ wv[g, :, kb, :].T  # [T, N], exact
            sc = np.asarray(x_scale_f, np.float64)[:, g, kb][:, None] * wsc[g, :, kb][None, :]
            out[:, g, :] += blk * sc
            if return_abs:
                sabs[:, g, :] += (np.abs(xv[:, g, kb, :]) @ np.abs(wv[g, :, kb, :]).T) * sc
    y = f64_to_bf16_rn(out)
    return (y, sabs) if return_abs else y


def ebyte_to_scale(ebyte: np.ndarray) -> np.ndarray:
    """UE8M0 bytes -> float64 powers of two 2^(byte - 127)."""
    return np.ldexp(1.0, np.asarray(ebyte).astype(np.int64) - 127)


def contraction_from_packed(xq, storage, T, wq, w_scale, **kw):
    """Contraction reading the activation scales from the packed int32 storage."""
    HG = xq.shape[2] // GROUP
    return fp8_grouped_contraction(xq, ebyte_to_scale(unpack_ue8m0(storage, T, HG)), wq, w_scale, **kw)


def mx_contraction(xq: np.ndarray, x_scale_f: np.ndarray, wq: np.ndarray, w_scale: np.ndarray,
                   *, return_abs: bool = False):
    """The contraction with MX-like 32-element blocks on both operands:
         out[t, g, n] = sum over 32-deep k blocks kb of
             x_scale_f[t, g, kb] * w_scale[g, n, kb] * sum_{k in kb} x[t, g, k] * W_g[n, k]

    xq: E4M3FN codes [T, G, D]; x_scale_f: powers of two [T, G, D/32]; wq: E4M3FN codes
    [G, N, D]; w_scale: powers of two [G, N, D/32].  Each 32-term block sum is exact in
    float64, the scaled block sums are added in float64 in block order and rounded once
    to bf16; with return_abs also S = sum of |scaled products| per output.
    """
    T, G, D = xq.shape
    Gw, N, Dw = wq.shape
    assert Gw == G and Dw == D and D % MX_GROUP == 0
    HG = D // MX_GROUP
    xv = e4m3_decode(xq).reshape(T, G, HG, MX_GROUP)
    wv = e4m3_decode(wq).reshape(G, N, HG, MX_GROUP)
    xs = np.asarray(x_scale_f, np.float64)
    ws = np.asarray(w_scale, np.float64)
    out = np.zeros((T, G, N), dtype=np.float64)
    sabs = np.zeros((T, G, N), dtype=np.float64)
    for g in range(G):
        for kb in range(HG):
            sc = xs[:, g, kb][:, None] * ws[g, :, kb][None, :]
            out[:, g, :] += (xv[:, g, kb, :] @ wv[g, :, kb, :].T) * sc  # block sum exact
            if return_abs:
                sabs[:, g, :] += (np.abs(xv[:, g, kb, :]) @ np.abs(wv[g, :, kb, :]).T) * sc
    y = f64_to_bf16_rn(out)
    return (y, sabs) if return_abs else y
