"""GPU parity of the FP8 per-token-group quant and its packed UE8M0 scales.

Bit-exact: E4M3 payload bytes and every int32 word of the packed storage (including
the zeroed pack tails and token-padding words), checked on a poisoned buffer.
"""

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import DEV, bf16_dev, dev, host
from oracle import fp8_group as fg
from oracle import numerics as nm
import mfma_model as mm

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_dynamic_quant_amd as wq


def _check(x_bits):
    T, G, D = x_bits.shape
    payload, storage, _ = fg.group_quant_fp8_packed(x_bits)
    xd = bf16_dev(x_bits)
    # poison a storage buffer first by running the wrapper on a 0xA5-filled allocation
    HG, PH, TA = wq.packed_scale_dims(T, D)
    xq, xs, st = wq.wq_group_quant_fp8_ue8m0(xd)
    torch.cuda.synchronize()
    assert xs.shape == (T, G, PH)
    if T > 0:
        assert tuple(xs.stride()) == (1, PH * TA, TA)
    assert st.shape == (G, PH, TA) and st.dtype == torch.int32
    assert np.array_equal(host(xq), payload)
    assert np.array_equal(host(st), storage)
    assert np.array_equal(host(xs), fg.logical_view(storage, T))


@pytest.mark.parametrize("T", syn.FP8_WO_A["T_sweep"])
def test_group_quant_dsv4_wo_a(T):
    _check(syn.fp8_group_x(T))


@pytest.mark.parametrize("T,G,D", [(1, 3, 384), (5, 3, 640), (7, 2, 128), (9, 1, 1152), (3, 8, 4096)])
def test_group_quant_pack_tails(T, G, D):
    _check(syn.fp8_group_x(T, G=G, D=D, layout_variant=True))


@pytest.mark.parametrize("T,G,D", [(1023, 6, 1152), (2048, 4, 1024)])
def test_group_quant_large_grid(T, G, D):
    # TA * G * PH >= 16384: the kernel takes two packs per wave; PH = 3 leaves the
    # second pack of the last wave per (t, g) empty
    _check(syn.fp8_group_x(T, G=G, D=D, layout_variant=True))


def test_group_quant_poisoned_storage_fully_written():
    T, G, D = 6, 3, 640
    x = syn.fp8_group_x(T, G=G, D=D, layout_variant=True)
    _, storage, _ = fg.group_quant_fp8_packed(x)
    HG, PH, TA = wq.packed_scale_dims(T, D)
    st = torch.full((G, PH, TA), -0x5A5A5A5B, dtype=torch.int32, device=DEV)  # 0xA5A5A5A5
    xq = torch.full((T, G, D), 0xA5, dtype=torch.uint8, device=DEV)
    ctx = wq.context(DEV)
    rc = wq.lib().wq_group_quant_fp8_ue8m0(ctx.handle, bf16_dev(x).data_ptr(), T, G, D, xq.data_ptr(), st.data_ptr(),
                                           torch.cuda.current_stream().cuda_stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert np.array_equal(host(st), storage)


def test_group_quant_special_values():
    # zero groups, a group at exactly 448, ties in the subnormal range, negative zero
    T, G, D = 2, 1, 512
    x = np.zeros((T, G, D), np.uint16)
    x[0, 0, 128] = 0x43E0  # 448.0
    x[0, 0, 129] = 0x3A80  # 2^-10 -> tie to 0
    x[0, 0, 130] = 0x3AC0  # 3*2^-11 -> 1 subnormal unit
    x[0, 0, 131] = 0x8000  # -0
    x[1, 0, 256] = 0x3F80  # 1.0
    x[1, 0, 257] = 0xBE9A  # -0.30078125
    x[1, 0, 384:512] = syn.to_bf16_bits(np.linspace(-1e-30, 1e-30, 128).astype(np.float32))
    _check(x)


def test_empty_tokens():
    x = torch.empty((0, 3, 384), dtype=torch.bfloat16, device=DEV)
    xq, xs, st = wq.wq_group_quant_fp8_ue8m0(x)
    assert list(xs.shape) == [0, 3, 1]


def test_cvt_covers_every_reachable_code():
    # one group per (significand, exponent): every bf16 significand scaled across the
    # E4M3 range, so the hardware conversion meets each rounding case the method can make
    vals = []
    for m in range(128, 256):
        for k in range(-20, 2):
            v = m * 2.0 ** k
            if v <= 448.0:
                vals.append(v)
    vals = np.array(vals, np.float32)
    flat = np.concatenate([vals, -vals])
    cols = 127
    rows = (flat.size + cols - 1) // cols
    body = np.zeros(rows * cols, np.float32)
    body[: flat.size] = flat
    x2 = np.zeros((rows, 128), np.float32)
    x2[:, 0] = 448.0  # pins e = 0 in every group
    x2[:, 1:] = body.reshape(rows, cols)
    _check(syn.to_bf16_bits(x2).reshape(rows, 1, 128))


# ---------------------------------------------------------------- grouped FP8 contraction


def _bf16_ulp_of_larger(a, b):
    """The bf16 spacing at the larger of |a|, |b| (float64 arrays of bf16 values); 0 where both
    are 0."""
    m = np.maximum(np.abs(a), np.abs(b))
    _, e = np.frexp(m)  # m = f * 2^e, f in [0.5, 1)
    return np.where(m > 0, np.ldexp(1.0, e - 8), 0.0)


def _check_model(payload, xs_exp, wq_codes, ws_exp, y_ref, sabs, y_gpu, dsv4=False, n_sample=2048):
    """The contraction's tolerance, derived from the accumulation model of the block-scaled
    MFMA (tests/mfma_model.py; rules M1-M3 there are pinned by test_gpu_fp8_mfma_model.py):

    * every output lies within the model's rigorous bound of the oracle's exact value (or
      within 1 bf16 ulp of it);
    * on sampled outputs, the kernel's result lies within the model's alignment and f32
      residual of the exact sum of the M2-truncated products: the model explains the
      result, not only bounds it;
    * the DeepSeek-shaped cases (K = 4096, normal-like codes) also stay within the plain
      f32-summation reading K 2^-24 S + 1 ulp, with at least 99.8 % of outputs within 1 ulp;
    * on the samples, the kernel and the model agree on which outputs are within 1 ulp.

    xs_exp: activation scale exponents per block [T, G, K/blk]; ws_exp: weight scale exponents
    per column and block [G, N, K/blk']."""
    got = host(y_gpu.view(torch.int16)).view(np.uint16)
    d = nm.bf16_ulp_distance(got, y_ref)
    T, G, K = payload.shape
    N = wq_codes.shape[1]
    g64, r64 = nm.bf16_to_f32(got).astype(np.float64), nm.bf16_to_f32(y_ref).astype(np.float64)
    diff = np.abs(g64 - r64)
    ulp = _bf16_ulp_of_larger(g64, r64)
    bound = mm.contraction_bound(payload, xs_exp, wq_codes, ws_exp, sabs) + ulp
    ok = (d <= 1) | (diff <= bound)
    bad = np.argwhere(~ok)
    assert ok.all(), (f"{(~ok).sum()} outputs outside the model bound; first {bad[:4].tolist()} ulp "
                      f"{d[~ok][:4].tolist()} y {r64[~ok][:4]} got {g64[~ok][:4]} bound {bound[~ok][:4]}")
    frac = float((d <= 1).mean())

    # residual against the M2-truncated products, on sampled outputs
    total = T * G * N
    rng = np.random.default_rng(20261203)
    flat = rng.choice(total, n_sample, replace=False) if total > n_sample else np.arange(total)
    t, g, c = np.unravel_index(flat, (T, G, N))
    a_codes = payload[t, g, :]
    a_se = np.repeat(np.asarray(xs_exp, np.int64)[t, g, :], K // xs_exp.shape[-1], axis=-1)
    b_codes = wq_codes[g, c, :]
    b_se = np.repeat(np.asarray(ws_exp, np.int64)[g, c, :], K // ws_exp.shape[-1], axis=-1)
    y_t, upow, s_t = mm.truncated_products(a_codes, np.ldexp(nm.e4m3_decode(a_codes), a_se), mm.code_exponent(a_codes) + a_se,
                                           b_codes, np.ldexp(nm.e4m3_decode(b_codes), b_se), mm.code_exponent(b_codes) + b_se)
    r = mm.residual_bound(upow, s_t, K)
    gs = g64[t, g, c]
    lim = r + _bf16_ulp_of_larger(gs, np.abs(y_t) + r)
    res = np.abs(gs - y_t)
    assert (res <= lim).all(), (f"{(res > lim).sum()} sampled outputs off the model: got {gs[res > lim][:4]} "
                                f"model {y_t[res > lim][:4]} limit {lim[res > lim][:4]}")
    # which sampled outputs end within 1 ulp of the exact value: the model (its truncated sums
    # rounded to bf16) and the kernel must agree, up to the rare output that the residual moves
    # across an ulp boundary
    m1 = nm.bf16_ulp_distance(nm.f64_to_bf16_rn(y_t), y_ref[t, g, c]) <= 1
    g1 = d[t, g, c] <= 1
    n_s = m1.size
    msg = (f"fp8 contraction T={T} G={G} K={K} N={N}: {frac:.5f} within 1 bf16 ulp (model on {n_s} samples "
           f"{m1.mean():.5f}, kernel {g1.mean():.5f}, {(m1 != g1).sum()} differ); max |err|/bound "
           f"{float((diff / bound).max()):.3g}; sampled max |y - model|/limit {float((res / np.maximum(lim, 1e-300)).max()):.3g}")
    assert (m1 != g1).sum() <= max(2, n_s // 500), msg
    if dsv4:
        # K = 4096, normal-like codes: the plain f32-summation reading K 2^-24 S + 1 ulp also
        # holds, and rule M2 alone leaves 0.05-0.15 % of outputs beyond 1 ulp (the model's own
        # fraction on the samples), so at least 99.8 % are within 1 ulp
        a25 = K * 2.0 ** -24 * sabs + ulp
        assert ((d <= 1) | (diff <= a25)).all(), "outside K 2^-24 S + 1 ulp: " + msg
        assert frac >= 0.998, msg
    print(msg)
    return d


def _check_contraction(payload, storage, eb, wq_codes, ws, y_gpu, dsv4=False):
    """128-element blocks: activation bytes eb [T, G, K/128], f32 power-of-two weight block
    scales ws [G, N/128, K/128]."""
    y_ref, sabs = fg.fp8_grouped_contraction(payload, fg.ebyte_to_scale(eb), wq_codes, ws, return_abs=True)
    ws_exp = np.repeat(np.frexp(np.asarray(ws, np.float64))[1] - 1, 128, axis=1)  # [G, N, K/128]
    return _check_model(payload, eb.astype(np.int64) - 127, wq_codes, ws_exp, y_ref, sabs, y_gpu, dsv4=dsv4)


@pytest.mark.parametrize("T", [1, 7, 64, 512])
def test_fp8_contraction_dsv4_wo_a(T):
    G, D, N = 8, 4096, 1024
    x = syn.fp8_group_x(T, G=G, D=D)
    payload, storage, eb = fg.group_quant_fp8_packed(x)
    wq_codes, ws = syn.fp8_weights(42, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(dev(payload), dev(storage), dev(wq_codes), dev(ws), fp8_groups=G)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, G, N)
    _check_contraction(payload, storage, eb, wq_codes, ws, y, dsv4=True)


@pytest.mark.parametrize("T,G,D,N", [(3, 3, 384, 128), (130, 2, 256, 256), (9, 1, 1152, 384),
                                     (5, 2, 512, 128), (17, 1, 4096, 1024), (64, 3, 2048, 256)])
def test_fp8_contraction_small_shapes_wide_codes(T, G, D, N):
    x = syn.fp8_group_x(T, G=G, D=D, layout_variant=True)
    payload, storage, eb = fg.group_quant_fp8_packed(x)
    wq_codes, ws = syn.fp8_weights(7, G=G, N=N, D=D, normalish=False)
    y = wq.wq_quant_matmul(dev(payload), dev(storage), dev(wq_codes), dev(ws), fp8_groups=G)
    torch.cuda.synchronize()
    # weight codes spanning the whole E4M3 range (2^-9 .. 448) with full cancellation: the
    # MFMA's truncation of each product to 13 bits below its group's largest (rule M2 of
    # tests/mfma_model.py) dominates the error here
    _check_contraction(payload, storage, eb, wq_codes, ws, y)


@pytest.mark.parametrize("T,G,D,N", [(100, 2, 128, 128), (65, 3, 384, 256), (200, 2, 256, 384), (129, 1, 640, 128),
                                     (1000, 1, 2048, 640), (300, 4, 1024, 256)])
def test_fp8_contraction_tile_ring_depths(T, G, D, N):
    """Shapes of the tiled kernel (T > 64): K of one, two, three and more 128-deep slices
    (the ring's prologue and its shallower waits at the end of K), ragged token and column
    tiles, and several tiles per group."""
    x = syn.fp8_group_x(T, G=G, D=D, layout_variant=True)
    payload, storage, eb = fg.group_quant_fp8_packed(x)
    wq_codes, ws = syn.fp8_weights(13, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(dev(payload), dev(storage), dev(wq_codes), dev(ws), fp8_groups=G)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, G, N)
    _check_contraction(payload, storage, eb, wq_codes, ws, y)


@pytest.mark.parametrize("T,G,D,N", [(33, 2, 3072, 256), (48, 1, 1024, 384), (64, 2, 4096, 128), (20, 3, 2048, 512),
                                     (17, 1, 1024, 128), (50, 1, 4096, 256)])
def test_fp8_contraction_wide_decode_kernel(T, G, D, N):
    """Shapes of the 32-column decode kernel (17 <= T <= 64, K % 1024 == 0, K <= 4096): two
    to four token tiles with ragged ends, K ranges of one to four blocks per wave, and a wave's blocks
    spanning two packed scale words (K = 3072)."""
    x = syn.fp8_group_x(T, G=G, D=D, layout_variant=True)
    payload, storage, eb = fg.group_quant_fp8_packed(x)
    wq_codes, ws = syn.fp8_weights(11, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(dev(payload), dev(storage), dev(wq_codes), dev(ws), fp8_groups=G)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, G, N)
    _check_contraction(payload, storage, eb, wq_codes, ws, y)


def test_fp8_chain_gpu_quant_then_contraction():
    T, G, D, N = 64, 8, 4096, 1024
    x = syn.fp8_group_x(T, G=G, D=D)
    xq, xs, st = wq.wq_group_quant_fp8_ue8m0(bf16_dev(x))
    wq_codes, ws = syn.fp8_weights(43, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(xq, st, dev(wq_codes), dev(ws), fp8_groups=G)
    torch.cuda.synchronize()
    payload, storage, eb = fg.group_quant_fp8_packed(x)
    assert np.array_equal(host(xq), payload) and np.array_equal(host(st), storage)
    _check_contraction(payload, storage, eb, wq_codes, ws, y, dsv4=True)


def test_fp8_contraction_subnormal_and_extreme_codes():
    """Single nonzero products: every finite E4M3 code of x against 1.0 (0x38) weights with
    unit scales, so each output is exactly one code's value (subnormals included)."""
    T, G, D, N = 254, 1, 128, 128
    xq = np.zeros((T, G, D), np.uint8)
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], np.uint8)
    xq[:, 0, 0] = codes
    eb = np.full((T, G, 1), 127, np.uint8)  # unit activation scales
    storage = fg.pack_ue8m0(eb)
    w = np.zeros((G, N, D), np.uint8)
    w[0, :, 0] = 0x38
    ws = np.ones((G, 1, 1), np.float32)
    y = wq.wq_quant_matmul(dev(xq), dev(storage), dev(w), dev(ws), fp8_groups=G)
    torch.cuda.synchronize()
    got = nm.bf16_to_f32(host(y.view(torch.int16)).view(np.uint16)[:, 0, 0]).astype(np.float64)
    want = nm.e4m3_decode(codes)
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, f"codes {[hex(int(c)) for c in codes[bad][:8]]}: got {got[bad][:8]} want {want[bad][:8]}"


# ---- MX-like 32-element blocks (wq_group_quant_mxfp8) ------------------------------------

def _check_mx(x_bits, poison_storage=True):
    T, G, D = x_bits.shape
    payload, storage, _ = fg.group_quant_fp8_packed(x_bits, 32)
    HG, PH, TA = wq.packed_scale_dims(T, D, 32)
    st = torch.full((G, PH, TA), -0x5A5A5A5B, dtype=torch.int32, device=DEV)  # 0xA5A5A5A5: unwritten words show
    xq = torch.full((T, G, D), 0xA5, dtype=torch.uint8, device=DEV)
    xq, xs, st = wq.wq_group_quant_fp8_ue8m0(bf16_dev(x_bits), x_q=xq, storage=st if poison_storage else None,
                                             group=32)
    torch.cuda.synchronize()
    assert xs.shape == (T, G, PH)
    assert np.array_equal(host(xq), payload)
    assert np.array_equal(host(st), storage)


@pytest.mark.parametrize("T", [1, 7, 64, 512])
def test_mx_group_quant_dsv4_wo_a(T):
    _check_mx(syn.fp8_group_x(T))


@pytest.mark.parametrize("T,G,D", [(5, 3, 96), (9, 2, 160), (6, 1, 544), (3, 2, 32), (4, 8, 4096), (2, 1, 4160)])
def test_mx_group_quant_pack_tails(T, G, D):
    """Blocks per row 3, 5, 17, 1, 128, 130: partial last packs (zero tail bytes) and
    partial last groups of four packs in a wave, with token padding."""
    _check_mx(syn.fp8_group_x(T, G=G, D=D, layout_variant=True))


def test_mx_group_quant_hand_row_and_special_values():
    """The hand-worked row of tests/golden/mx_blocks.txt, and special values per block."""
    x = np.zeros((2, 1, 128), np.uint16)
    x[0, 0, 0], x[0, 0, 40], x[0, 0, 100] = 0x3F80, 0x43E1, 0xBE9A  # 1.0, 450, -0.30078125
    x[1, 0, 32] = 0x43E0  # 448 alone in block 1
    x[1, 0, 64] = 0x3A80  # 2^-10 -> tie to 0
    x[1, 0, 65] = 0x3AC0  # 3*2^-11
    x[1, 0, 66] = 0x8000  # -0
    _check_mx(x)
    q, _, st = wq.wq_group_quant_fp8_ue8m0(bf16_dev(x), group=32)
    torch.cuda.synchronize()
    assert host(st)[0, 0, 0] == 0x75008077  # bytes 0x77, 0x80, 0x00, 0x75 (little-endian)
    assert [int(host(q)[0, 0, i]) for i in (0, 40, 100)] == [0x78, 0x76, 0xFA]


def test_mx_group_quant_empty_and_errors():
    xq, xs, st = wq.wq_group_quant_fp8_ue8m0(torch.empty((0, 2, 64), dtype=torch.bfloat16, device=DEV), group=32)
    assert tuple(xs.shape) == (0, 2, 1)
    rc = wq.lib().wq_group_quant_mxfp8(wq.context(DEV).handle, 0, 1, 1, 48, 0, 0, 0)
    assert rc == 2  # WQ_ERR_SHAPE: D not a multiple of 32


# ---- MX-like contraction (payload WQ_PAYLOAD_MXFP8) ---------------------------------------

def _check_mx_contraction(payload, eb, wq_codes, wb, y, dsv4=False):
    """eb: activation bytes [T, G, D/32]; wb: weight bytes [G, N, D/32]; the same model-derived
    tolerance as the 128-block contraction."""
    y_ref, sabs = fg.mx_contraction(payload, fg.ebyte_to_scale(eb), wq_codes, fg.ebyte_to_scale(wb), return_abs=True)
    return _check_model(payload, eb.astype(np.int64) - 127, wq_codes, wb.astype(np.int64) - 127, y_ref, sabs, y,
                        dsv4=dsv4)


@pytest.mark.parametrize("T", [1, 7, 16, 33, 64, 65, 512])
def test_mx_contraction_dsv4_wo_a(T):
    G, D, N = 8, 4096, 1024
    x = syn.fp8_group_x(T, G=G, D=D)
    payload, storage, eb = fg.group_quant_fp8_packed(x, 32)
    wq_codes, wb = syn.mx_weights(44, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(dev(payload), dev(storage), dev(wq_codes), dev(wb), fp8_groups=G, mx=True)
    torch.cuda.synchronize()
    assert tuple(y.shape) == (T, G, N)
    _check_mx_contraction(payload, eb, wq_codes, wb, y, dsv4=True)


@pytest.mark.parametrize("T,G,D,N", [(3, 2, 512, 128), (17, 1, 1536, 256), (64, 3, 2048, 384), (5, 1, 4096, 128),
                                     (130, 2, 256, 256), (3, 3, 384, 128), (200, 1, 1152, 384),
                                     (100, 2, 128, 128), (65, 3, 384, 256), (129, 1, 640, 128)])
def test_mx_contraction_small_shapes(T, G, D, N):
    x = syn.fp8_group_x(T, G=G, D=D, layout_variant=True)
    payload, storage, eb = fg.group_quant_fp8_packed(x, 32)
    wq_codes, wb = syn.mx_weights(45, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(dev(payload), dev(storage), dev(wq_codes), dev(wb), fp8_groups=G, mx=True)
    torch.cuda.synchronize()
    _check_mx_contraction(payload, eb, wq_codes, wb, y)


def test_mx_chain_gpu_quant_then_contraction():
    T, G, D, N = 64, 8, 4096, 1024
    x = syn.fp8_group_x(T, G=G, D=D)
    xq, xs, st = wq.wq_group_quant_fp8_ue8m0(bf16_dev(x), group=32)
    wq_codes, wb = syn.mx_weights(46, G=G, N=N, D=D)
    y = wq.wq_quant_matmul(xq, st, dev(wq_codes), dev(wb), fp8_groups=G, mx=True)
    torch.cuda.synchronize()
    payload, storage, eb = fg.group_quant_fp8_packed(x, 32)
    assert np.array_equal(host(xq), payload) and np.array_equal(host(st), storage)
    _check_mx_contraction(payload, eb, wq_codes, wb, y, dsv4=True)


@pytest.mark.parametrize("T", [4, 70])
def test_mx_scales_are_per_32_element_block(T):
    """One nonzero product per 32-element block of the first 128, each block with its own
    activation and weight exponents: every output is the bf16 rounding of an exact sum of
    four powers of two (exact in f32), so a scale applied to the wrong block, lane or byte
    shows.  (K = 512, the smallest the decode kernel takes; blocks 4..15 are zero.)  T = 4
    runs the weight-streaming kernel, T = 70 the tiled one."""
    G, D, N = 1, 512, 128
    xq = np.zeros((T, G, D), np.uint8)
    wqc = np.zeros((G, N, D), np.uint8)
    xq[:, 0, [0, 32, 64, 96]] = 0x38          # 1.0 in each of the first four blocks
    wqc[0, :, [0, 32, 64, 96]] = 0x38
    eb = np.full((T, G, D // 32), 127, np.uint8)
    for t in range(T):
        eb[t, 0, :4] = [127 + t % 7, 127 - 2, 127 + 3, 127 - 5]
    wb = np.full((G, N, D // 32), 127, np.uint8)
    for n in range(N):
        wb[0, n, :4] = [127, 127 + (n % 3), 127 - (n % 5), 127 + 1]
    storage = fg.pack_ue8m0(eb)
    y = wq.wq_quant_matmul(dev(xq), dev(storage), dev(wqc), dev(wb), fp8_groups=G, mx=True)
    torch.cuda.synchronize()
    got = nm.bf16_to_f32(host(y.view(torch.int16)).view(np.uint16)[:, 0, :]).astype(np.float64)
    exact = np.array([[sum(2.0 ** (int(eb[t, 0, b]) - 127 + int(wb[0, n, b]) - 127) for b in range(4))
                       for n in range(N)] for t in range(T)])
    want = nm.bf16_to_f32(nm.f64_to_bf16_rn(exact)).astype(np.float64)  # one rounding of the exact sum
    assert np.array_equal(got, want)
