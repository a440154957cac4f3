"""GPU parity of the INT8 path (quant, split-K and tiled GEMM, fused) against the oracle.

Bit-exact: INT8 payloads, f32 scales, int32 accumulators.  BF16 outputs: within 1 bf16
ulp of the oracle's correctly rounded value (relative error <= 2^-8).
"""

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import DEV, bf16_dev, dev, host, host_bf16_bits, poison
from oracle import int8_linear as il
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_dynamic_quant_amd as wq


def _y_within_one_ulp(y_gpu_bits, y_ref_bits):
    d = nm.bf16_ulp_distance(y_gpu_bits, y_ref_bits)
    assert d.max() <= 1, f"max bf16 ulp distance {d.max()}"


def _check_linear(x, w, sw, *, fused, split=0):
    ref = il.linear_w8a8(x, w, sw)
    M, K = x.shape
    N = w.shape[0]
    wq.set_split(DEV, split)
    try:
        xd, wd, swd = bf16_dev(x), dev(w), dev(sw)
        acc = poison((M, N), torch.int32)
        if fused:
            xq = poison((M, K), torch.int8)
            xs = poison((M,), torch.float32)
            y = wq.wq_fused_quant_matmul(xd, wd, swd, x_q_out=xq, x_scale_out=xs, acc_out=acc)
        else:
            xq, xs = wq.wq_dynamic_quant(xd)
            y = wq.wq_quant_matmul(xq, xs, wd, swd, acc_out=acc)
        torch.cuda.synchronize()
    finally:
        wq.set_split(DEV, 0)
    assert np.array_equal(host(xq), ref["q"])
    assert np.array_equal(host(xs).view(np.uint32), ref["s"].view(np.uint32))
    assert np.array_equal(host(acc), ref["acc"])
    _y_within_one_ulp(host_bf16_bits(y), ref["y"])
    return y


def test_tiny_linear():
    x, w, sw = syn.tiny_linear()
    _check_linear(x, w, sw, fused=False)
    _check_linear(x, w, sw, fused=True)


@pytest.mark.parametrize("M", syn.WQ_A["M_sweep"])
def test_wq_a_decode_standalone_and_fused(M):
    x, w, sw = syn.wq_a_linear(M)
    y1 = _check_linear(x, w, sw, fused=False)
    y2 = _check_linear(x, w, sw, fused=True)
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    # without the optional outputs (the payload stays on chip, or in the workspace)
    y3 = wq.wq_fused_quant_matmul(bf16_dev(x), dev(w), dev(sw))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y3.view(torch.int16))


def test_wq_a_m256_two_launch_path():
    """wq_a at M = 256, above the one-launch limit: the fused call runs the quant kernel and
    the GEMM, through the workspace or the exported tuple, with the same bytes."""
    x, w, sw = syn.wq_a_linear(256)
    assert wq.wq_fused_path(256, 4096, 1024) == 0
    y1 = _check_linear(x, w, sw, fused=True)
    y2 = wq.wq_fused_quant_matmul(bf16_dev(x), dev(w), dev(sw))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))


@pytest.mark.parametrize("M,K,N", [(1, 512, 64), (15, 1024, 128), (16, 2048, 256), (17, 4096, 1040), (31, 4096, 48),
                                   (48, 1024, 1040), (64, 4096, 1024), (2, 4096, 32768), (9, 512, 4096),
                                   (65, 4096, 1024), (128, 4096, 1024), (200, 2048, 272), (255, 512, 48)])
def test_fused_one_launch_shapes(M, K, N):
    # the one-launch fused kernel takes K % 512 == 0, K <= 4096, M < 256: one 16-row group
    # and several, a partial last group, narrow and wide N, exported x_q / x_scale / acc
    assert wq.wq_fused_path(M, K, N) == 2
    x = syn.activations((97, M, K), M, K, outlier_frac=0.005, outlier_mul=30.0)
    w, sw = syn.int8_weights((98, N, K), N, K)
    _check_linear(x, w, sw, fused=True)


@pytest.mark.parametrize("M,K,N", [(1, 16, 16), (3, 1040, 96), (2, 8192, 256), (4, 6144, 64)])
def test_fused_gemv_for_k_the_mfma_kernel_does_not_take(M, K, N):
    # K % 512 != 0 or 4096 < K <= 8192 at M <= 4: one launch of the dot4 GEMV kernel
    assert wq.wq_fused_path(M, K, N) == 1
    x = syn.activations((105, M, K), M, K, outlier_frac=0.005, outlier_mul=30.0)
    w, sw = syn.int8_weights((106, N, K), N, K)
    _check_linear(x, w, sw, fused=True)


@pytest.mark.parametrize("M,K,N", [(33, 1040, 272), (64, 8192, 96), (7, 1552, 48), (2, 4112, 64)])
def test_quant_matmul_decode_other_k(M, K, N):
    # given codes at decode M with a K the fused kernel does not take (K % 512 != 0 or
    # K > 4096): the decode GEMM kernel, or the dot4 GEMV at M <= 4
    x = syn.activations((109, M, K), M, K, outlier_frac=0.005, outlier_mul=30.0)
    w, sw = syn.int8_weights((110, N, K), N, K)
    _check_linear(x, w, sw, fused=False)


@pytest.mark.parametrize("M,K,N", [(260, 128, 272), (300, 256, 512), (512, 384, 256)])
def test_prefill_short_k(M, K, N):
    # the persistent 256 x 256 kernel with 1, 2 and 3 K slices per tile (its tile scales
    # reach LDS one slice after the tile's first), ragged M and N
    x = syn.activations((111, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    w, sw = syn.int8_weights((112, N, K), N, K)
    _check_linear(x, w, sw, fused=False)


FUSED_SHAPES = [(r, nt) for r in (1, 2, 4, 8, 16) for nt in (4, 8, 16, 32)]


@pytest.mark.parametrize("R,NT", FUSED_SHAPES)
def test_every_fused_shape_gives_identical_bytes(R, NT):
    # the one-launch kernel with each rows x columns per workgroup: ragged row tiles (M = 23)
    # and column slices (N = 1040 is not a multiple of 32), x_q / x_scale / acc exported
    for (M, K, N, seed) in ((23, 2048, 1040, 101), (64, 4096, 256, 102)):
        x = syn.activations((seed, M, K), M, K, outlier_frac=0.005, outlier_mul=30.0)
        w, sw = syn.int8_weights((seed + 50, N, K), N, K)
        wq.set_fused_shape(DEV, R, NT)
        try:
            assert wq.wq_fused_path(M, K, N) == 2
            _check_linear(x, w, sw, fused=True)
            _check_linear(x, w, sw, fused=False)  # the same kernel on the given codes
        finally:
            wq.set_fused_shape(DEV, 0, 0)


def _tie_rows(M, K, seed):
    """Rows whose values sit on or next to rounding ties of v / s: every chunk of them fails
    the multiply-by-reciprocal check and takes the exact division."""
    rng = np.random.default_rng(seed)
    x = syn.activations((seed, M, K), M, K)
    for m in range(0, M, 2):
        a = np.float32([127.0, 100.0, 0.375, 7.5][(m // 2) % 4])
        s = np.float32(a / np.float32(127.0))
        k = rng.integers(-127, 127, size=K).astype(np.float32)
        v = (k + np.float32(0.5)) * s
        row = syn.to_bf16_bits(v.astype(np.float32))
        row[0] = syn.to_bf16_bits(np.array([a], np.float32))[0]
        x[m] = row
    return x


@pytest.mark.parametrize("R,NT", [(1, 4), (4, 16), (16, 32), (0, 0)])
def test_fused_ties_take_the_exact_path(R, NT):
    M, K, N = 16, 4096, 512
    x = _tie_rows(M, K, 103)
    x[5] = 0  # zero scale: the exact path's s == 0 rule
    x[7, :] = syn.to_bf16_bits(np.full(K, 1.0e-38, np.float32))[:]  # subnormal scale
    w, sw = syn.int8_weights((104, N, K), N, K)
    wq.set_fused_shape(DEV, R, NT)
    try:
        _check_linear(x, w, sw, fused=True)
    finally:
        wq.set_fused_shape(DEV, 0, 0)


@pytest.mark.parametrize("M,R,NT", [(5, 4, 16), (21, 16, 32), (3, 2, 16), (9, 8, 16)])
def test_fused_ties_in_a_partial_row_tile(M, R, NT):
    """The last row tile holds fewer than R rows and its missing rows are clamped copies of
    a tie row: the live tie rows take the exact path, the copies are never stored."""
    K, N = 4096, 1024
    x = _tie_rows(M, K, 107)
    x[M - 1] = x[M - 1 - ((M - 1) % 2)]  # the last row is a tie row
    w, sw = syn.int8_weights((108, N, K), N, K)
    wq.set_fused_shape(DEV, R, NT)
    try:
        _check_linear(x, w, sw, fused=True)
    finally:
        wq.set_fused_shape(DEV, 0, 0)


@pytest.mark.parametrize("M,K,N", [(5, 4096, 1024), (64, 2048, 272), (3, 1040, 96), (80, 1024, 256)])
def test_fused_strided_rows(M, K, N):
    # x rows ldx = K + 64 apart and y rows ldy = N + 8 apart (views into wider buffers), on
    # the one-launch MFMA kernel, the GEMV and the two-launch path; the padding of y stays
    # untouched
    xw = syn.activations((107, M, K + 64), M, K + 64, outlier_frac=0.005, outlier_mul=30.0)
    x = np.ascontiguousarray(xw[:, :K])
    w, sw = syn.int8_weights((108, N, K), N, K)
    ref = il.linear_w8a8(x, w, sw)
    yw = poison((M, N + 8), torch.bfloat16)
    y = wq.wq_fused_quant_matmul(bf16_dev(xw)[:, :K], dev(w), dev(sw), y=yw[:, :N])
    torch.cuda.synchronize()
    assert y.stride(0) == N + 8
    _y_within_one_ulp(host_bf16_bits(y), ref["y"])
    assert (host_bf16_bits(yw[:, N:]) == 0xA5A5).all()


@pytest.mark.parametrize("split", [1, 2, 4, 8, 16, 64])
def test_every_split_gives_identical_bytes(split):
    x, w, sw = syn.wq_a_linear(7)
    _check_linear(x, w, sw, fused=False, split=split)
    _check_linear(x, w, sw, fused=True, split=split)


@pytest.mark.parametrize("M", [1, 8, 64, 512])
def test_wq_b_wide(M):
    x = syn.wq_b_x(M)
    w, sw = syn.wq_b_w()
    _check_linear(x, w, sw, fused=False)


def _bf16_rne_bits(f32):
    u = np.ascontiguousarray(f32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("M,K,N", [(2, 4096, 1024), (8, 4096, 1024), (70, 1024, 48), (300, 1024, 528), (512, 1024, 32768),
                                   (1000, 2048, 1536), (257, 128, 256), (260, 256, 272), (2600, 256, 8208)])
def test_epilogue_is_the_documented_f32_sequence(M, K, N):
    """Stricter than the 1-ulp bound: the bf16 output equals bf16_RN(RN(RN(f32(acc) * s_m) * sw_n))
    bit for bit, the f32 operation sequence the kernels document (f32(acc) rounds to nearest
    even too), here emulated with numpy float32 arithmetic on the oracle's exact accumulators."""
    x = syn.activations((99, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    w, sw = syn.int8_weights((100, N, K), N, K)
    q, s = il.quant_int8_per_token(x)
    acc = il.gemm_int8_int32(q, w)
    want = _bf16_rne_bits((acc.astype(np.float32) * s[:, None]).astype(np.float32) * sw[None, :].astype(np.float32))
    for fused in (False, True):
        if fused:
            y = wq.wq_fused_quant_matmul(bf16_dev(x), dev(w), dev(sw))
        else:
            xq, xs = wq.wq_dynamic_quant(bf16_dev(x))
            y = wq.wq_quant_matmul(xq, xs, dev(w), dev(sw))
        torch.cuda.synchronize()
        got = host_bf16_bits(y)
        assert np.array_equal(got, want), f"fused={fused}: {(got != want).sum()} outputs differ"


@pytest.mark.parametrize("M,K,N", [(1000, 128, 16384), (1024, 256, 16400), (2048, 128, 16384), (2600, 128, 4112)])
def test_large_gemm_tile_orders_sampled_rows(M, K, N):
    """The M, N >= 256 GEMM in both tile orders: N-range (each XCD walks a range of W's columns,
    nontemporal output; 1000 x 16384, 2048 x 16384) and row groups (cached output; 1024 x
    16400, 2600 x 4112), with a last tile row or column shifted back to end at M or N, so some
    rows or columns are computed by two tiles, and with several tiles per workgroup (the
    epilogue carried into the next tile's first slice) at one slice per tile (K = 128).
    Sampled rows (every row the shifted tile shares) against the oracle's accumulators and
    the documented f32 epilogue, and the production launch against the one that also exports
    the accumulators."""
    x = syn.activations((101, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    w, sw = syn.int8_weights((102, N, K), N, K)
    xq, xs = wq.wq_dynamic_quant(bf16_dev(x))
    wd, swd = dev(w), dev(sw)
    acc = poison((M, N), torch.int32)
    y_acc = wq.wq_quant_matmul(xq, xs, wd, swd, acc_out=acc)
    y = wq.wq_quant_matmul(xq, xs, wd, swd)
    torch.cuda.synchronize()
    assert torch.equal(y.view(torch.int16), y_acc.view(torch.int16))
    last = (M - 1) // 256 * 256  # the last tile row's nominal origin; the shifted one is M - 256
    rows = np.unique(np.concatenate([[0, 1, 255, 256], np.arange(M - 256 - 2, M - 256 + 3), np.arange(last - 3, last + 3),
                                     np.random.default_rng(M).choice(M, 24, replace=False), [M - 2, M - 1]]))
    rows = rows[(rows >= 0) & (rows < M)]
    q, s = il.quant_int8_per_token(x[rows])
    accr = il.gemm_int8_int32(q, w)
    ridx = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(host(acc[ridx]), accr)
    want = _bf16_rne_bits((accr.astype(np.float32) * s[:, None]).astype(np.float32) * sw[None, :].astype(np.float32))
    got = host_bf16_bits(y[ridx])
    assert np.array_equal(got, want), f"{(got != want).sum()} outputs differ"


@pytest.mark.parametrize("M,K,N", [(256, 128, 256), (511, 384, 272), (777, 640, 1040), (1300, 1152, 2064)])
def test_large_gemm_odd_shapes(M, K, N):
    """The M, N >= 256 GEMM at the smallest shape it takes and at shapes where M, N and the
    number of K slices (1, 3, 5, 9) fit no power of two: every output against the oracle's
    documented f32 epilogue, and the accumulator export against the oracle."""
    x = syn.activations((103, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    w, sw = syn.int8_weights((104, N, K), N, K)
    xq, xs = wq.wq_dynamic_quant(bf16_dev(x))
    acc = poison((M, N), torch.int32)
    y_acc = wq.wq_quant_matmul(xq, xs, dev(w), dev(sw), acc_out=acc)
    y = wq.wq_quant_matmul(xq, xs, dev(w), dev(sw))
    torch.cuda.synchronize()
    q, s = il.quant_int8_per_token(x)
    accr = il.gemm_int8_int32(q, w)
    assert np.array_equal(host(acc), accr)
    want = _bf16_rne_bits((accr.astype(np.float32) * s[:, None]).astype(np.float32) * sw[None, :].astype(np.float32))
    assert np.array_equal(host_bf16_bits(y), want)
    assert torch.equal(y.view(torch.int16), y_acc.view(torch.int16))


def test_wq_b_prefill_8192_sampled_rows():
    M = 8192
    x = syn.wq_b_x(M)
    w, sw = syn.wq_b_w()
    xd, wd, swd = bf16_dev(x), dev(w), dev(sw)
    xq, xs = wq.wq_dynamic_quant(xd)
    acc = torch.empty((M, w.shape[0]), dtype=torch.int32, device=DEV)
    y = wq.wq_quant_matmul(xq, xs, wd, swd, acc_out=acc)
    torch.cuda.synchronize()
    rows = np.random.default_rng(0).choice(M, 48, replace=False)
    rows = np.concatenate([rows, [0, 127, 128, M - 1]])
    q, s = il.quant_int8_per_token(x[rows])
    assert np.array_equal(host(xq[torch.from_numpy(rows).to(DEV)]), q)
    accr = il.gemm_int8_int32(q, w)
    assert np.array_equal(host(acc[torch.from_numpy(rows).to(DEV)]), accr)
    _y_within_one_ulp(host_bf16_bits(y[torch.from_numpy(rows).to(DEV)]), il.epilogue_bf16(accr, s, sw))
    # the production launch (no accumulator export) writes the same bytes
    y2 = wq.wq_quant_matmul(xq, xs, wd, swd)
    torch.cuda.synchronize()
    assert torch.equal(y2.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("M,K,N", [(3, 272, 48), (65, 272, 48), (130, 1040, 208), (64, 64, 16), (17, 4096, 1040),
                                   (5, 512, 4096), (33, 528, 2064), (2, 8192, 528), (40, 1024, 96),
                                   (3, 16384, 64), (8, 12288, 80), (1, 16, 16),
                                   (300, 1024, 528), (257, 128, 256), (1000, 2048, 1536)])
def test_ragged_shapes(M, K, N):
    x = syn.activations((90, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    w, sw = syn.int8_weights((91, N, K), N, K)
    _check_linear(x, w, sw, fused=False)
    if M <= 64:
        _check_linear(x, w, sw, fused=True)


def test_zero_rows_and_extremes():
    M, K, N = 5, 512, 64
    x = syn.activations((92,), M, K)
    x[1] = 0  # all-zero row: s = 0, q = 0, y = 0
    x[3, :] = syn.to_bf16_bits(np.full(K, -1.0e30, np.float32))[:]  # large magnitudes (the f32 epilogue stays finite)
    w, sw = syn.int8_weights((93,), N, K)
    _check_linear(x, w, sw, fused=False)
    _check_linear(x, w, sw, fused=True)


def test_quant_strided_rows_and_splits():
    M, K = 6, 4096
    big = syn.activations((94,), M, K + 64, outlier_frac=0.01, outlier_mul=30.0)
    xd = bf16_dev(big)[:, :K]
    q_ref, s_ref = il.quant_int8_per_token(big[:, :K])
    for split in (0, 1, 2, 4, 8):
        wq.set_split(DEV, split)
        try:
            q, s = wq.wq_dynamic_quant(xd)
            torch.cuda.synchronize()
        finally:
            wq.set_split(DEV, 0)
        assert np.array_equal(host(q), q_ref) and np.array_equal(host(s), s_ref)


@pytest.mark.parametrize("M,K,f32", [(4096, 1024, False), (4097, 16, False), (4099, 528, False), (4103, 1008, False),
                                     (5000, 512, True), (4098, 272, True)])
def test_quant_many_short_rows(M, K, f32):
    """Thousands of short rows (a row per wave, one or two 16-byte chunks per lane, lanes past
    the row idle), row counts that leave the last workgroup partly empty."""
    x = syn.activations((97, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    if f32:
        xf = nm.bf16_to_f32(x) * np.float32(1.0 + 2.0 ** -9)  # values off the bf16 grid
        q, s = wq.wq_dynamic_quant(torch.from_numpy(xf).to(DEV))
        q_ref, s_ref = il.quant_int8_per_token(xf, is_bf16_bits=False)
    else:
        q, s = wq.wq_dynamic_quant(bf16_dev(x))
        q_ref, s_ref = il.quant_int8_per_token(x)
    torch.cuda.synchronize()
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)


def test_quant_long_rows_streamed():
    M, K = 3, 32768  # beyond the register cache: three streamed passes
    x = syn.activations((95,), M, K, outlier_frac=0.001, outlier_mul=100.0)
    q, s = wq.wq_dynamic_quant(bf16_dev(x))
    torch.cuda.synchronize()
    q_ref, s_ref = il.quant_int8_per_token(x)
    assert np.array_equal(host(q), q_ref) and np.array_equal(host(s), s_ref)


def test_empty_and_errors():
    w, sw = syn.int8_weights((96,), 64, 256)
    x = torch.empty((0, 256), dtype=torch.bfloat16, device=DEV)
    q, s = wq.wq_dynamic_quant(x)
    assert q.shape == (0, 256)
    y = wq.wq_fused_quant_matmul(x, dev(w), dev(sw))
    assert y.shape == (0, 64)
    with pytest.raises(wq.WqError) as e:
        wq.wq_dynamic_quant(torch.zeros((2, 24), dtype=torch.bfloat16, device=DEV))  # K % 16 != 0
    assert e.value.status == 2
    xb = torch.zeros((2, 256 + 4), dtype=torch.bfloat16, device=DEV)[:, 4:]  # base 8 bytes off
    with pytest.raises(wq.WqError) as e:
        wq.wq_dynamic_quant(xb)
    assert e.value.status == 3


def test_deterministic_bytes():
    x, w, sw = syn.wq_a_linear(16)
    xd, wd, swd = bf16_dev(x), dev(w), dev(sw)
    ys = [wq.wq_fused_quant_matmul(xd, wd, swd).view(torch.int16).clone() for _ in range(3)]
    ys += [wq.wq_quant_matmul(*wq.wq_dynamic_quant(xd), wd, swd).view(torch.int16).clone() for _ in range(2)]
    torch.cuda.synchronize()
    for y in ys[1:]:
        assert torch.equal(ys[0], y)
