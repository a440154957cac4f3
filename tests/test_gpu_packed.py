"""GPU checks of the fragment-order weight layout (wq_pack_weight_i8) and of the fused call
that reads it (wq_fused_quant_matmul_packed).

The layout is a fixed permutation of the weight bytes (include/wq.h states the address of
byte (n, k)); the test builds it here with numpy reshapes and compares the GPU's bytes.  The
packed call must give the same bytes as the plain fused call, which the oracle pins: INT8
payloads, scales and accumulators bit-exact, BF16 within 1 ulp of the oracle.
"""

import contextlib
import os

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import DEV, assert_same, bf16_dev, dev, host, host_bf16_bits, poison
from oracle import int8_linear as il
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_dynamic_quant_amd as wq


def fragment_order(w: np.ndarray) -> np.ndarray:
    """Byte (n, k) of w [N, K] at ((k//64 * N//4 + n//4) * 4 + (k%64)//16) * 64 + (n%4) * 16 + k%16."""
    N, K = w.shape
    v = w.reshape(N // 4, 4, K // 64, 4, 16)          # [n//4, n%4, k//64, (k%64)//16, k%16]
    return np.ascontiguousarray(v.transpose(2, 0, 3, 1, 4)).reshape(-1)


def test_fragment_order_reference_addresses():
    """The reshape above against the address formula, element by element, on a small w."""
    N, K = 8, 128
    w = np.arange(N * K, dtype=np.int64).reshape(N, K)
    got = fragment_order(w)
    for n in range(N):
        for k in range(K):
            a = ((k // 64 * (N // 4) + n // 4) * 4 + (k % 64) // 16) * 64 + (n % 4) * 16 + k % 16
            assert got[a] == w[n, k]


@pytest.mark.parametrize("N,K", [(1024, 4096), (528, 1536), (16, 64), (48, 512)])
def test_pack_layout(N, K):
    w, _ = syn.int8_weights((9, N, K), N, K)
    wp = wq.wq_pack_weight_i8(dev(w))
    torch.cuda.synchronize()
    assert_same("wp", host(wp), fragment_order(w))


def test_pack_strided_rows():
    N, K, ld = 64, 512, 640
    full, _ = syn.int8_weights((10, N, ld), N, ld)
    wd = dev(full)[:, :K]
    wp = wq.wq_pack_weight_i8(wd)
    torch.cuda.synchronize()
    assert_same("wp", host(wp), fragment_order(np.ascontiguousarray(full[:, :K])))


def _check_packed(x, w, sw):
    M, K = x.shape
    N = w.shape[0]
    ref = il.linear_w8a8(x, w, sw)
    xd, wd, swd = bf16_dev(x), dev(w), dev(sw)
    wp = wq.wq_pack_weight_i8(wd)
    outs = {}
    for packed in (False, True):
        acc = poison((M, N), torch.int32)
        xq = poison((M, K), torch.int8)
        xs = poison((M,), torch.float32)
        if packed:
            y = wq.wq_fused_quant_matmul_packed(xd, wp, swd, N, x_q_out=xq, x_scale_out=xs, acc_out=acc)
        else:
            y = wq.wq_fused_quant_matmul(xd, wd, swd, x_q_out=xq, x_scale_out=xs, acc_out=acc)
        torch.cuda.synchronize()
        outs[packed] = (host_bf16_bits(y), host(xq), host(xs), host(acc))
    for name, a, b in zip(("y", "x_q", "x_scale", "acc"), outs[True], outs[False]):
        assert_same(name, a, b)
    yb, xq, xs, acc = outs[True]
    assert_same("x_q vs oracle", xq, ref["q"])
    assert_same("x_scale vs oracle", xs, ref["s"])
    assert_same("acc vs oracle", acc, ref["acc"])
    assert nm.bf16_ulp_distance(yb, ref["y"]).max() <= 1


@pytest.mark.parametrize("M", syn.WQ_A["M_sweep"])
def test_packed_wq_a_decode(M):
    x, w, sw = syn.wq_a_linear(M)
    _check_packed(x, w, sw)


@pytest.mark.parametrize("M", [1, 8, 64])
def test_packed_wkv_decode(M):
    """The wkv-shaped projection (K = 4096, N = 512) of the same family."""
    x = syn.activations((16, M, 4096), M, 4096, outlier_frac=0.005, outlier_mul=30.0)
    w, sw = syn.int8_weights((16, 512, 4096), 512, 4096)
    _check_packed(x, w, sw)


@pytest.mark.parametrize("M,K,N", [(3, 512, 528), (33, 1536, 272), (64, 2048, 48), (17, 4096, 1040), (5, 1024, 16),
                                   (96, 4096, 1024), (128, 4096, 1024), (255, 512, 48)])
def test_packed_ragged_shapes(M, K, N):
    x = syn.activations((12, M, K), M, K, outlier_frac=0.01, outlier_mul=40.0)
    w, sw = syn.int8_weights((12, N, K), N, K)
    _check_packed(x, w, sw)


@pytest.mark.parametrize("R,NT", [(1, 4), (1, 8), (2, 16), (4, 32), (16, 32)])
def test_packed_every_column_width(R, NT):
    """Column widths 4 and 8 read one or two 4-column blocks per fragment, 32 two fragments."""
    x, w, sw = syn.wq_a_linear(16)
    wq.set_fused_shape(DEV, R, NT)
    try:
        _check_packed(x, w, sw)
    finally:
        wq.set_fused_shape(DEV, 0, 0)


@pytest.mark.parametrize("M,K,N", [(1, 4096, 1024), (2, 512, 64), (7, 4096, 1024), (33, 1536, 272), (64, 4096, 1024)])
def test_quant_matmul_on_packed_weights(M, K, N):
    """The standalone GEMM on given codes (wq_quant_matmul, decode M) on fragment-order
    weights: the same bytes as on the plain ones, the oracle's accumulators and outputs."""
    x = syn.activations((14, M, K), M, K, outlier_frac=0.01, outlier_mul=25.0)
    w, sw = syn.int8_weights((14, N, K), N, K)
    ref = il.linear_w8a8(x, w, sw)
    xq, xs = wq.wq_dynamic_quant(bf16_dev(x))
    wd, swd = dev(w), dev(sw)
    wp = wq.wq_pack_weight_i8(wd)
    acc_p, acc_f = poison((M, N), torch.int32), poison((M, N), torch.int32)
    y_plain = wq.wq_quant_matmul(xq, xs, wd, swd, acc_out=acc_p)
    y_frag = wq.wq_quant_matmul(xq, xs, wp, swd, acc_out=acc_f, b_fragment=True, n=N)
    torch.cuda.synchronize()
    assert_same("y", host_bf16_bits(y_frag), host_bf16_bits(y_plain))
    assert_same("acc", host(acc_f), ref["acc"])
    assert nm.bf16_ulp_distance(host_bf16_bits(y_frag), ref["y"]).max() <= 1


@pytest.mark.parametrize("M,K,N", [(65, 4096, 1024), (128, 4096, 1024), (200, 2048, 272), (255, 512, 48)])
def test_quant_matmul_mid_m(M, K, N):
    """64 < M < 256: the decode kernel on the given codes with row tiles of 16, on plain and
    on fragment-order weights: the oracle's accumulators and outputs, the same bytes."""
    x = syn.activations((17, M, K), M, K, outlier_frac=0.01, outlier_mul=25.0)
    w, sw = syn.int8_weights((17, N, K), N, K)
    ref = il.linear_w8a8(x, w, sw)
    xq, xs = wq.wq_dynamic_quant(bf16_dev(x))
    wd, swd = dev(w), dev(sw)
    acc_p, acc_f = poison((M, N), torch.int32), poison((M, N), torch.int32)
    y_plain = wq.wq_quant_matmul(xq, xs, wd, swd, acc_out=acc_p)
    y_frag = wq.wq_quant_matmul(xq, xs, wq.wq_pack_weight_i8(wd), swd, acc_out=acc_f, b_fragment=True, n=N)
    torch.cuda.synchronize()
    assert_same("acc", host(acc_p), ref["acc"])
    assert_same("acc (fragment order)", host(acc_f), ref["acc"])
    assert_same("y", host_bf16_bits(y_frag), host_bf16_bits(y_plain))
    assert nm.bf16_ulp_distance(host_bf16_bits(y_plain), ref["y"]).max() <= 1


@contextlib.contextmanager
def _context_with_env(**env):
    """A fresh library context created with the given knobs in the environment (the context
    reads it once, at creation), used by the binding's calls on DEV for the with-block."""
    old = {k: os.environ.get(k) for k in env}
    os.environ.update({k: str(v) for k, v in env.items()})
    try:
        ctx = wq.Context(DEV)
    finally:
        for k, v in old.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    idx = DEV.index
    saved = wq._CTX.get(idx)
    wq._CTX[idx] = ctx
    try:
        yield ctx
    finally:
        if saved is None:
            wq._CTX.pop(idx, None)
        else:
            wq._CTX[idx] = saved


@pytest.mark.parametrize("M", [65, 128, 255])
@pytest.mark.parametrize("nt,mt", [(8, 0), (0, 2), (16, 4)])
def test_quant_matmul_mid_m_fragment_order_with_decode_knobs(M, nt, mt):
    """Fragment-order weights at 64 < M < 256 with the decode knobs set: the call must still
    read them in fragment order (the knobs only steer the plain-layout kernels), giving the
    oracle's accumulators and the plain call's bytes."""
    K, N = 4096, 1024
    x = syn.activations((18, M, K), M, K, outlier_frac=0.01, outlier_mul=25.0)
    w, sw = syn.int8_weights((18, N, K), N, K)
    ref = il.linear_w8a8(x, w, sw)
    with _context_with_env(WQ_DECODE_NT=nt, WQ_DECODE_MT=mt):
        xq, xs = wq.wq_dynamic_quant(bf16_dev(x))
        wd, swd = dev(w), dev(sw)
        acc_p, acc_f = poison((M, N), torch.int32), poison((M, N), torch.int32)
        y_plain = wq.wq_quant_matmul(xq, xs, wd, swd, acc_out=acc_p)
        y_frag = wq.wq_quant_matmul(xq, xs, wq.wq_pack_weight_i8(wd), swd, acc_out=acc_f, b_fragment=True, n=N)
        torch.cuda.synchronize()
    assert_same("acc (fragment order)", host(acc_f), ref["acc"])
    assert_same("acc", host(acc_p), ref["acc"])
    assert_same("y", host_bf16_bits(y_frag), host_bf16_bits(y_plain))
    assert nm.bf16_ulp_distance(host_bf16_bits(y_frag), ref["y"]).max() <= 1


def test_quant_matmul_packed_unsupported_sizes():
    K, N = 512, 64
    w, sw = syn.int8_weights((15, N, K), N, K)
    wp = wq.wq_pack_weight_i8(dev(w))
    for M in (256, 300):
        q = torch.zeros((M, K), dtype=torch.int8, device=DEV)
        with pytest.raises(wq.WqError):
            wq.wq_quant_matmul(q, torch.ones(M, device=DEV), wp, dev(sw), b_fragment=True, n=N)


def test_packed_errors():
    N, K = 64, 512
    w, sw = syn.int8_weights((13, N, K), N, K)
    wp = wq.wq_pack_weight_i8(dev(w))
    for M, Kx in ((256, 512), (4, 4608), (4, 528)):
        x = bf16_dev(syn.activations((13, M, Kx), M, Kx))
        with pytest.raises(wq.WqError):
            wq.wq_fused_quant_matmul_packed(x, torch.zeros(N * Kx, dtype=torch.int8, device=DEV), dev(sw), N)
    with pytest.raises(wq.WqError):  # K % 64 != 0
        wq.wq_pack_weight_i8(torch.zeros((16, 80), dtype=torch.int8, device=DEV))
    y = wq.wq_fused_quant_matmul_packed(torch.empty((0, K), dtype=torch.bfloat16, device=DEV), wp, dev(sw), N)
    assert tuple(y.shape) == (0, N)
