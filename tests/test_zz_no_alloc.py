"""The allocation-free entry point wq_fused_quant_matmul_static, called through the C ABI,
against wq_fused_quant_matmul (context and workspace) on the same inputs: identical bytes
for y, the accumulators and the exported payload, on calls that stage the INT8 payload in
the library's static buffer (M above the one-launch limit), two in a row with the second
smaller, and on a one-launch size; sizes beyond the buffer are refused with nothing written."""

import ctypes

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import DEV, assert_same, bf16_dev, dev, host, host_bf16_bits, poison
from oracle import int8_linear as il

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_dynamic_quant_amd as wq

WQ_ERR_WORKSPACE, WQ_ERR_DEVICE = 4, 5


def _static(x, w, sw, y, acc=None, xq=None, xs=None, device=None):
    M, K = x.shape
    N = w.shape[0]
    return wq.lib().wq_fused_quant_matmul_static(
        DEV.index if device is None else device, x.data_ptr(), M, K, x.stride(0), w.data_ptr(), sw.data_ptr(), N,
        y.data_ptr(), y.stride(0), None if xq is None else xq.data_ptr(), None if xs is None else xs.data_ptr(),
        None if acc is None else acc.data_ptr(), torch.cuda.current_stream().cuda_stream)


def _compare(M, K, N, seed):
    x = syn.activations((90, seed, M, K), M, K, outlier_frac=0.005, outlier_mul=30.0)
    w, sw = syn.int8_weights((90, seed, N, K), N, K)
    xd, wd, swd = bf16_dev(x), dev(w), dev(sw)
    acc_c, y_c = poison((M, N), torch.int32), poison((M, N), torch.bfloat16)
    wq.wq_fused_quant_matmul(xd, wd, swd, y=y_c, acc_out=acc_c)
    acc_s, y_s = poison((M, N), torch.int32), poison((M, N), torch.bfloat16)
    print(f"static entry point M={M} K={K} N={N}", flush=True)
    assert _static(xd, wd, swd, y_s, acc=acc_s) == 0
    torch.cuda.synchronize()
    assert_same("y", host_bf16_bits(y_s), host_bf16_bits(y_c))
    assert_same("acc", host(acc_s), host(acc_c))
    assert_same("acc vs oracle", host(acc_s), il.linear_w8a8(x, w, sw)["acc"])
    # the exported payload: same bytes as the context call's
    xq_c, xs_c = poison((M, K), torch.int8), poison((M,), torch.float32)
    xq_s, xs_s = poison((M, K), torch.int8), poison((M,), torch.float32)
    wq.wq_fused_quant_matmul(xd, wd, swd, y=y_c, x_q_out=xq_c, x_scale_out=xs_c)
    assert _static(xd, wd, swd, y_s, xq=xq_s, xs=xs_s) == 0
    torch.cuda.synchronize()
    assert_same("x_q", host(xq_s), host(xq_c))
    assert_same("x_scale", host(xs_s), host(xs_c))


def test_static_entry_two_calls_second_smaller():
    _compare(200, 4096, 1024, 1)   # staged in the static buffer (800 KiB of payload)
    _compare(96, 2048, 512, 2)     # smaller, on the buffer the first call left behind


def test_static_entry_one_launch_size():
    _compare(8, 4096, 1024, 3)


def test_static_entry_refuses_sizes_beyond_its_buffer():
    N = 64
    for M, K in ((4100, 4096), (16400, 16)):   # payload above 16 MiB; scales above 16384 rows
        x = torch.zeros((M, K), dtype=torch.bfloat16, device=DEV)
        w = torch.zeros((N, K), dtype=torch.int8, device=DEV)
        sw = torch.ones((N,), dtype=torch.float32, device=DEV)
        y = poison((M, N), torch.bfloat16)
        assert _static(x, w, sw, y) == WQ_ERR_WORKSPACE
        torch.cuda.synchronize()
        assert (host(y.view(torch.int16)) == -0x5A5B).all()  # 0xA5A5: nothing written
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    w = torch.zeros((16, 64), dtype=torch.int8, device=DEV)
    assert _static(x, w, torch.ones(16, device=DEV), torch.empty((4, 16), dtype=torch.bfloat16, device=DEV),
                   device=torch.cuda.device_count()) == WQ_ERR_DEVICE
