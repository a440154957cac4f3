"""GPU parity of the FP8 per-token-group quant and its packed UE8M0 scales.

Bit-exact: E4M3 payload bytes and every int32 word of the packed storage (including
the zeroed pack tails and token-padding words), checked on a poisoned buffer.
"""

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import DEV, bf16_dev, host
from oracle import fp8_group as fg

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
