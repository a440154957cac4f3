"""Pins for oracle/moe.py: expert sort, RMSNorm, SiLU*up, and the segmented GEMMs."""

import math

import numpy as np
import pytest

import synthetic as syn
from exact import bf16_bits_of
from oracle import int8_linear as il
from oracle import moe
from oracle import numerics as nm


def test_sort_against_python_sorted():
    ids = syn.zipf_topk_ids((77, 1), 32, 16, 4)
    perm, off = moe.expert_sort(ids, 16)
    flat = ids.reshape(-1)
    want = sorted(range(flat.size), key=lambda p: (int(flat[p]), p))
    assert perm.tolist() == want
    assert off[0] == 0 and off[-1] == flat.size and (np.diff(off) >= 0).all()
    for e in range(16):
        assert (flat[perm[off[e]:off[e + 1]]] == e).all()
    # every token's ids are distinct
    assert all(len(set(r)) == 4 for r in ids.tolist())


def test_rmsnorm_constant_row_closed_form():
    K = 256
    c = 3.0
    x = np.full((1, K), bf16_bits_of(c), np.uint16)
    gamma = np.full(K, bf16_bits_of(1.5), np.uint16)
    v = moe.rmsnorm_f32(x, gamma)
    want = c / math.sqrt(c * c + 1e-6) * 1.5
    assert np.abs(v.astype(np.float64) - want).max() <= 4 * np.spacing(np.float32(want))


def test_rmsnorm_against_float64_formula():
    h = syn.activations((78, 1), 4, 512)
    gamma = syn.to_bf16_bits(np.random.default_rng(1).uniform(0.5, 1.5, 512).astype(np.float32))
    v = moe.rmsnorm_f32(h, gamma).astype(np.float64)
    xf = nm.bf16_to_f32(h).astype(np.float64)
    gf = nm.bf16_to_f32(gamma).astype(np.float64)
    ref = xf / np.sqrt((xf ** 2).mean(1, keepdims=True) + 1e-6) * gf
    assert (np.abs(v - ref) <= 4 * np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)).all()


def test_silu_mul_special_values_and_accuracy():
    acc = np.array([[0, 1000, -1000, 10 ** 6, -(10 ** 6), 1, 1, 1, 1, 1]], np.int32)  # I = 5
    s = np.array([0.01], np.float32)
    sw = np.ones((1, 10), np.float32)
    h = moe.silu_mul_f32(acc, s, sw)[0]
    g = acc[0, :5] * 0.01
    ref = g / (1 + np.exp(-g)) * 0.01
    assert h[0] == 0.0
    assert abs(h[1] - ref[1]) <= 2 * np.spacing(np.float32(ref[1]))
    assert h[3] == np.float32(np.float32(10 ** 4) * np.float32(0.01))  # silu(g) = g for large g
    assert h[4] == 0.0 and math.copysign(1.0, h[4]) < 0  # silu(g) -> -0 for g << 0
    rng = np.random.default_rng(2)
    acc = rng.integers(-600000, 600000, (8, 64)).astype(np.int32)
    s = rng.uniform(0.01, 0.05, 8).astype(np.float32)
    sw = rng.uniform(1e-3, 1e-2, (8, 64)).astype(np.float32)
    h = moe.silu_mul_f32(acc, s, sw).astype(np.float64)
    val = acc * s[:, None].astype(np.float64) * sw
    gg, uu = val[:, :32], val[:, 32:]
    ref = gg / (1 + np.exp(-gg)) * uu
    assert np.allclose(h, ref, rtol=1e-5, atol=1e-30)


def test_block_segments_equal_dense_per_row():
    d = syn.moe_inputs(seed=3, T=16, H=256, I=128, E=8, TOPK=2)
    r = moe.moe_block(d["h"], d["gamma"], d["ids"], d["w13"], d["sw13"], d["w2"], d["sw2"], keep=True)
    perm, off = r["perm"], r["offsets"]
    flat = d["ids"].reshape(-1)
    tok = perm // 2
    # row r is handled by expert flat[perm[r]]: recompute each row with its own expert
    for row in range(perm.size):
        e = int(flat[perm[row]])
        assert off[e] <= row < off[e + 1]
        acc13 = il.gemm_int8_int32(r["q1"][row:row + 1], d["w13"][e])
        assert np.array_equal(acc13, r["acc13"][row:row + 1])
        acc2 = il.gemm_int8_int32(r["q2"][row:row + 1], d["w2"][e])
        assert np.array_equal(acc2, r["acc2"][row:row + 1])
    # rows of one token share the RMSNorm+quant result
    q1_tok, s1_tok = il.quant_int8_per_token(r["v"], is_bf16_bits=False)
    assert np.array_equal(r["q1"], q1_tok[tok]) and np.array_equal(r["s1"], s1_tok[tok])
    assert r["y"].shape == (32, 256)


def test_rmsnorm_boundary_flag():
    """A18: [1, 1, 2^-12, 2^-12] has sum of squares 2 + 2^-23, so the mean square is exactly
    halfway between 0.5 and 0.5 + 2^-24: ties to even give 0.5, and a float64 sum in another
    order could land on either side, so the row is flagged with the other neighbour.  A row
    of N(0,1) values far from such a boundary is not flagged."""
    x = np.array([[0x3F80, 0x3F80, 0x3980, 0x3980]], np.uint16)
    ms, other, flagged = moe.rmsnorm_mean_squares(x)
    assert ms[0] == np.float32(0.5) and other[0] == np.float32(0.5 + 2.0 ** -24) and flagged[0]
    v, v_alt, fl = moe.rmsnorm_f32(x, np.full(4, bf16_bits_of(1.0), np.uint16), alternates=True)
    assert fl[0] and not np.array_equal(v, v_alt)
    h = syn.activations((78, 2), 32, 4096)
    ms, other, flagged = moe.rmsnorm_mean_squares(h)
    assert not flagged.any() and np.array_equal(ms, other)


def test_rmsnorm_other_summation_orders_stay_within_the_flag():
    """Recursive float64 sums in forward, reverse and sorted order all give the oracle's mean
    square, or the flagged neighbour."""
    h = syn.activations((78, 3), 64, 2048)
    ms, other, _ = moe.rmsnorm_mean_squares(h)
    xf = nm.bf16_to_f32(h).astype(np.float64)
    for order in (lambda r: r, lambda r: r[::-1], np.sort, lambda r: np.sort(r)[::-1]):
        for m in range(h.shape[0]):
            acc = 0.0
            for v in order(xf[m] * xf[m]):
                acc += float(v)
            got = np.float32(acc / h.shape[1])
            assert got == ms[m] or got == other[m]


def test_expert_sort_drop_invalid():
    """Out-of-range ids: an error by default; with drop_invalid their pairs take no row and
    the kept pairs keep their stable order."""
    ids = np.array([[2, -1], [0, 2], [5, 1]], np.int32)
    with pytest.raises(ValueError):
        moe.expert_sort(ids, 4)
    perm, off = moe.expert_sort(ids, 4, drop_invalid=True)
    assert perm.tolist() == [2, 5, 0, 3] and off.tolist() == [0, 1, 2, 4, 4]
