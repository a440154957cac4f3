"""GPU parity of the MoE W8A8 expert block: expert sort, fused RMSNorm+quant with the
expert-sorted gather, segmented gate/up GEMM with the SwiGLU epilogue, INT8 requant of
the f32 activation, segmented down GEMM.

Bit-exact: sort outputs, INT8 payloads and scales, the f32 SwiGLU activations (same
fixed operation sequence on both sides).  BF16 outputs within 1 bf16 ulp.
"""

import numpy as np
import pytest
import torch

import synthetic as syn
from gpu_util import DEV, assert_same, bf16_dev, dev, host, host_bf16_bits
from oracle import int8_linear as il
from oracle import moe
from oracle import numerics as nm

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    import fp8_dynamic_quant_amd as wq


@pytest.mark.parametrize("T,E,topk,seed", [(256, 256, 8, 51), (37, 16, 3, 1), (1, 4, 4, 2), (0, 8, 2, 3)])
def test_expert_sort(T, E, topk, seed):
    ids = syn.zipf_topk_ids((9, seed), T, E, topk) if T > 0 else np.zeros((0, topk), np.int32)
    perm, row_token, offsets = wq.wq_moe_sort(dev(ids), E)
    torch.cuda.synchronize()
    p_ref, off_ref = moe.expert_sort(ids, E)
    assert np.array_equal(host(perm), p_ref)
    assert np.array_equal(host(row_token), p_ref // topk)
    assert np.array_equal(host(offsets), off_ref)


def test_expert_sort_drops_out_of_range_ids():
    """Ids outside [0, E) drop their pairs: the kept pairs sort as the oracle sorts them,
    offsets[E] counts them, and the slots past them hold perm = -1, row_token = 0."""
    T, E, topk = 40, 16, 4
    ids = syn.zipf_topk_ids((9, 7), T, E, topk)
    ids[3, 1], ids[17, 0], ids[39, 3] = -1, E, 1 << 20
    perm, row_token, offsets = wq.wq_moe_sort(dev(ids), E)
    torch.cuda.synchronize()
    p_ref, off_ref = moe.expert_sort(ids, E, drop_invalid=True)
    kept = p_ref.size
    assert kept == T * topk - 3 and off_ref[E] == kept
    assert np.array_equal(host(offsets), off_ref)
    assert np.array_equal(host(perm)[:kept], p_ref)
    assert np.array_equal(host(row_token)[:kept], p_ref // topk)
    assert (host(perm)[kept:] == -1).all() and (host(row_token)[kept:] == 0).all()


@pytest.mark.parametrize("T,H", [(16, 512), (8, 4096), (5, 2064), (1025, 1024), (1100, 272)])
def test_rmsnorm_quant_gather(T, H):
    h = syn.activations((60, T, H), T, H)
    gamma = syn.to_bf16_bits(np.random.default_rng(T).uniform(0.5, 1.5, H).astype(np.float32))
    ids = syn.zipf_topk_ids((61, T), T, 8, 4)
    p_ref, _ = moe.expert_sort(ids, 8)
    tok = p_ref // 4
    q, s = wq.wq_dynamic_quant(bf16_dev(h), rms_gamma=bf16_dev(gamma), row_index=dev(tok.astype(np.int32)))
    torch.cuda.synchronize()
    v, v_alt, flagged = moe.rmsnorm_f32(h, gamma, alternates=True)
    q_ref, s_ref = _rms_quant_ref(v, v_alt, flagged, tok, host(q), host(s))
    assert np.array_equal(host(s).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(q), q_ref)


def _rms_quant_ref(v, v_alt, flagged, tok, q_got, s_got):
    """The oracle's (q, s) for the RMSNorm rows of tokens `tok`: the primary reading, or for
    a flagged token (oracle.moe.rmsnorm_mean_squares) whichever of the two readings the kernel's
    row matches.  Rows that match neither keep the primary, so assert_same reports them."""
    q_ref, s_ref = il.quant_int8_per_token(v[tok], is_bf16_bits=False)
    if flagged[tok].any():
        q_alt, s_alt = il.quant_int8_per_token(v_alt[tok], is_bf16_bits=False)
        take = flagged[tok] & (s_got.view(np.uint32) == s_alt.view(np.uint32)) & (q_got == q_alt).all(1)
        q_ref[take], s_ref[take] = q_alt[take], s_alt[take]
    return q_ref, s_ref


def _run_block_gpu(d, E, frag=False):
    ids_d = dev(d["ids"])
    perm, row_token, offsets = wq.wq_moe_sort(ids_d, E)
    q1, s1 = wq.wq_dynamic_quant(bf16_dev(d["h"]), rms_gamma=bf16_dev(d["gamma"]), row_index=row_token)
    w13, sw13, w2, sw2 = d["w13_d"], d["sw13_d"], d["w2_d"], d["sw2_d"]
    if frag:
        w13, w2 = wq.wq_pack_weight_i8(w13), wq.wq_pack_weight_i8(w2)
    hmid = wq.wq_quant_matmul(q1, s1, w13, sw13, seg_offsets=offsets, epilogue=wq.WQ_EPI_SWIGLU_F32,
                              b_fragment=frag)
    q2, s2 = wq.wq_dynamic_quant(hmid)
    y = wq.wq_quant_matmul(q2, s2, w2, sw2, seg_offsets=offsets, b_fragment=frag)
    torch.cuda.synchronize()
    return dict(perm=perm, offsets=offsets, q1=q1, s1=s1, h=hmid, q2=q2, s2=s2, y=y)


@pytest.mark.parametrize("T,H,I,E,topk,frag", [(32, 256, 128, 8, 2, False), (64, 1024, 512, 32, 8, False),
                                              (300, 512, 256, 4, 2, False), (64, 1024, 512, 32, 8, True),
                                              (300, 512, 256, 4, 2, True)])
def test_moe_block_against_oracle(T, H, I, E, topk, frag):
    d = syn.moe_inputs(seed=T, T=T, H=H, I=I, E=E, TOPK=topk)
    d.update(w13_d=dev(d["w13"]), sw13_d=dev(d["sw13"]), w2_d=dev(d["w2"]), sw2_d=dev(d["sw2"]))
    g = _run_block_gpu(d, E, frag)
    # a token whose RMSNorm row is flagged takes the reading the kernel's rows match
    v, v_alt, flagged = moe.rmsnorm_f32(d["h"], d["gamma"], alternates=True)
    perm_ref, _ = moe.expert_sort(d["ids"], E)
    tok = perm_ref // topk
    _, s1_ref = _rms_quant_ref(v, v_alt, flagged, tok, host(g["q1"]), host(g["s1"]))
    _, s1_alt = il.quant_int8_per_token(v_alt[tok], is_bf16_bits=False)
    for t in np.flatnonzero(flagged):
        rows = np.flatnonzero(tok == t)
        if rows.size and (s1_ref[rows].view(np.uint32) == s1_alt[rows].view(np.uint32)).all():
            v[t] = v_alt[t]
    r = moe.moe_block(d["h"], d["gamma"], d["ids"], d["w13"], d["sw13"], d["w2"], d["sw2"], keep=True, v_rows=v)
    assert_same("perm", host(g["perm"]), r["perm"])
    assert_same("offsets", host(g["offsets"]), r["offsets"])
    assert_same("s1", host(g["s1"]), r["s1"])
    assert_same("q1", host(g["q1"]), r["q1"])
    assert_same("h", host(g["h"]), r["h"])
    assert_same("s2", host(g["s2"]), r["s2"])
    assert_same("q2", host(g["q2"]), r["q2"])
    assert nm.bf16_ulp_distance(host_bf16_bits(g["y"]), r["y"]).max() <= 1


def test_moe_block_full_size_sampled_experts():
    """DeepSeek-V4 shape (256 tokens, hidden 4096, 256 experts of 2x2048, top-8 Zipf(1.1)):
    weights generated on the GPU from a seeded generator, then the rows of three experts
    (the busiest, a median one and a one-row one) checked against the oracle."""
    T, H, I, E, topk = 256, 4096, 2048, 256, 8
    d = syn.moe_inputs(seed=51, T=T, H=H, I=I, E=E, TOPK=topk, weights=False)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(5151)
    w13 = torch.randint(-127, 128, (E, 2 * I, H), generator=gen, device=DEV, dtype=torch.int8)
    w2 = torch.randint(-127, 128, (E, H, I), generator=gen, device=DEV, dtype=torch.int8)
    sw13 = torch.rand((E, 2 * I), generator=gen, device=DEV) * 9e-3 + 1e-3
    sw2 = torch.rand((E, H), generator=gen, device=DEV) * 9e-3 + 1e-3
    d.update(w13_d=w13, sw13_d=sw13, w2_d=w2, sw2_d=sw2)
    g = _run_block_gpu(d, E)
    offsets = host(g["offsets"])
    counts = np.diff(offsets)
    perm_ref, off_ref = moe.expert_sort(d["ids"], E)
    assert np.array_equal(offsets, off_ref) and np.array_equal(host(g["perm"]), perm_ref)
    assert counts.sum() == T * topk
    order = np.argsort(counts)
    busiest = int(order[-1])
    one_row = int(np.flatnonzero(counts == 1)[0]) if (counts == 1).any() else int(order[0])
    median = int(order[np.searchsorted(counts[order], np.median(counts[counts > 0]))])
    v, v_alt, flagged = moe.rmsnorm_f32(d["h"], d["gamma"], alternates=True)
    for e in {busiest, one_row, median}:
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        tok = perm_ref[lo:hi] // topk
        q1, s1 = _rms_quant_ref(v, v_alt, flagged, tok, host(g["q1"][lo:hi]), host(g["s1"][lo:hi]))
        assert_same(f"q1[e={e}]", host(g["q1"][lo:hi]), q1)
        acc13 = il.gemm_int8_int32(q1, host(w13[e]))
        hmid = moe.silu_mul_f32(acc13, s1, np.broadcast_to(host(sw13[e]), (hi - lo, 2 * I)))
        assert_same(f"h[e={e}, rows {lo}:{hi}]", host(g["h"][lo:hi]), hmid)
        q2, s2 = il.quant_int8_per_token(hmid, is_bf16_bits=False)
        assert_same(f"q2[e={e}]", host(g["q2"][lo:hi]), q2)
        y = il.epilogue_bf16(il.gemm_int8_int32(q2, host(w2[e])), s2, host(sw2[e]))
        assert nm.bf16_ulp_distance(host_bf16_bits(g["y"][lo:hi]), y).max() <= 1


BOUNDARY_COUNTS = [0, 1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 129]
# experts of three to five 128-row tiles between small ones: the tiled kernel's work list
# names a tile by its index within the expert
MANY_TILE_COUNTS = [300, 0, 513, 1, 256, 257, 16, 384]
# both sides of the 128-row mark, where an expert's rows become one 256-row tile, and of
# the 256- and 384-row marks, where a 128-row tile follows the 256-row ones
TALL_COUNTS = [127, 128, 129, 130, 17, 160, 192, 255, 0, 256, 257, 260, 383, 384, 385, 640]


@pytest.mark.parametrize("counts", [BOUNDARY_COUNTS, MANY_TILE_COUNTS, TALL_COUNTS],
                         ids=["boundary", "many_tiles", "tall_tiles"])
@pytest.mark.parametrize("frag", [False, True])
@pytest.mark.parametrize("epi", ["bf16", "swiglu"])
def test_segments_across_the_small_expert_boundary(epi, frag, counts, N=512):
    """Expert row counts on both sides of the 16-row split between the weight-streaming
    kernel and the tiled one, and of the tiled kernel's 64- and 128-row marks (0, 1, 15,
    16, 17, 31, 32, 33, 63, 64, 65, 129 rows); experts of several 128-row tiles; and
    127 .. 640 rows around the marks where the tiled kernel takes an expert's rows as
    256-row tiles (more than 128 rows in a unit of 256) or as a last 128-row tile.
    K = 1024 so both kernels take part; every expert's rows against the oracle's dense
    per-expert product.
    frag: the expert weights cast to fragment order (both kernels read that layout)."""
    counts = np.array(counts, np.int64)
    E, K = counts.size, 1024
    M = int(counts.sum())
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    x = syn.activations((62, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    q, s = il.quant_int8_per_token(x)
    w = np.empty((E, N, K), np.int8)
    sw = np.empty((E, N), np.float32)
    for e in range(E):
        w[e], sw[e] = syn.int8_weights((63, e), N, K)
    wd = wq.wq_pack_weight_i8(dev(w)) if frag else dev(w)
    if epi == "bf16":
        y = wq.wq_quant_matmul(dev(q), dev(s), wd, dev(sw), seg_offsets=dev(offsets), b_fragment=frag)
    else:
        y = wq.wq_quant_matmul(dev(q), dev(s), wd, dev(sw), seg_offsets=dev(offsets), epilogue=wq.WQ_EPI_SWIGLU_F32,
                               b_fragment=frag)
    torch.cuda.synchronize()
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        acc = il.gemm_int8_int32(q[lo:hi], w[e])
        if epi == "bf16":
            ref = il.epilogue_bf16(acc, s[lo:hi], sw[e])
            d = nm.bf16_ulp_distance(host_bf16_bits(y[lo:hi]), ref)
            assert d.max() <= 1, f"expert {e} ({hi - lo} rows): max ulp {d.max()}"
        else:
            ref = moe.silu_mul_f32(acc, s[lo:hi], np.broadcast_to(sw[e], (hi - lo, N)))
            assert_same(f"h[expert {e}, {hi - lo} rows]", host(y[lo:hi]), ref)


@pytest.mark.parametrize("counts", [BOUNDARY_COUNTS, MANY_TILE_COUNTS, TALL_COUNTS],
                         ids=["boundary", "many_tiles", "tall_tiles"])
@pytest.mark.parametrize("epi", ["bf16", "swiglu"])
def test_expected_rows_hint_gives_the_same_bytes(epi, counts):
    """The expected-rows hint (W8A8 article, section 五: the grouped GEMM's tiling chosen
    from the expected tokens per expert) only chooses launches: no streaming kernel above
    64 expected rows, no 256-row tiles at most 128.  Every hint, right or wrong for the
    actual counts, gives the bytes of the call without one (fragment-order weights)."""
    counts = np.array(counts, np.int64)
    E, K, N = counts.size, 1024, 512
    M = int(counts.sum())
    offsets = dev(np.concatenate([[0], np.cumsum(counts)]).astype(np.int64))
    x = syn.activations((64, M, K), M, K, outlier_frac=0.01, outlier_mul=20.0)
    q, s = il.quant_int8_per_token(x)
    w = np.empty((E, N, K), np.int8)
    sw = np.empty((E, N), np.float32)
    for e in range(E):
        w[e], sw[e] = syn.int8_weights((65, e), N, K)
    wd = wq.wq_pack_weight_i8(dev(w))
    kw = {} if epi == "bf16" else {"epilogue": wq.WQ_EPI_SWIGLU_F32}
    base = host(wq.wq_quant_matmul(dev(q), dev(s), wd, dev(sw), seg_offsets=offsets, b_fragment=True,
                                   **kw).view(torch.uint8))
    for hint in (1, 16, 64, 65, 128, 129, 100000):
        got = host(wq.wq_quant_matmul(dev(q), dev(s), wd, dev(sw), seg_offsets=offsets, b_fragment=True,
                                      expected_rows=hint, **kw).view(torch.uint8))
        assert np.array_equal(got, base), f"expected_rows={hint}"


@pytest.mark.parametrize("frag", [False, True])
def test_segments_ragged_columns(frag):
    """bf16 expert segments with N = 400 (the last column tile is 16 columns wide, its
    weight rows clamped) over 128-row and 256-row tiles."""
    test_segments_across_the_small_expert_boundary("bf16", frag, [129, 1, 300, 17, 64], N=400)
