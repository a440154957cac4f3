"""Pins for oracle/fp8_group.py: group quant, packed UE8M0 layout, contraction."""

import os
from fractions import Fraction as F

import numpy as np
import pytest

import synthetic as syn
from exact import bf16_bits_of, f32_bits, rn_bf16
from oracle import fp8_group as fg
from oracle import numerics as nm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_lines(name):
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or not line.strip():
            continue
        yield line.strip()


def _groups():
    out = []
    for line in _golden_lines("fp8_groups.txt"):
        name, xs, eb, cs = [p.strip() for p in line.split("|")]
        out.append((name, [float(v) for v in xs.split()], int(eb, 16), [int(c, 16) for c in cs.split()]))
    return out


@pytest.mark.parametrize("grp", _groups(), ids=lambda g: g[0])
def test_hand_groups(grp):
    name, xs, ebyte, codes = grp
    x = np.zeros((1, 1, 128), np.uint16)
    for i, v in enumerate(xs):
        x[0, 0, i] = bf16_bits_of(v) if v != 0 or str(v)[0] != "-" else 0x8000
    payload, eb = fg.group_quant_fp8(x)
    assert int(eb[0, 0, 0]) == ebyte
    assert payload[0, 0, : len(codes)].tolist() == codes
    assert (payload[0, 0, len(xs):] == 0).all()


def test_packed_layout_worked_example():
    words = None
    for line in _golden_lines("packed_layout_d640.txt"):
        if line.startswith("words_hex:"):
            words = [int(w, 16) for w in line.split(":", 1)[1].split()]
    x = np.zeros((1, 1, 640), np.uint16)
    x[0, 0, ::128] = bf16_bits_of(1.0)  # absmax 1.0 in each of the 5 groups
    _, storage, eb = fg.group_quant_fp8_packed(x)
    assert storage.shape == (1, 2, 4) and storage.dtype == np.int32
    assert [int(v) & 0xFFFFFFFF for v in storage.reshape(-1)] == words


def test_empty_token_shape():
    for line in _golden_lines("empty_tokens_shape.txt"):
        lhs, rhs = line.split("->")
        kv = dict(p.split("=") for p in lhs.split())
        T, G, D = int(kv["T"]), int(kv["G"]), int(kv["D"])
        x = np.zeros((T, G, D), np.uint16)
        payload, storage, _ = fg.group_quant_fp8_packed(x)
        view = fg.logical_view(storage, T)
        assert list(view.shape) == [int(v) for v in rhs.split()]
        assert payload.shape == (T, G, D)


def test_pack_address_formula_bruteforce_and_roundtrip():
    g = np.random.default_rng(7)
    for T, G, HG in [(1, 1, 1), (5, 3, 3), (7, 2, 9), (8, 8, 32), (3, 3, 4)]:
        eb = g.integers(0, 255, (T, G, HG)).astype(np.uint8)
        st = fg.pack_ue8m0(eb)
        PH, TA = (HG + 3) // 4, (T + 3) // 4 * 4
        assert st.shape == (G, PH, TA)
        raw = st.reshape(-1).view(np.uint8)
        seen = np.zeros(raw.size, bool)
        for t in range(T):
            for gg in range(G):
                for h in range(HG):
                    off = ((gg * PH + h // 4) * TA + t) * 4 + h % 4
                    assert raw[off] == eb[t, gg, h]
                    seen[off] = True
        assert (raw[~seen] == 0).all()  # pack tails and token padding are zero
        assert np.array_equal(fg.unpack_ue8m0(st, T, HG), eb)
        v = fg.logical_view(st, T)
        assert v.shape == (T, G, PH)
        assert tuple(s // 4 for s in v.strides) == (1, PH * TA, TA)


def test_group_quant_invariants_and_error_bound():
    for T in (1, 7):
        x = syn.fp8_group_x(T, G=2, D=512, layout_variant=True)
        payload, eb = fg.group_quant_fp8(x)
        e = eb.astype(np.int64) - 127
        xf = nm.bf16_to_f32(x).astype(np.float64).reshape(T, 2, 4, 128)
        a = np.abs(xf).max(-1)
        assert (np.ldexp(448.0, e) >= a).all() and (np.ldexp(448.0, e - 1) < a).all()
        assert (eb <= 254).all()
        assert not np.isin(payload, [0x7F, 0xFF]).any()
        dq = nm.e4m3_decode(payload).reshape(T, 2, 4, 128) * np.ldexp(1.0, e)[..., None]
        # E4M3 keeps 3 fraction bits: relative error <= 2^-4 for normals, absolute
        # error <= 2^-10 * 2^e in the subnormal range
        err = np.abs(dq - xf)
        bound = np.maximum(np.abs(xf) * 2.0 ** -4, np.ldexp(1.0, e - 10)[..., None])
        assert (err <= bound).all()


def _exact_contraction(xq, xs_f, wq, ws):
    T, G, D = xq.shape
    N = wq.shape[1]
    xv = nm.e4m3_decode(xq)
    wv = nm.e4m3_decode(wq)
    out = np.zeros((T, G, N), np.uint16)
    for t in range(T):
        for g in range(G):
            for n in range(N):
                tot = F(0)
                for k in range(D):
                    kb = k // 128
                    tot += F(float(xv[t, g, k])) * F(float(wv[g, n, k])) * F(float(xs_f[t, g, kb])) * F(float(ws[g, n // 128, kb]))
                r = rn_bf16(tot)
                out[t, g, n] = 0 if r == 0 else f32_bits(float(r)) >> 16
    return out


def test_contraction_against_exact_fractions():
    g = np.random.default_rng(9)
    T, G, D, N = 2, 2, 256, 128
    xq = syn.random_e4m3_codes(g, (T, G, D))
    xs_f = np.ldexp(1.0, g.integers(-6, 6, (T, G, D // 128)))
    wq = syn.random_e4m3_codes(g, (G, N, D))
    ws = np.ldexp(np.float32(1.0), g.integers(-3, 4, (G, N // 128, D // 128))).astype(np.float32)
    y = fg.fp8_grouped_contraction(xq, xs_f, wq, ws)
    want = _exact_contraction(xq, xs_f, wq, ws)
    # the oracle's only rounding before bf16 is the float64 sum of block partials
    assert (nm.bf16_ulp_distance(y, want) == 0).mean() > 0.999
    assert nm.bf16_ulp_distance(y, want).max() <= 1


def test_contraction_integer_special_case():
    # unit scales and integer-valued codes (1.0 = 0x38, 2.0 = 0x40, -1.0 = 0xB8):
    # the result is an exact small integer
    T, G, D, N = 3, 1, 256, 128
    g = np.random.default_rng(10)
    xq = g.choice(np.array([0x38, 0x40, 0xB8, 0x00], np.uint8), (T, G, D))
    wq = g.choice(np.array([0x38, 0xB8, 0x00], np.uint8), (G, N, D))
    y = fg.fp8_grouped_contraction(xq, np.ones((T, G, 2)), wq, np.ones((G, 1, 2), np.float32))
    ints = nm.e4m3_decode(xq)[:, 0, :] @ nm.e4m3_decode(wq)[0].T
    assert np.array_equal(nm.bf16_to_f32(y[:, 0, :]).astype(np.float64), ints)  # |.| <= 512 is exact in bf16


def test_packed_and_f32_scales_give_identical_bytes():
    T, G, D, N = 5, 2, 512, 128
    x = syn.fp8_group_x(T, G=G, D=D)
    payload, storage, eb = fg.group_quant_fp8_packed(x)
    wq, ws = syn.fp8_weights(G=G, N=N, D=D)
    y_f32 = fg.fp8_grouped_contraction(payload, fg.ebyte_to_scale(eb), wq, ws)
    y_pk = fg.contraction_from_packed(payload, storage, T, wq, ws)
    assert np.array_equal(y_f32, y_pk)


# ---- MX-like 32-element blocks ("DeepSeek V4 950" section 2.1) ---------------------------

def _mx_golden():
    lines = list(_golden_lines("mx_blocks.txt"))
    row = {int(k): float(v) for k, v in (e.split("=") for e in lines[0].split("|")[1].split())}
    out = {}
    for line in lines[1:]:
        name, bs, cs = [p.strip() for p in line.split("|")]
        out[name] = ([int(b, 16) for b in bs.split()], {int(k): int(v, 16) for k, v in (e.split("=") for e in cs.split())})
    return row, out


@pytest.mark.parametrize("group", [128, 32])
def test_mx_hand_row(group):
    row, want = _mx_golden()
    x = np.zeros((1, 1, 128), np.uint16)
    for i, v in row.items():
        x[0, 0, i] = bf16_bits_of(v)
    payload, eb = fg.group_quant_fp8(x, group)
    bytes_want, codes_want = want[f"group{group}"]
    assert eb[0, 0].tolist() == bytes_want
    for i, c in codes_want.items():
        assert int(payload[0, 0, i]) == c, (i, hex(int(payload[0, 0, i])), hex(c))
    zero = [i for i in range(128) if i not in row]
    assert not payload[0, 0, zero].any()


def test_mx_blocks_invariants():
    x = syn.fp8_group_x(9, G=2, D=512, layout_variant=True)
    payload, eb = fg.group_quant_fp8(x, 32)
    a = np.abs(nm.bf16_to_f32(x).astype(np.float64)).reshape(9, 2, 16, 32).max(axis=-1)
    e = eb.astype(np.int64) - 127
    live = e > -127
    assert np.all(np.ldexp(448.0, e[live]) >= a[live])          # 2^e covers absmax / 448
    assert np.all(np.ldexp(448.0, e[live] - 1) < a[live])       # and is the smallest power that does
    dec = nm.e4m3_decode(payload).reshape(9, 2, 16, 32)
    assert np.all(np.abs(dec) <= 448)                           # never saturates


def test_mx_blocks_equal_groups_of_128_when_every_block_holds_the_max():
    """If each 32-element block holds an element equal to its 128-group's absmax, both
    block sizes pick the same exponent, so the bytes repeat 4 times and the codes agree."""
    x = syn.fp8_group_x(5, G=3, D=384)
    T, G, D = x.shape
    xf = nm.bf16_to_f32(x).astype(np.float32).reshape(T, G, D // 128, 4, 32)
    m = np.abs(xf).max(axis=(-1, -2))                           # [T, G, HG]
    xf[:, :, :, :, 0] = m[:, :, :, None]                        # the group's absmax in every block
    # every value is still a bf16 value, so its bits are the high half of the f32 bits
    xb = (np.ascontiguousarray(xf.reshape(T, G, D)).view(np.uint32) >> 16).astype(np.uint16)
    p128, e128 = fg.group_quant_fp8(xb, 128)
    p32, e32 = fg.group_quant_fp8(xb, 32)
    assert np.array_equal(p32, p128)
    assert np.array_equal(e32, np.repeat(e128, 4, axis=-1))


def _exact_mx(xq, xs_f, wq, ws):
    xv, wv = nm.e4m3_decode(xq), nm.e4m3_decode(wq)
    T, G, D = xq.shape
    N = wq.shape[1]
    out = np.zeros((T, G, N), np.uint16)
    for t in range(T):
        for g in range(G):
            for n in range(N):
                tot = F(0)
                for k in range(D):
                    kb = k // 32
                    tot += F(float(xv[t, g, k])) * F(float(wv[g, n, k])) * F(float(xs_f[t, g, kb])) * F(float(ws[g, n, kb]))
                r = rn_bf16(tot)
                out[t, g, n] = 0 if r == 0 else f32_bits(float(r)) >> 16
    return out


def test_mx_contraction_against_exact_fractions():
    g = np.random.default_rng(33)
    T, G, D, N = 2, 2, 128, 6
    xq = syn.random_e4m3_codes(g, (T, G, D))
    xs_f = np.ldexp(1.0, g.integers(-6, 6, (T, G, D // 32)))
    wq = syn.random_e4m3_codes(g, (G, N, D))
    ws = np.ldexp(1.0, g.integers(-3, 4, (G, N, D // 32)))
    y = fg.mx_contraction(xq, xs_f, wq, ws)
    want = _exact_mx(xq, xs_f, wq, ws)
    assert nm.bf16_ulp_distance(y, want).max() <= 1
    assert (nm.bf16_ulp_distance(y, want) == 0).mean() > 0.99


def test_mx_contraction_equals_128_blocks_when_scales_repeat():
    """Scales constant over each 128-deep block (and, for the weights, over 128 columns):
    the MX contraction is the 128-block contraction, byte for byte."""
    g = np.random.default_rng(34)
    T, G, D, N = 3, 2, 256, 128
    xq = syn.random_e4m3_codes(g, (T, G, D))
    wq = syn.random_e4m3_codes(g, (G, N, D))
    xs128 = np.ldexp(1.0, g.integers(-5, 5, (T, G, D // 128)))
    ws128 = np.ldexp(np.float32(1.0), g.integers(-3, 4, (G, N // 128, D // 128))).astype(np.float32)
    y128 = fg.fp8_grouped_contraction(xq, xs128, wq, ws128)
    xs32 = np.repeat(xs128, 4, axis=-1)
    ws32 = np.repeat(np.repeat(ws128.astype(np.float64), 128, axis=1), 4, axis=-1)
    y32 = fg.mx_contraction(xq, xs32, wq, ws32)
    assert np.array_equal(y32, y128)
