"""Seeded synthetic inputs shaped like the DeepSeek-V4 projections.

Shared by the tests, the oracle checks and the benchmark.  This module only
draws random numbers and rounds them to storage types (bf16 rounding is done by
torch); it holds none of the quantisation, GEMM or packing arithmetic.

Every generator takes an integer key tuple and uses
numpy.random.Generator(PCG64(SeedSequence(key))), so a case is reproduced from
its key alone.

Workloads (sizes from "DeepSeek-V4 W8A8 性能分析" sections 三-五 and the
SGLang PR #34277 wrapper):
* tiny linear: X [4, 256], 1% of entries scaled x50; W [256 -> 512];
* wq_a decode linear: X [M, 4096], M in {1,2,4,7,8,16,32,64}, 0.5% outliers x30;
  W [4096 -> 1024];
* wq_b wide linear: X [M, 1024], M in {1,8,64,512,8192}; W [1024 -> 32768];
* FP8 group quant: X [T, 8, 4096] = N(0,1) * U(0.1,10) per token,
  T in {0,1,7,64,512}; FP8 weights [8, 1024, 4096] with 128x128 power-of-two
  block scales;
* MoE block: T=256 tokens, hidden 4096, 256 experts, top-8 ids from a
  truncated Zipf(1.1) law, W13 [256, 4096, 4096], W2 [256, 4096, 2048].
"""

from __future__ import annotations

import numpy as np

WQ_A = dict(K=4096, N=1024, M_sweep=(1, 2, 4, 7, 8, 16, 32, 64))
WQ_B = dict(K=1024, N=32768, M_sweep=(1, 8, 64, 512, 8192))
FP8_WO_A = dict(G=8, D=4096, N=1024, T_sweep=(0, 1, 7, 64, 512))
MOE = dict(T=256, H=4096, I=2048, E=256, TOPK=8, zipf=1.1)


def rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(k) for k in key])))


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """f32 values -> bf16 bit patterns (uint16), rounded by torch."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def activations(key, M, K, *, outlier_frac=0.0, outlier_mul=1.0, row_scale=None):
    """bf16 bits [M, K]: N(0,1), a Bernoulli(outlier_frac) mask scaled by outlier_mul."""
    g = rng(*key)
    x = g.standard_normal((M, K), dtype=np.float32)
    if outlier_frac > 0:
        mask = g.random((M, K)) < outlier_frac
        x = np.where(mask, x * np.float32(outlier_mul), x)
    if row_scale is not None:
        x = x * np.asarray(row_scale, np.float32)[:, None]
    return to_bf16_bits(x)


def int8_weights(key, N, K):
    """int8 [N, K] (output-channel rows, K contiguous) uniform in [-127, 127] and
    f32 per-channel scales uniform in [1e-3, 1e-2)."""
    g = rng(*key)
    w = g.integers(-127, 128, size=(N, K), dtype=np.int8)
    sw = g.uniform(1e-3, 1e-2, size=N).astype(np.float32)
    return w, sw


def tiny_linear(seed=11):
    x = activations((1, seed, 0), 4, 256, outlier_frac=0.01, outlier_mul=50.0)
    w, sw = int8_weights((1, seed, 1), 512, 256)
    return x, w, sw


def wq_a_linear(M, seed=21):
    x = activations((2, seed, M, 0), M, WQ_A["K"], outlier_frac=0.005, outlier_mul=30.0)
    w, sw = int8_weights((2, seed, 1), WQ_A["N"], WQ_A["K"])
    return x, w, sw


def wq_b_x(M, seed=31):
    return activations((3, seed, M, 0), M, WQ_B["K"])


def wq_b_w(seed=31):
    return int8_weights((3, seed, 1), WQ_B["N"], WQ_B["K"])


def fp8_group_x(T, seed=41, G=8, D=4096, layout_variant=False):
    """bf16 bits [T, G, D] = N(0,1) * u_t, u_t ~ U(0.1, 10) per token.  With
    layout_variant, hidden group h is also scaled by 2^(h mod 5) so neighbouring
    packed bytes differ."""
    g = rng(4, seed, T, G, D, 0)
    x = g.standard_normal((T, G, D), dtype=np.float32)
    u = g.uniform(0.1, 10.0, size=T).astype(np.float32)
    x = x * u[:, None, None]
    if layout_variant:
        h = np.arange(D) // 128
        x = x * np.exp2(h % 5).astype(np.float32)[None, None, :]
    return to_bf16_bits(x.reshape(T, G * D)).reshape(T, G, D)


def random_e4m3_codes(g: np.random.Generator, shape):
    """Uniform over the 254 finite E4M3FN codes (0x7F and 0xFF are NaN)."""
    c = g.integers(0, 254, size=shape, dtype=np.int64)
    c = np.where(c >= 0x7F, c + 1, c)  # skip 0x7F; 253 -> 254 = 0xFE, never 0xFF
    return c.astype(np.uint8)


def fp8_weights(seed=42, G=8, N=1024, D=4096, exp_range=4, normalish=True):
    """FP8 weights [G, N, D] and f32 power-of-two block scales [G, N/128, D/128].

    normalish=True draws codes whose magnitudes look like a quantised N(0,1)
    block (exponent field 4..9, i.e. 2^-3 .. 4, random sign and fraction);
    otherwise codes are uniform over all finite codes."""
    g = rng(4, seed, G, N, D, 1)
    if normalish:
        ef = g.integers(4, 10, size=(G, N, D), dtype=np.int64)
        fr = g.integers(0, 8, size=(G, N, D), dtype=np.int64)
        sg = g.integers(0, 2, size=(G, N, D), dtype=np.int64)
        wq = ((sg << 7) | (ef << 3) | fr).astype(np.uint8)
    else:
        wq = random_e4m3_codes(g, (G, N, D))
    j = g.integers(-exp_range, exp_range + 1, size=(G, N // 128, D // 128))
    ws = np.ldexp(np.float32(1.0), j).astype(np.float32)
    return wq, ws


def mx_weights(seed=43, G=8, N=1024, D=4096, exp_range=4):
    """FP8 weights [G, N, D] (normal-like codes, as fp8_weights) with one UE8M0 scale byte
    per (column, 32-deep block) [G, N, D/32], 127 + j with j uniform in [-exp_range, exp_range]."""
    g = rng(5, seed, G, N, D, 1)
    ef = g.integers(4, 10, size=(G, N, D), dtype=np.int64)
    fr = g.integers(0, 8, size=(G, N, D), dtype=np.int64)
    sg = g.integers(0, 2, size=(G, N, D), dtype=np.int64)
    wq = ((sg << 7) | (ef << 3) | fr).astype(np.uint8)
    wb = (127 + g.integers(-exp_range, exp_range + 1, size=(G, N, D // 32))).astype(np.uint8)
    return wq, wb


def zipf_topk_ids(key, T, E, TOPK, a=1.1):
    """[T, TOPK] distinct expert ids per token from a truncated Zipf(a) law over
    ranks 1..E (rank k -> expert k-1), drawn slot by slot without replacement."""
    g = rng(*key)
    p = np.arange(1, E + 1, dtype=np.float64) ** (-a)
    ids = np.empty((T, TOPK), np.int32)
    for t in range(T):
        w = p.copy()
        for j in range(TOPK):
            k = g.choice(E, p=w / w.sum())
            ids[t, j] = k
            w[k] = 0.0
    return ids


def moe_inputs(seed=51, T=256, H=4096, I=2048, E=256, TOPK=8, weights=True):
    """MoE block inputs: h bf16 [T, H], gamma bf16 [H] ~ U(0.5, 1.5), ids [T, TOPK],
    and (when weights) W13 int8 [E, 2I, H], sw13 [E, 2I], W2 int8 [E, H, I], sw2 [E, H]."""
    h = activations((5, seed, 0), T, H)
    gamma = to_bf16_bits(rng(5, seed, 1).uniform(0.5, 1.5, size=H).astype(np.float32))
    ids = zipf_topk_ids((5, seed, 2), T, E, TOPK)
    out = dict(h=h, gamma=gamma, ids=ids)
    if weights:
        w13 = np.empty((E, 2 * I, H), np.int8)
        sw13 = np.empty((E, 2 * I), np.float32)
        w2 = np.empty((E, H, I), np.int8)
        sw2 = np.empty((E, H), np.float32)
        for e in range(E):
            w13[e], sw13[e] = int8_weights((5, seed, 3, e), 2 * I, H)
            w2[e], sw2[e] = int8_weights((5, seed, 4, e), H, I)
        out.update(w13=w13, sw13=sw13, w2=w2, sw2=sw2)
    return out
