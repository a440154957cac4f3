// Grouped FP8 contraction for decode-sized token counts (T <= 64): weight streaming.
//
// Operation: the SGLang PR #34277 summary (功能与动机, 实现拆解): the grouped FP8 einsum
// that consumes the activation scales exactly as the group quant writes them, packed 4
// UE8M0 bytes per int32 in [G, ceil(HG/4), align4(T)]:
//   out[t, g, n] = bf16( sum_kb 2^(ea(t,g,kb)) * ws[g, n/128, kb] * sum_{k in kb} q[t,g,k] w[g,n,k] )
// with 128-wide K blocks, E4M3 payloads and f32 accumulation.
//
// At T <= 64 the 32 MiB of FP8 weights bound the run (a 128 x 128 output tile would put
// only G * N / 128 = 64 workgroups on the chip).  So each workgroup owns 16 output columns
// of one group and the whole K range, G * N / 16 = 512 workgroups for the DeepSeek shape:
//  * four waves split K; each wave loads its weights (32 bytes per lane per 128-deep step)
//    straight into registers in the v_mfma_scale_f32_16x16x128_f8f6f4 B layout, after the
//    scale words and before the first wait; the token tiles follow, each loading while the
//    previous one multiplies;
//  * a 128-deep step is exactly one scale block, so the block scales ride in the MFMA's
//    E8M0 scale operands: the activation byte is read from the packed storage as written,
//    the weight byte is the exponent field of the f32 power-of-two block scale;
//  * tokens go in tiles of 16 rows; the four waves' f32 16 x 16 tiles are summed in LDS in
//    a fixed order and written as bf16.
// Above 16 tokens every workgroup re-reads each token tile from L2, 64 times per group at
// N = 1024; k_fp8_decode32 below halves that with 32 columns per workgroup.
// Both kernels also take the MX-like 32-element blocks of "重塑大模型推理数据流：DeepSeek
// V4 950 低精度优化全复盘", section 2.1 (template flag MX): then every lane group passes
// the scale bytes of its own 32-element block of activations and weights.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

namespace {
constexpr int kF8NT = 16;       // output columns per workgroup
constexpr int kF8Waves = 4;
constexpr int kF8MaxSteps = 8;  // 128-deep K steps per wave: K <= 4096
constexpr int kF8MaxRT = 4;     // 16-token row tiles: T <= 64
}  // namespace

// MX: the MX-like 32-element blocks ("DeepSeek V4 950 低精度优化全复盘", section 2.1) on
// both operands: the activation words hold the four 32-element scales of one 128-deep
// block (storage [G, K/128, TA] from wq_group_quant_mxfp8) and p.w_scale holds UE8M0
// bytes [G][N][K/32].  The MFMA applies the scale operand of lane group kq to K bytes
// 32 kq .. 32 kq + 31 of the block (its operand layout is stated at the loads below), so
// lane group kq passes byte kq of the activation word and of the column's scale word.
// Workgroup -> (column slice, group, token-tile block).  Workgroups go to the 8 XCDs round
// robin by linear id; each XCD gets a contiguous run of items ordered group-major, so with G
// a multiple of 8 an XCD serves whole groups and its L2 fetches each group's activation
// codes once (with the plain order every XCD read every group's: 1.41x the algorithmic
// bytes at T = 64).
struct Fp8Item {
  int x, g, z;
};
__device__ __forceinline__ Fp8Item fp8_item() {
  const int S = gridDim.x, G = gridDim.y, Z = gridDim.z;
  const int L = blockIdx.x + S * (blockIdx.y + G * blockIdx.z);
  const int total = S * G * Z;
  const int w = (total & 7) == 0 ? (L & 7) * (total >> 3) + (L >> 3) : L;
  return Fp8Item{w % S, w / (S * Z), (w / S) % Z};
}

template <int TPW, bool MX>
__global__ __launch_bounds__(256) void k_fp8_decode(TileArgs p) {
  constexpr int NW = MX ? kF8MaxSteps : 3;  // packed activation words per token tile
  __shared__ float red[4][TPW][4][64];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: the weight-scale loads go scalar
  const Fp8Item item = fp8_item();
  const int T = p.M, N = p.N, K = p.K, g = item.g;
  const int n0 = item.x * kF8NT;
  const int KT = K >> 7;                 // 128-deep blocks
  const int steps = KT / 4;              // per wave
  const int kb0 = wv * steps;
  const int cl = lane & 15, kq = lane >> 4;  // column (B) / row (A) in the tile; 32-byte quarter of the step
  const int n = n0 + cl;
  const int PH = MX ? KT : (KT + 3) >> 2;
  const int32_t* xs_g = p.a_scale_packed + (int64_t)g * PH * p.a_scale_tokens;
  // operand layout of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on gfx950 with one-hot
  // inputs and distinct 32-element block scales): lane group q (lanes 16q .. 16q+15) holds
  // K bytes 16q .. 16q+15 in its first four registers and 64+16q .. 64+16q+15 in the last
  // four, and the scale operand of lane group s applies to K bytes 32s .. 32s+31
  const int8_t* A = p.a + (int64_t)g * p.a_batch_stride + kq * 16;
  const int rt_lo = item.z * TPW;    // this workgroup's 16-token tiles [rt_lo, rt_lo + TPW)

  // Every load is issued before the first wait and none sits under a branch (K steps and
  // rows out of range read clamped in-range addresses; their values go unused), so the
  // compiler keeps them in flight together: a scale load waited for next to each MFMA
  // had cost a memory round trip per MFMA.  (At most 63 vector loads can be counted in
  // flight; the weight block scales are wave-uniform scalar loads outside that count.)
  // this wave's K blocks [kb0, kb0 + steps) touch at most 3 packed activation-scale words
  // (with MX, one word per block: up to 8)
  const int w0 = kb0 >> 2;
  // ---- weights, 32 bytes per lane per 128-deep step, straight into the B layout ----------
  const int8_t* W = p.w + (int64_t)g * p.w_batch_stride + (int64_t)n * K + kq * 16;
  v8i b[kF8MaxSteps];
#pragma unroll
  for (int j = 0; j < kF8MaxSteps; ++j) {
    const int8_t* src = W + (int64_t)(kb0 + min(j, steps - 1)) * 128;
    const v4i lo = *reinterpret_cast<const v4i*>(src);
    const v4i hi = *reinterpret_cast<const v4i*>(src + 64);
    b[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  }
  // ---- token tiles (fragments and packed scale words): the next tile loads while the
  // current one multiplies -------------------------------------------------------------------
  auto load_tile = [&](int rt, v8i (&a)[kF8MaxSteps], int32_t (&wd)[NW]) {
    // rows past T read row T-1: they only feed output rows that are not stored
    const int row = min((rt_lo + rt) * 16 + cl, T - 1);
#pragma unroll
    for (int q = 0; q < NW; ++q)
      wd[q] = MX ? xs_g[(int64_t)(kb0 + min(q, steps - 1)) * p.a_scale_tokens + row]
                 : xs_g[(int64_t)min(w0 + q, PH - 1) * p.a_scale_tokens + row];
    const int8_t* arow = A + (int64_t)row * p.lda;
#pragma unroll
    for (int j = 0; j < kF8MaxSteps; ++j) {
      const int8_t* src = arow + (int64_t)(kb0 + min(j, steps - 1)) * 128;
      const v4i lo = *reinterpret_cast<const v4i*>(src);
      const v4i hi = *reinterpret_cast<const v4i*>(src + 64);
      a[j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  };
  v8i abuf[2][kF8MaxSteps];
  int32_t words[2][NW];
  load_tile(0, abuf[0], words[0]);
  if (TPW > 1) load_tile(1, abuf[1], words[1]);
  // keep the issue order: a load the scheduler sinks next to its use is waited for at once
  __builtin_amdgcn_sched_barrier(0);
  // ---- the weight block-scale exponents (wave-uniform scalar loads, while the vector loads
  // are in flight; the empty asm pins each value here, so no load is sunk next to its MFMA)
  int sbx[kF8MaxSteps];
  if constexpr (MX) {
    // per lane: the column's word of four 32-element scales for block kb0 + j, byte kq
    const uint32_t* wsw = reinterpret_cast<const uint32_t*>(p.w_scale) + ((int64_t)g * N + n) * KT + kb0;
#pragma unroll
    for (int j = 0; j < kF8MaxSteps; ++j) sbx[j] = (int)((wsw[min(j, steps - 1)] >> (8 * kq)) & 0xFF);
  } else {
    const float* wsc = p.w_scale + ((int64_t)g * (N >> 7) + (n0 >> 7)) * KT + kb0;
    uint32_t wsb[kF8MaxSteps];
#pragma unroll
    for (int j = 0; j < kF8MaxSteps; ++j) wsb[j] = __float_as_uint(wsc[min(j, steps - 1)]);
    static_assert(kF8MaxSteps == 8, "one pin for the eight scales");
    asm volatile("" : "+s"(wsb[0]), "+s"(wsb[1]), "+s"(wsb[2]), "+s"(wsb[3]), "+s"(wsb[4]), "+s"(wsb[5]),
                 "+s"(wsb[6]), "+s"(wsb[7]));
#pragma unroll
    for (int j = 0; j < kF8MaxSteps; ++j) sbx[j] = (int)((wsb[j] >> 23) & 0xFF);
  }
  v4f acc[TPW];
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt) {
    if (rt >= 1 && rt + 1 < TPW) {
      load_tile(rt + 1, abuf[(rt + 1) & 1], words[(rt + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
    }
    acc[rt] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < kF8MaxSteps; ++j) {
      if (j < steps) {  // uniform
        const int kb = kb0 + j;
        int sa;
        if constexpr (MX) {
          sa = (words[rt & 1][j] >> (8 * kq)) & 0xFF;  // this lane's 32-element block of block kb
        } else {
          const int q = (kb >> 2) - w0;  // 0, 1 or 2
          const int32_t w = q == 0 ? words[rt & 1][0] : (q == 1 ? words[rt & 1][1] : words[rt & 1][2]);
          sa = (w >> (8 * (kb & 3))) & 0xFF;
        }
        // sbx[j]: the exponent field of the power-of-two weight block scale
        acc[rt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(abuf[rt & 1][j], b[j], acc[rt], 0, 0, 0, sa, 0, sbx[j]);
      }
    }
  }

  // ---- the four waves' partial sums, in a fixed order, then bf16 ----------------------------
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wv][rt][i][lane] = acc[rt][i];
  __syncthreads();
  uint16_t* Y = reinterpret_cast<uint16_t*>(p.y) + (int64_t)g * p.y_batch_stride;
  for (int e = t; e < TPW * 4 * 64; e += 256) {
    const int ln = e & 63, ri = e >> 6, rt = ri >> 2, i = ri & 3;
    const int row = (rt_lo + rt) * 16 + 4 * (ln >> 4) + i;  // MFMA 16x16 output: col = lane % 16, row = 4 (lane / 16) + i
    if (row < T) {
      const float v = __fadd_rn(__fadd_rn(__fadd_rn(red[0][rt][i][ln], red[1][rt][i][ln]), red[2][rt][i][ln]),
                                red[3][rt][i][ln]);
      Y[(int64_t)row * p.ldy + n0 + (ln & 15)] = (uint16_t)f32_to_bf16_rn(v);
    }
  }
}

// Wider variant: 32 output columns (two 16-column MFMA tiles) per workgroup of 8 waves,
// each wave owning K/8 and multiplying every activation fragment it loads into both column
// tiles.  Half as many workgroups read each token tile from L2 as with 16 columns, and all
// token tiles are in flight at once (at most 56 vector loads per wave: 16 for the weights,
// 8 per token tile for the fragments and 2 for its packed scale words).
// MX: the MX-like 32-element blocks, as in k_fp8_decode<TPW, true> (operands in the MFMA's
// own K layout, per-lane scale bytes of the activation and column words)
template <int TPW, bool MX>
__global__ __launch_bounds__(512) void k_fp8_decode32(TileArgs p) {
  constexpr int NWD = MX ? 4 : 2;  // packed activation words per token tile
  __shared__ float red[8][TPW][2][4][64];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const Fp8Item item = fp8_item();
  const int T = p.M, N = p.N, K = p.K, g = item.g;
  const int n0 = item.x * 32;
  const int KT = K >> 7;
  const int steps = KT >> 3;             // 128-deep blocks per wave (1..4)
  const int kb0 = wv * steps;
  const int cl = lane & 15, kq = lane >> 4;
  const int PH = MX ? KT : (KT + 3) >> 2;
  const int32_t* xs_g = p.a_scale_packed + (int64_t)g * PH * p.a_scale_tokens;
  // plain: a lane's 32 bytes of a block at 32 kq (halves 16 apart); MX: at 16 kq and 64 + 16 kq
  const int koff = MX ? kq * 16 : kq * 32, khalf = MX ? 64 : 16;
  const int8_t* A = p.a + (int64_t)g * p.a_batch_stride + koff;
  const int rt_lo = item.z * TPW;
  const int w0 = kb0 >> 2;               // the wave's blocks touch packed words w0 and w0 + 1 at most

  // ---- weights of both column tiles, 32 bytes per lane per block ----------------------------
  v8i b[2][4];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int8_t* W = p.w + (int64_t)g * p.w_batch_stride + (int64_t)(n0 + ct * 16 + cl) * K + koff;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // streaming loads (both halves of each 128-byte line by the same lanes, back to back):
      // measured 13.4 -> 13.05 us at T = 32 and 17.3 -> 17.0 us at T = 64; the 16-column
      // kernel above measured slower with them at T = 7 and 16 and keeps ordinary loads
      const int8_t* src = W + (int64_t)(kb0 + min(j, steps - 1)) * 128;
      const v4i lo = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src));
      const v4i hi = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src + khalf));
      b[ct][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  // ---- every token tile's fragments and packed scale words --------------------------------
  v8i a[TPW][4];
  int32_t wd[TPW][NWD];
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt) {
    // rows past T read row T-1: they only feed output rows that are not stored
    const int row = min((rt_lo + rt) * 16 + cl, T - 1);
#pragma unroll
    for (int q = 0; q < NWD; ++q)
      wd[rt][q] = MX ? xs_g[(int64_t)(kb0 + min(q, steps - 1)) * p.a_scale_tokens + row]
                     : xs_g[(int64_t)min(w0 + q, PH - 1) * p.a_scale_tokens + row];
    const int8_t* arow = A + (int64_t)row * p.lda;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int8_t* src = arow + (int64_t)(kb0 + min(j, steps - 1)) * 128;
      const v4i lo = *reinterpret_cast<const v4i*>(src);
      const v4i hi = *reinterpret_cast<const v4i*>(src + khalf);
      a[rt][j] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
  }
  __builtin_amdgcn_sched_barrier(0);
  // ---- weight block-scale exponents: both column tiles lie in one 128-column block --------
  int sbx[2][4];  // [column tile][step]
  if constexpr (MX) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t* wsw =
          reinterpret_cast<const uint32_t*>(p.w_scale) + ((int64_t)g * N + n0 + ct * 16 + cl) * KT + kb0;
#pragma unroll
      for (int j = 0; j < 4; ++j) sbx[ct][j] = (int)((wsw[min(j, steps - 1)] >> (8 * kq)) & 0xFF);
    }
  } else {
    const float* wsc = p.w_scale + ((int64_t)g * (N >> 7) + (n0 >> 7)) * KT + kb0;
    uint32_t wsb[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) wsb[j] = __float_as_uint(wsc[min(j, steps - 1)]);
    asm volatile("" : "+s"(wsb[0]), "+s"(wsb[1]), "+s"(wsb[2]), "+s"(wsb[3]));
#pragma unroll
    for (int j = 0; j < 4; ++j) sbx[0][j] = sbx[1][j] = (int)((wsb[j] >> 23) & 0xFF);
  }

  v4f acc[TPW][2];
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < steps) {  // uniform
        const int kb = kb0 + j;
        int sa;
        if constexpr (MX) {
          sa = (wd[rt][j] >> (8 * kq)) & 0xFF;
        } else {
          const int32_t w = (kb >> 2) == w0 ? wd[rt][0] : wd[rt][1];
          sa = (w >> (8 * (kb & 3))) & 0xFF;
        }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
          acc[rt][ct] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a[rt][j], b[ct][j], acc[rt][ct], 0, 0, 0, sa,
                                                                         0, sbx[ct][j]);
      }
    }
  }

  // ---- the eight waves' partial sums, in a fixed order, then bf16 ---------------------------
#pragma unroll
  for (int rt = 0; rt < TPW; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wv][rt][ct][i][lane] = acc[rt][ct][i];
  __syncthreads();
  uint16_t* Y = reinterpret_cast<uint16_t*>(p.y) + (int64_t)g * p.y_batch_stride;
  for (int e = t; e < TPW * 2 * 4 * 64; e += 512) {
    const int ln = e & 63, ri = e >> 6, i = ri & 3, ct = (ri >> 2) & 1, rt = ri >> 3;
    const int row = (rt_lo + rt) * 16 + 4 * (ln >> 4) + i;  // MFMA 16x16 output: col = lane % 16, row = 4 (lane / 16) + i
    if (row < T) {
      float v = red[0][rt][ct][i][ln];
#pragma unroll
      for (int w = 1; w < 8; ++w) v = __fadd_rn(v, red[w][rt][ct][i][ln]);
      Y[(int64_t)row * p.ldy + n0 + ct * 16 + (ln & 15)] = (uint16_t)f32_to_bf16_rn(v);
    }
  }
}

bool fp8_decode32_fits(int T, int N, int K) {
  return T > 16 && T <= 16 * kF8MaxRT && N % 32 == 0 && K % 1024 == 0 && K <= 4096;
}

hipError_t launch_fp8_decode32(const TileArgs& a, hipStream_t st, bool mx) {
  if (!fp8_decode32_fits(a.M, a.N, a.K)) return hipErrorInvalidValue;
  const int rt = (a.M + 15) / 16;
  const dim3 grid((unsigned)(a.N / 32), (unsigned)a.batch, 1);
#define WQ_F8D32(TP)                                                             \
  if (mx)                                                                        \
    hipLaunchKernelGGL((k_fp8_decode32<TP, true>), grid, dim3(512), 0, st, a);   \
  else                                                                           \
    hipLaunchKernelGGL((k_fp8_decode32<TP, false>), grid, dim3(512), 0, st, a);
  switch (rt) {
    case 2: WQ_F8D32(2) break;
    case 3: WQ_F8D32(3) break;
    default: WQ_F8D32(4) break;
  }
#undef WQ_F8D32
  return hipGetLastError();
}

bool fp8_decode_fits(int T, int N, int K) {
  return T >= 1 && T <= 16 * kF8MaxRT && N % kF8NT == 0 && K % (128 * kF8Waves) == 0 &&
         K / (128 * kF8Waves) <= kF8MaxSteps;
}

hipError_t launch_fp8_decode(const TileArgs& a, int rt_per_wg, hipStream_t st, bool mx) {
  if (!fp8_decode_fits(a.M, a.N, a.K) || rt_per_wg < 1 || rt_per_wg > kF8MaxRT) return hipErrorInvalidValue;
  const int rt = (a.M + 15) / 16;
  const int tpw = min(rt_per_wg, rt);  // token tiles per workgroup
  const dim3 grid((unsigned)(a.N / kF8NT), (unsigned)a.batch, (unsigned)((rt + tpw - 1) / tpw));
#define WQ_F8D(TP)                                                            \
  if (mx)                                                                     \
    hipLaunchKernelGGL((k_fp8_decode<TP, true>), grid, dim3(256), 0, st, a);  \
  else                                                                        \
    hipLaunchKernelGGL((k_fp8_decode<TP, false>), grid, dim3(256), 0, st, a);
  switch (tpw) {
    case 1: WQ_F8D(1) break;
    case 2: WQ_F8D(2) break;
    case 3: WQ_F8D(3) break;
    default: WQ_F8D(4) break;
  }
#undef WQ_F8D
  return hipGetLastError();
}

}  // namespace wq
