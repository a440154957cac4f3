// INT8 x INT8 -> INT32 GEMMs with the per-token x per-channel scale epilogue.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (npu_quant_matmul: INT8 X and
// per-token scale times pre-quantised weights, BF16 Y) and section 三 (the tiling is
// derived from the real M, N, K).
//
// k_gemm_i8_tile - the fallback for K not a multiple of 128 above the decode sizes: 128x128
// workgroup tiles, LDS double buffering, v_mfma_i32_16x16x64_i8.  Decode-sized M runs in
// k_decode.hip / k_fused.hip, K % 128 == 0 in k_gemm_tile.hip / k_gemm_big.hip.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

// ------------------------------------------------------------------------------------
// epilogues
// ------------------------------------------------------------------------------------
__device__ __forceinline__ uint16_t epi_bf16(int acc, float s, float sw) {
  return (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)acc, s), sw));
}

// ------------------------------------------------------------------------------------
// tiled kernel for large M (optionally over expert segments)
// ------------------------------------------------------------------------------------
constexpr int kTM = 128, kTN = 128, kTK = 64;
constexpr int kTLDS = kTK + 16;  // padded LDS row (bytes)

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_i8_tile(TileArgs p, int tiles_n) {
  __shared__ __attribute__((aligned(16))) int8_t sa[2][kTM * kTLDS];
  __shared__ __attribute__((aligned(16))) int8_t sb[2][kTN * kTLDS];

  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;  // 2x2 waves, 64x64 each
  // tile indices; for segments blockIdx.y is the expert
  int row_lo = 0, row_hi = p.M;
  const int8_t* w = p.w;
  const float* wsc = p.w_scale;
  if (p.seg_offsets) {
    const int e = blockIdx.y;
    row_lo = (int)p.seg_offsets[e];
    row_hi = (int)p.seg_offsets[e + 1];
    w += (int64_t)e * p.w_batch_stride;
    wsc += (int64_t)e * p.N;
  }
  const int rows = row_hi - row_lo;
  const int tm = blockIdx.x / tiles_n, tn = blockIdx.x % tiles_n;
  if (tm * kTM >= rows) return;
  const int m0 = row_lo + tm * kTM, n0 = tn * kTN;
  const int K = p.K, N = p.N;

  // global -> register staging: each thread moves 2 chunks of A and 2 of B per K step
  v4i ra[2], rb[2];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + 256 * i;             // 0..511
      const int r = c >> 2, kc = (c & 3) * 16;  // 128 rows x 4 chunks
      const int kk = kt * kTK + kc;
      const int m = m0 + r, n = n0 + r;
      ra[i] = (m < row_hi && kk < K) ? *reinterpret_cast<const v4i*>(p.a + (int64_t)m * p.lda + kk) : v4i{0, 0, 0, 0};
      rb[i] = (n < N && kk < K) ? *reinterpret_cast<const v4i*>(w + (int64_t)n * K + kk) : v4i{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int c = t + 256 * i;
      const int r = c >> 2, kc = (c & 3) * 16;
      *reinterpret_cast<v4i*>(&sa[buf][r * kTLDS + kc]) = ra[i];
      *reinterpret_cast<v4i*>(&sb[buf][r * kTLDS + kc]) = rb[i];
    }
  };

  v4i acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int KT = (K + kTK - 1) / kTK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
    v4i af[4], bf[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      af[i] = *reinterpret_cast<const v4i*>(&sa[buf][(wm * 64 + i * 16 + (lane & 15)) * kTLDS + 16 * (lane >> 4)]);
      bf[i] = *reinterpret_cast<const v4i*>(&sb[buf][(wn * 64 + i * 16 + (lane & 15)) * kTLDS + 16 * (lane >> 4)]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[i], bf[j], acc[i][j], 0, 0, 0);
    if (kt + 1 < KT) {
      sstore(buf ^ 1);
    }
    __syncthreads();
  }

  // epilogue: acc[i][j] lane holds column n0 + wn*64 + j*16 + (lane&15), rows +4*(lane>>4)+r
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int m = m0 + wm * 64 + i * 16 + 4 * (lane >> 4) + r;
      if (m >= row_hi) continue;
      const float s = p.a_scale[m];
      if constexpr (EPI == 1) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int n = n0 + wn * 64 + j * 16 + (lane & 15);
          if (n < N) {
            reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * p.ldy + n] = epi_bf16(acc[i][j][r], s, wsc[n]);
            if (p.acc_out) p.acc_out[(int64_t)m * N + n] = acc[i][j][r];
          }
        }
      }
    }
  }
  if constexpr (EPI == 2) {
    // SwiGLU needs column n and n + N/2 together: go through LDS (the A/B buffers are free)
    // Each workgroup writes its raw accumulators; pairing happens in k_swiglu below.
  }
}

// SwiGLU epilogue over int32 accumulators [rows, 2I] of one expert segment set.
__global__ __launch_bounds__(256) void k_swiglu_from_acc(const int32_t* __restrict__ acc, int64_t rows, int I,
                                                          const float* __restrict__ a_scale,
                                                          const float* __restrict__ w_scale, int64_t w_scale_stride,
                                                          const int64_t* __restrict__ seg_offsets, int E,
                                                          float* __restrict__ h) {
  const int64_t r = blockIdx.y;
  if (r >= rows) return;
  // expert of row r: binary search in the offsets
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (seg_offsets[mid] <= r) lo = mid; else hi = mid;
  }
  const float* sw = w_scale + (int64_t)lo * w_scale_stride;
  const float s = a_scale[r];
  for (int n = blockIdx.x * 256 + threadIdx.x; n < I; n += gridDim.x * 256) {
    const float g = __fmul_rn(__fmul_rn((float)acc[r * 2 * I + n], s), sw[n]);
    const float u = __fmul_rn(__fmul_rn((float)acc[r * 2 * I + I + n], s), sw[I + n]);
    const float e = exp_fixed(-g);
    const float sg = __fdiv_rn(g, __fadd_rn(1.0f, e));
    h[r * I + n] = __fmul_rn(sg, u);
  }
}

hipError_t launch_gemm_i8_tile(const TileArgs& a, hipStream_t st) {
  const int tiles_n = (a.N + kTN - 1) / kTN;
  int max_rows = a.M;
  unsigned gy = 1;
  if (a.seg_offsets) gy = (unsigned)a.batch;  // rows per segment unknown on host: cover M
  const int tiles_m = (max_rows + kTM - 1) / kTM;
  dim3 grid((unsigned)(tiles_m * tiles_n), gy), block(256);
  if (a.epilogue == 1)
    hipLaunchKernelGGL((k_gemm_i8_tile<1>), grid, block, 0, st, a, tiles_n);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace wq
