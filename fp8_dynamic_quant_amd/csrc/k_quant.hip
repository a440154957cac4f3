// Per-token dynamic INT8 quantisation, with an optional RMSNorm prologue and row gather.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (BF16 X -> INT8 X + per-token scale)
// and section 二 (row-parallel work limited by the row count; long rows split along K).
// RMSNorm fusion and the expert-sorted gather: "DeepSeek V4 950 低精度优化全复盘",
// sections 2.3 and 3.2.
//
// Mapping: one wave64 per (row, K-split).  A wave reads the whole source row into
// registers (16-byte loads, lane l takes chunks l, l+64, ...), reduces the absmax with
// cross-lane shuffles, and quantises only the chunks of its own K slice.  With S > 1
// splits the S waves of a row sit in different workgroups and so spread the quantise and
// store work of a short batch over more CUs; each still reads the full row for the
// absmax (served from L2 after the first), which keeps every wave independent: no
// cross-workgroup barrier, nothing to wait on.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

template <typename T>
struct In;
template <>
struct In<uint16_t> {  // bf16
  static constexpr int EPC = 8;  // elements per 16-byte chunk
  __device__ static void load(const uint16_t* p, float* v) { unpack(*reinterpret_cast<const uint4*>(p), v); }
  __device__ static void unpack(const uint4 u, float* v) {
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <>
struct In<float> {
  static constexpr int EPC = 4;
  __device__ static void load(const float* p, float* v) { unpack(*reinterpret_cast<const uint4*>(p), v); }
  __device__ static void unpack(const uint4 u, float* v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y); v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
  }
};

template <int EPC>
__device__ __forceinline__ void load_gamma(const uint16_t* g, float* v) {
  if constexpr (EPC == 8) {
    uint4 u = *reinterpret_cast<const uint4*>(g);
    uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  } else {
    uint2 u = *reinterpret_cast<const uint2*>(g);
    v[0] = __uint_as_float(u.x << 16);
    v[1] = __uint_as_float(u.x & 0xFFFF0000u);
    v[2] = __uint_as_float(u.y << 16);
    v[3] = __uint_as_float(u.y & 0xFFFF0000u);
  }
}

template <int EPC>
__device__ __forceinline__ void store_codes(int8_t* dst, const float* v, float s, float inv) {
  if constexpr (EPC == 8) {
    *reinterpret_cast<uint2*>(dst) = quant8(v, s, inv);
  } else {
    *reinterpret_cast<uint32_t*>(dst) = quant4(v, s, inv);
  }
}

// RMSNorm scale 1 / sqrt(f32(ss / K) + eps), every step correctly rounded.  sqrtf is
// the correctly rounded square root under -fhip-fp32-correctly-rounded-divide-sqrt (the
// library's build flag); __fsqrt_rn is not correctly rounded on gfx950 (measured: about
// 15% of inputs land one ulp off), so it is not used.
__device__ __forceinline__ float rms_inv(double ss, int K, float eps) {
  float ms = (float)(ss / (double)K);
  float d = __fadd_rn(ms, eps);
  return __fdiv_rn(1.0f, sqrtf(d));
}

// The row in registers (CH chunks of 16 bytes per lane, lane l taking chunks l, l + 64, ...):
// every chunk load (and, with RMSNorm, every gamma chunk) is issued before the first use,
// and none sits under a branch: lanes past the row re-read its last chunk.  (Loads under a
// per-lane branch made the compiler wait for each one before issuing the next.)
template <typename TIn, int CH>
__device__ __forceinline__ void load_row(const TIn* xr, int C, int lane, uint4 (&raw)[CH]) {
  constexpr int EPC = In<TIn>::EPC;
#pragma unroll
  for (int i = 0; i < CH; ++i)
    raw[i] = *reinterpret_cast<const uint4*>(xr + (uint32_t)(min(lane + 64 * i, C - 1) * EPC));
}

template <typename TIn, int CH>
__device__ __forceinline__ void load_gamma_chunks(const uint16_t* gamma, int C, int lane, uint4 (&graw)[CH]) {
  constexpr int EPC = In<TIn>::EPC;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = min(lane + 64 * i, C - 1);
    if constexpr (EPC == 8) {
      graw[i] = *reinterpret_cast<const uint4*>(gamma + (int64_t)c * 8);
    } else {
      const uint2 g2 = *reinterpret_cast<const uint2*>(gamma + (int64_t)c * 4);
      graw[i] = uint4{g2.x, g2.y, 0u, 0u};
    }
  }
}

// Quantise one row held in registers: chunks [c0, c1) of it are stored (a K slice), and the
// scale goes to *xs_row when xs_row is not null.
template <typename TIn, int CH, bool RMS>
__device__ __forceinline__ void quant_row(const uint4 (&raw)[CH], const uint4* graw, int C, int K, float eps,
                                          int lane, int c0, int c1, int8_t* qr, float* xs_row) {
  constexpr int EPC = In<TIn>::EPC;
  float v[CH][EPC];
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    In<TIn>::unpack(raw[i], v[i]);
    if constexpr (RMS) {
      // lanes past the row hold copies of its last chunk: no part of the sum of squares
      // (for the absmax alone they are harmless, and they are never stored)
      const bool in = lane + 64 * i < C;
#pragma unroll
      for (int e = 0; e < EPC; ++e) v[i][e] = in ? v[i][e] : 0.0f;
    }
  }
  if constexpr (RMS) {
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
      for (int e = 0; e < EPC; ++e) ss += (double)v[i][e] * (double)v[i][e];
    ss = wave_sum_f64(ss);
    const float inv = rms_inv(ss, K, eps);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const bool in = lane + 64 * i < C;
      const uint32_t gw[4] = {graw[i].x, graw[i].y, graw[i].z, graw[i].w};
#pragma unroll
      for (int e = 0; e < EPC; ++e) {
        const float g = (e & 1) ? __uint_as_float(gw[e >> 1] & 0xFFFF0000u) : __uint_as_float(gw[e >> 1] << 16);
        v[i][e] = in ? __fmul_rn(__fmul_rn(v[i][e], inv), g) : 0.0f;
      }
    }
  }
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < CH; ++i)
#pragma unroll
    for (int e = 0; e < EPC; ++e) a = fmaxf(a, fabsf(v[i][e]));
  a = wave_max_nonneg(a);
  // s = RN(a / 127): for bf16 rows without RMSNorm a is a bf16 value and the corrected
  // product gives the quotient exactly (checked for every bf16 value on the CPU); the fast
  // quant path needs 1/s only within 2^-22.4 (quant_fast), which rcp and one Newton step give
  const float s = (sizeof(TIn) == 2 && !RMS) ? div127_bf16(a) : __fdiv_rn(a, 127.0f);
  const float inv = recip_refined(s);
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int c = lane + 64 * i;
    if (c >= c0 && c < c1) store_codes<EPC>(qr + (uint32_t)(c * EPC), v[i], s, inv);
  }
  if (xs_row && lane == 0) *xs_row = s;
}

// CH > 0: the row is cached in registers (CH chunks per lane).  CH == 0: rows longer than
// the register cache are streamed in three passes (sum of squares, absmax, quantise).
template <typename TIn, int CH, bool RMS>
__global__ __launch_bounds__(256) void k_dynamic_quant(const TIn* __restrict__ x, int64_t M, int K,
                                                       int64_t ldx, const uint16_t* __restrict__ gamma,
                                                       float eps, const int32_t* __restrict__ row_index,
                                                       int8_t* __restrict__ xq, float* __restrict__ xs,
                                                       int S) {
  constexpr int EPC = In<TIn>::EPC;
  const int lane = threadIdx.x & 63;
  // the wave's row and K slice, in scalar registers (no division when S == 1)
  const int64_t gw = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int64_t row = S == 1 ? gw : gw / S;
  const int j = S == 1 ? 0 : (int)(gw - row * S);
  if (row >= M) return;
  const int64_t src = row_index ? (int64_t)row_index[row] : row;
  const TIn* xr = x + src * ldx;
  const int C = K / EPC;
  const int c0 = S == 1 ? 0 : (int)((int64_t)C * j / S), c1 = S == 1 ? C : (int)((int64_t)C * (j + 1) / S);
  int8_t* qr = xq + row * (int64_t)K;

  if constexpr (CH > 0) {
    uint4 raw[CH];
    load_row<TIn, CH>(xr, C, lane, raw);
    uint4 graw[RMS ? CH : 1];
    if constexpr (RMS) load_gamma_chunks<TIn, CH>(gamma, C, lane, graw);
    __builtin_amdgcn_sched_barrier(0);  // keep every load above the first use
    quant_row<TIn, CH, RMS>(raw, graw, C, K, eps, lane, c0, c1, qr, j == 0 ? xs + row : nullptr);
  } else {
    float inv = 1.0f;
    if constexpr (RMS) {
      double ss = 0.0;
      for (int c = lane; c < C; c += 64) {
        float v[EPC];
        In<TIn>::load(xr + (int64_t)c * EPC, v);
#pragma unroll
        for (int e = 0; e < EPC; ++e) ss += (double)v[e] * (double)v[e];
      }
      ss = wave_sum_f64(ss);
      inv = rms_inv(ss, K, eps);
    }
    float a = 0.0f;
    for (int c = lane; c < C; c += 64) {
      float v[EPC];
      In<TIn>::load(xr + (int64_t)c * EPC, v);
      if constexpr (RMS) {
        float g[EPC];
        load_gamma<EPC>(gamma + (int64_t)c * EPC, g);
#pragma unroll
        for (int e = 0; e < EPC; ++e) v[e] = __fmul_rn(__fmul_rn(v[e], inv), g[e]);
      }
#pragma unroll
      for (int e = 0; e < EPC; ++e) a = fmaxf(a, fabsf(v[e]));
    }
    a = wave_max(a);
    const float s = __fdiv_rn(a, 127.0f);
    const float qinv = __fdiv_rn(1.0f, s);
    for (int c = c0 + lane; c < c1; c += 64) {
      float v[EPC];
      In<TIn>::load(xr + (int64_t)c * EPC, v);
      if constexpr (RMS) {
        float g[EPC];
        load_gamma<EPC>(gamma + (int64_t)c * EPC, g);
#pragma unroll
        for (int e = 0; e < EPC; ++e) v[e] = __fmul_rn(__fmul_rn(v[e], inv), g[e]);
      }
      store_codes<EPC>(qr + (int64_t)c * EPC, v, s, qinv);
    }
    if (j == 0 && lane == 0) xs[row] = s;
  }
}

template <typename TIn, bool RMS>
static hipError_t launch_t(const TIn* x, int64_t M, int K, int64_t ldx, const uint16_t* gamma, float eps,
                           const int32_t* row_index, int8_t* xq, float* xs, int S, hipStream_t st,
                           int* ch_used) {
  constexpr int EPC = In<TIn>::EPC;
  const int C = K / EPC;
  const int need = (C + 63) / 64;
  const int64_t waves = M * S;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
#define WQ_QL(CHV)                                                                                     \
  do {                                                                                                 \
    *ch_used = CHV;                                                                                    \
    hipLaunchKernelGGL((k_dynamic_quant<TIn, CHV, RMS>), grid, block, 0, st, x, M, K, ldx, gamma, eps, \
                       row_index, xq, xs, S);                                                          \
    return hipGetLastError();                                                                          \
  } while (0)
  if (need <= 1) WQ_QL(1);
  if (need <= 2) WQ_QL(2);
  if (need <= 4) WQ_QL(4);
  if (need <= 8) WQ_QL(8);
  if (need <= 16) WQ_QL(16);
  WQ_QL(0);
#undef WQ_QL
}

hipError_t launch_dynamic_quant(const void* x, bool x_f32, int64_t M, int K, int64_t ldx,
                                const uint16_t* gamma, float eps, const int32_t* row_index, int8_t* xq,
                                float* xs, int S, hipStream_t st, int* ch_used) {
  if (x_f32) {
    return gamma ? launch_t<float, true>((const float*)x, M, K, ldx, gamma, eps, row_index, xq, xs, S, st, ch_used)
                 : launch_t<float, false>((const float*)x, M, K, ldx, gamma, eps, row_index, xq, xs, S, st, ch_used);
  }
  return gamma ? launch_t<uint16_t, true>((const uint16_t*)x, M, K, ldx, gamma, eps, row_index, xq, xs, S, st, ch_used)
               : launch_t<uint16_t, false>((const uint16_t*)x, M, K, ldx, gamma, eps, row_index, xq, xs, S, st, ch_used);
}

}  // namespace wq
