// Per-token-group FP8 quantisation with packed UE8M0 scales.
//
// Operation: SGLang PR #34277 summary, 实现拆解 items 1-2 and the kernel write-logic
// snippet: each 128-wide hidden group of each (token, outer group) gets a power-of-two
// scale whose UE8M0 exponent byte is written straight into the int32-packed
// [G, ceil(HG/4), align4(T)] layout the FP8 contraction reads; the rest of the last pack
// is zeroed.  Here the token-padding words are zeroed too, so the whole storage is
// defined.
//
// Mapping: one wave64 per (token t, outer group g, pack p).  Its four 16-lane quarters
// take hidden groups 4p .. 4p+3 (128 bf16 = 256 bytes each, 16 bytes per lane), so a
// wave reads 1 KiB contiguous and writes 512 bytes of E4M3 codes contiguous.  Quarter
// absmax by shuffles; e = ceil(log2(RN(a / 448))) read off the f32 bits (for bf16
// absmax values this equals the exact smallest power of two >= a / 448); the codes come
// from v_cvt_pk_fp8_f32 (OCP E4M3FN, round to nearest even) applied to x * 2^-e, an exact
// power-of-two scaling.  The four exponent bytes meet in lane 0, which writes the whole
// packed word - no byte-granular read-modify-write and no dependence on prior contents.
// Waves with t in [T, TA) write the zero padding words.  On large grids (16384 waves or
// more at one pack per wave) a wave takes two, from 32768 four, consecutive packs of its
// (t, g), with every pack's loads issued before the first is quantised.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

// e = ceil(log2(r)) for r = RN_f32(a / 448) >= 0, clamped to >= -127, for a bf16 value a
// (an absmax of bf16 elements).  r comes without a division: m = RN(a c) with c = RN(1/448),
// then r = fma(fma(-448, m, a), c, m), which equals the correctly rounded quotient for every
// non-negative finite bf16 a (checked exhaustively with exact rationals on the CPU).
__device__ __forceinline__ int ue8m0_exp(float a) {
  const float c = 2.23214295692741870880126953125e-3f;  // RN_f32(1/448) = 0x3B124925
  const float m = __fmul_rn(a, c);
  const float r = __fmaf_rn(__fmaf_rn(-448.0f, m, a), c, m);
  const uint32_t b = __float_as_uint(r);
  const int ef = (int)(b >> 23) & 0xFF;
  const uint32_t fr = b & 0x7FFFFFu;
  int e;
  if (ef != 0) {
    e = ef - 127 + (fr != 0 ? 1 : 0);
  } else if (fr == 0) {
    e = -127;  // a == 0
  } else {
    // subnormal r = fr * 2^-149: ceil(log2 r) = bit_length(fr - 1) - 149
    e = (32 - __clz((int)(fr - 1))) - 149;
  }
  return e < -127 ? -127 : e;
}

// max over the 16 lanes of each DPP row (non-negative f32): quad swaps, then the half-row
// and row mirrors; every lane of the row ends with the row's max
__device__ __forceinline__ float row16_max(float a) {
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, false)));   // [1,0,3,2]
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, false)));   // [2,3,0,1]
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x141, 0xF, 0xF, false)));  // half mirror
  a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x140, 0xF, 0xF, false)));  // row mirror
  return a;
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// PPW packs per wave (consecutive packs of one (t, g)); their loads are issued first.  The
// wave's indices are scalar (TA * G * PH < 2^31, checked by the host) and every access is a
// scalar row base plus a 32-bit lane offset, so the address arithmetic stays off the vector
// ALU, which bounds this kernel once the loads are in flight.
template <int PPW>
__global__ __launch_bounds__(256) void k_group_quant_fp8(const uint16_t* __restrict__ x, int T, int G, int D,
                                                         uint8_t* __restrict__ xq, int32_t* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int HG = D / 128, PH = (HG + 3) / 4, PW = (PH + PPW - 1) / PPW;
  const int TA = (T + 3) / 4 * 4;
  const int wid = (int)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  if (wid >= TA * G * PW) return;
  const int pw = wid % PW, tg = wid / PW;
  const int g = tg % G, t = tg / G;
  const int q = lane >> 4;  // quarter: hidden group 4p + q
  const int64_t row = (int64_t)(min(t, T - 1) * G + g) * D;
  const uint16_t* xr = x + row;
  uint4 u[PPW];
#pragma unroll
  for (int i = 0; i < PPW; ++i) {  // clamped in-range loads, all before the first use
    const int h = min(4 * (pw * PPW + i) + q, HG - 1);
    const uint16_t* src = xr + (uint32_t)(h * 128 + (lane & 15) * 8);
    if constexpr (PPW >= 2) {
      // large grids: streaming loads (the rows are read once; measured 14.7 -> 13.7 us at
      // T = 512, while the small grids measured slower with them)
      const v4i v = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(src));
      u[i] = uint4{(uint32_t)v[0], (uint32_t)v[1], (uint32_t)v[2], (uint32_t)v[3]};
    } else {
      u[i] = *reinterpret_cast<const uint4*>(src);
    }
  }
  uint8_t* qr = xq + row;
#pragma unroll
  for (int i = 0; i < PPW; ++i) {
    const int p = pw * PPW + i;
    if (p >= PH) break;  // uniform
    const int h = 4 * p + q;
    int byte = 0;
    if (t < T && h < HG) {  // whole quarters (DPP rows) take part or not
      float v[8];
      const uint32_t w4[4] = {u[i].x, u[i].y, u[i].z, u[i].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[2 * j] = __uint_as_float(w4[j] << 16);
        v[2 * j + 1] = __uint_as_float(w4[j] & 0xFFFF0000u);
      }
      float a = 0.0f;
#pragma unroll
      for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(v[j]));
      a = row16_max(a);
      const int e = ue8m0_exp(a);
      const float sc = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 126]
      uint32_t lo = 0, hi = 0;
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[0], sc), __fmul_rn(v[1], sc), lo, false);
      lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[2], sc), __fmul_rn(v[3], sc), lo, true);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[4], sc), __fmul_rn(v[5], sc), hi, false);
      hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[6], sc), __fmul_rn(v[7], sc), hi, true);
      v2u* dst = reinterpret_cast<v2u*>(qr + (uint32_t)(h * 128 + (lane & 15) * 8));
      if constexpr (PPW >= 2) {
        // the codes are written once and read by another kernel: streaming stores
        __builtin_nontemporal_store(v2u{lo, hi}, dst);
      } else {
        *dst = v2u{lo, hi};
      }
      byte = e + 127;
    }
    // the four quarter bytes (0 for hidden groups past HG) form the pack word, read out of
    // lanes 0, 16, 32, 48 into scalar registers; lane 0 stores it
    const uint32_t word = (uint32_t)__builtin_amdgcn_readlane(byte, 0) |
                          ((uint32_t)__builtin_amdgcn_readlane(byte, 16) << 8) |
                          ((uint32_t)__builtin_amdgcn_readlane(byte, 32) << 16) |
                          ((uint32_t)__builtin_amdgcn_readlane(byte, 48) << 24);
    if (lane == 0) xs[(g * PH + p) * TA + t] = (int32_t)word;
  }
}

// MX-like 32-element blocks ("DeepSeek V4 950 低精度优化全复盘", section 2.1: every 32
// elements share one 8-bit scale), same exponent rule and packed layout with HG = D / 32.
// One wave64 per (token t, outer group g, 4 consecutive packs): its 16-lane row r takes
// pack p = 4 * pw + r, i.e. blocks 4p .. 4p+3 (128 bf16 contiguous, 16 bytes per lane),
// and each 4-lane quad of the row one block; the quad's absmax comes from two quad
// permutes, and lane 0 of the row writes the pack's word.
// NT: streaming loads of the rows, chosen on large grids (T = 512 measured 13.6 -> 12.9 us,
// T = 256 8.0 -> 7.6 us)
template <bool NT>
__global__ __launch_bounds__(256) void k_group_quant_mx(const uint16_t* __restrict__ x, int64_t T, int G, int D,
                                                        uint8_t* __restrict__ xq, int32_t* __restrict__ xs) {
  const int lane = threadIdx.x & 63;
  const int HG = D / 32, PH = (HG + 3) / 4, PW = (PH + 3) / 4;
  const int64_t TA = (T + 3) / 4 * 4;
  const int64_t wid = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (wid >= TA * G * PW) return;
  const int pw = (int)(wid % PW);
  const int64_t tg = wid / PW;
  const int g = (int)(tg % G);
  const int64_t t = tg / G;
  const int r = lane >> 4, q = (lane >> 2) & 3;
  const int p = 4 * pw + r;  // this row's pack
  const int h = 4 * p + q;   // this quad's block
  int byte = 0;
  if (t < T && p < PH && h < HG) {
    const int64_t off = (t * G + g) * (int64_t)D + (int64_t)h * 32 + (lane & 3) * 8;
    uint4 u;
    if constexpr (NT) {
      const v4i l = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(x + off));
      u = uint4{(uint32_t)l[0], (uint32_t)l[1], (uint32_t)l[2], (uint32_t)l[3]};
    } else {
      u = *reinterpret_cast<const uint4*>(x + off);
    }
    float v[8];
    const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[2 * i] = __uint_as_float(w4[i] << 16);
      v[2 * i + 1] = __uint_as_float(w4[i] & 0xFFFF0000u);
    }
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(v[i]));
    // max over the quad: swap neighbours, then pairs (exec covers whole quads here)
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0xB1, 0xF, 0xF, false)));
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(a), 0x4E, 0xF, 0xF, false)));
    const int e = ue8m0_exp(a);
    const float sc = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e, e in [-127, 126]
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[0], sc), __fmul_rn(v[1], sc), lo, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[2], sc), __fmul_rn(v[3], sc), lo, true);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[4], sc), __fmul_rn(v[5], sc), hi, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(__fmul_rn(v[6], sc), __fmul_rn(v[7], sc), hi, true);
    *reinterpret_cast<uint2*>(xq + off) = uint2{lo, hi};
    byte = e + 127;
  }
  // the row's four quad bytes (0 for blocks past HG) form the pack word; lane 16 r writes it
  const int base = lane & ~15;
  const int b1 = __shfl(byte, base + 4, 64), b2 = __shfl(byte, base + 8, 64), b3 = __shfl(byte, base + 12, 64);
  if ((lane & 15) == 0 && p < PH) {
    const uint32_t word = (uint32_t)byte | ((uint32_t)b1 << 8) | ((uint32_t)b2 << 16) | ((uint32_t)b3 << 24);
    xs[((int64_t)g * PH + p) * TA + t] = (int32_t)word;
  }
}

hipError_t launch_group_quant_mx(const uint16_t* x, int64_t T, int G, int D, uint8_t* xq, int32_t* xs,
                                 hipStream_t st) {
  const int HG = D / 32, PH = (HG + 3) / 4, PW = (PH + 3) / 4;
  const int64_t TA = (T + 3) / 4 * 4;
  const int64_t waves = TA * G * PW;
  if (waves == 0) return hipSuccess;
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  if (waves >= 16384)
    hipLaunchKernelGGL(k_group_quant_mx<true>, grid, block, 0, st, x, T, G, D, xq, xs);
  else
    hipLaunchKernelGGL(k_group_quant_mx<false>, grid, block, 0, st, x, T, G, D, xq, xs);
  return hipGetLastError();
}

hipError_t launch_group_quant_fp8(const uint16_t* x, int64_t T, int G, int D, uint8_t* xq, int32_t* xs,
                                  hipStream_t st, int ppw_force) {
  const int HG = D / 128, PH = (HG + 3) / 4;
  const int64_t TA = (T + 3) / 4 * 4;
  // two packs per wave once the grid is large (>= 64 waves per CU at one pack per wave),
  // four from 128: fewer, longer waves with every load in flight measured faster there and
  // slower on small grids (G = 8, D = 4096, us at T = 64 / 256 / 512: one pack 3.77 / 8.79 /
  // 14.2, two 4.61 / 7.81 / 13.75, four 4.77 / 8.05 / 12.62)
  int ppw = TA * G * PH >= 32768 ? 4 : (TA * G * PH >= 16384 ? 2 : 1);
  if (ppw_force == 1 || ppw_force == 2 || ppw_force == 4 || ppw_force == 8) ppw = ppw_force;
  const int64_t waves = TA * G * ((PH + ppw - 1) / ppw);
  if (waves == 0) return hipSuccess;
  if (TA * G * PH >= ((int64_t)1 << 31)) return hipErrorInvalidValue;  // 32-bit wave and word indices
  dim3 grid((unsigned)((waves + 3) / 4)), block(256);
  const int Ti = (int)T;
  if (ppw == 8)
    hipLaunchKernelGGL(k_group_quant_fp8<8>, grid, block, 0, st, x, Ti, G, D, xq, xs);
  else if (ppw == 4)
    hipLaunchKernelGGL(k_group_quant_fp8<4>, grid, block, 0, st, x, Ti, G, D, xq, xs);
  else if (ppw == 2)
    hipLaunchKernelGGL(k_group_quant_fp8<2>, grid, block, 0, st, x, Ti, G, D, xq, xs);
  else
    hipLaunchKernelGGL(k_group_quant_fp8<1>, grid, block, 0, st, x, Ti, G, D, xq, xs);
  return hipGetLastError();
}

}  // namespace wq
