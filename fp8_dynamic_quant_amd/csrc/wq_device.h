// Device-side helpers shared by the wq kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;

// Workgroup barrier for hand-offs through LDS.  __syncthreads() also carries a workgroup
// release fence, which the compiler implements by waiting for every outstanding global
// load first (s_waitcnt vmcnt(0)): loads issued ahead on purpose (the later slices of an
// LDS-DMA ring, the next item's operands) then land before anyone passes the barrier.
// This barrier waits only for the wave's own LDS operations; a wave that needs its LDS-DMA
// data waits for it with an explicit vmcnt first.  The memory clobber keeps the compiler
// from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// bf16 bits -> f32: the bf16 pattern is the high half of the binary32 pattern.
__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// f32 -> bf16 bits, round to nearest even (inputs are finite; overflow gives inf).
__device__ __forceinline__ uint32_t f32_to_bf16_rn(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// max over the 64 lanes of a wave of non-negative floats (compared as their bit patterns),
// returned to every lane: quad swaps, half-row and row mirrors by DPP, then the four rows'
// maxima through readlane
__device__ __forceinline__ float wave_max_nonneg(float f) {
  uint32_t v = __float_as_uint(f);
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row half mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return __uint_as_float(max(a, b));
}

// RN(a / 127) for a non-negative bf16 value a: m = RN(a c) with c = RN(1/127), then one
// correction step with the exact residual a - 127 m.  Equal to the correctly rounded
// quotient for every bf16 a (checked exhaustively with exact rationals on the CPU); the plain
// product alone misses it for some.
__device__ __forceinline__ float div127_bf16(float a) {
  constexpr float c = 1.0f / 127.0f;  // RN(1/127)
  const float m = __fmul_rn(a, c);
  const float r = __builtin_fmaf(-127.0f, m, a);
  return __builtin_fmaf(r, c, m);
}

// 1/s for a normal s with relative error below 2^-24 (1 + 2^-20): v_rcp_f32 (1 ulp) and one
// Newton step.  The fast quant paths need 1/s within 2^-22.4 (quant_fast) and 2^-23.4
// (quant_fast_lmin); the exact path divides by s itself.
__device__ __forceinline__ float recip_refined(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  const float e = __builtin_fmaf(-s, r0, 1.0f);
  return __builtin_fmaf(r0, e, r0);
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Per-token INT8 code: clamp(rint(RN(v / s)), -127, 127); s == 0 gives 0.
__device__ __forceinline__ int quant_i8(float v, float s) {
  if (s == 0.0f) return 0;
  float r = rintf(__fdiv_rn(v, s));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
}

// Fast path of quant_i8 for N values at once, without the division, for a normal finite
// scale s (s = RN(absmax/127), so |v/s| <= 127 (1 + 2^-23) for every value of the row).
// With inv = RN(1/s) (or any inv within relative 2^-22.4 of 1/s: the slack below allows
// 127 |inv s - 1| < 2^-15 - 2^-25 - 127 2^-24) and e = v * inv (exact product),
// |e - v/s| < 2^-17.  One fma gives
// u = RN(e + P) with P = 1.5 * 2^23: in that binade the unit is 1, so u = P + n with
// n = e rounded to the nearest integer, and u's low byte is n in two's complement.  A second
// fma gives d = RN(e - n) (P - u = -n is exact).  When every |d| < 0.5 - 2^-15, then
// |e - n| < 0.5 - 2^-15 + 2^-25 and RN(v/s), which lies within 2^-16 of e, is strictly
// within 0.5 of n, so it rounds to the same integer n, which is within [-127, 127],
// so n is quant_i8's code and the clamp is moot.  Returns false for a near-tie (the caller
// then takes the exact path for these N values; a wave branches once per N values, not per
// value).  u[i] receives the bit patterns of the biased sums.
template <int N>
__device__ __forceinline__ bool quant_fast(const float* v, float inv, uint32_t* u) {
  constexpr float kPlace = 12582912.0f;          // 1.5 * 2^23
  constexpr float kGuard = 0.499969482421875f;   // 0.5 - 2^-15
  float dmax = 0.0f;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const float b = __builtin_fmaf(v[i], inv, kPlace);
    u[i] = __float_as_uint(b);
    dmax = fmaxf(dmax, fabsf(__builtin_fmaf(v[i], inv, __fsub_rn(kPlace, b))));
  }
  return dmax < kGuard;
}

// four biased sums P + n (n in [-128, 127]) -> the four codes n packed little endian:
// v_perm_b32 gathers the low bytes
__device__ __forceinline__ uint32_t pack4_biased(const uint32_t* u) {
  // selector byte k picks output byte k: 0..3 = bytes of the second operand, 4..7 = bytes
  // of the first, 0x0c = zero
  const uint32_t lo = __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0400u);  // u0.byte0, u1.byte0, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(u[3], u[2], 0x04000c0cu);  // 0, 0, u2.byte0, u3.byte0
  return lo | hi;
}

// A second fast path of quant_i8, with one fma per value: for a normal finite scale
// s = RN(a/127) of the row's absmax a, so |v/s| <= 127 (1 + 2^-24) for every value.  It needs
// inv within relative 2^-23.4 of 1/s (RN(1/s) and recip_refined are within 2^-24 (1 + 2^-20)),
// so that e = v * inv (the exact product, inside the fma) lies within 2^-17 of v/s.  The fma
// gives b = RN(e + 384): in [256, 512) the unit is 2^-15, so b is 256 + M 2^-15 with M the low
// 23 bits of b's pattern, and |M 2^-15 - (e + 128)| <= 2^-16.  Adding 2^14 - 128 * 2^15 to the
// pattern and shifting it left by one leaves n = floor(M 2^-15 + 1/2) - 128 in bits 16..23
// (two's complement) and 2 L in the low 16 bits, L = (M + 2^14) mod 2^15.  When L != 0,
// M 2^-15 + 1/2 is at least 2^-15 from every integer, so v/s + 128 + 1/2 (within
// 2^-16 + 2^-17 of it) is more than 2^-17 from one: v/s lies strictly between n - 1/2 and
// n + 1/2 and more than half an ulp of either (at most 2^-18 below 128) inside, so RN(v/s)
// does too and rounds to n, which is in [-127, 127]: n is quant_i8's code and the clamp is
// moot.  Returns the minimum of the 2 L over the N values (0: a near-tie; the caller then
// takes the exact path for them); u[i] receives the shifted patterns (pack4_codes packs
// them).  Checked against exact rationals on the CPU for near-tie values at every bf16
// absmax, with rcp results one ulp either side of RN(1/s).  Per value it costs an fma, an
// add-and-shift and about one 16-bit minimum, against quant_fast's four: the fused decode
// GEMM quantises in a VALU-bound phase.
template <int N>
__device__ __forceinline__ uint16_t quant_fast_lmin(const float* v, float inv, uint32_t* u) {
  constexpr float kPlace = 384.0f;                // 1.5 * 2^8
  constexpr uint32_t kAdj = 0x4000u - 0x400000u;  // + 2^14 (rounds), - 128 * 2^15 (recentres)
#pragma unroll
  for (int i = 0; i < N; ++i) u[i] = (__float_as_uint(__builtin_fmaf(v[i], inv, kPlace)) + kAdj) << 1;
  uint16_t m = (uint16_t)u[0];
#pragma unroll
  for (int i = 1; i < N; ++i) m = __builtin_elementwise_min(m, (uint16_t)u[i]);
  return m;
}

// four shifted patterns of quant_fast_lmin -> the four codes (byte 2 of each) packed little
// endian, by v_perm_b32 as in pack4_biased
__device__ __forceinline__ uint32_t pack4_codes(const uint32_t* u) {
  const uint32_t lo = __builtin_amdgcn_perm(u[1], u[0], 0x0c0c0602u);  // u0.byte2, u1.byte2, 0, 0
  const uint32_t hi = __builtin_amdgcn_perm(u[3], u[2], 0x06020c0cu);  // 0, 0, u2.byte2, u3.byte2
  return lo | hi;
}

// the fast path's precondition on the scale: normal and finite (a zero, subnormal or
// infinite scale goes to the exact path, where the clamp and the s == 0 rule act)
__device__ __forceinline__ bool quant_scale_normal(float s) {
  return s >= 1.17549435e-38f && s <= 3.40282347e+38f;
}

// INT8 codes of 8 values (two packed words), bit-identical to quant_i8 on each value.
__device__ __forceinline__ uint2 quant8(const float* v, float s, float inv) {
  uint32_t u[8];
  if (quant_scale_normal(s) && quant_fast<8>(v, inv, u)) return uint2{pack4_biased(u), pack4_biased(u + 4)};
  return uint2{pack4_i8(quant_i8(v[0], s), quant_i8(v[1], s), quant_i8(v[2], s), quant_i8(v[3], s)),
               pack4_i8(quant_i8(v[4], s), quant_i8(v[5], s), quant_i8(v[6], s), quant_i8(v[7], s))};
}

// INT8 codes of 4 values (one packed word), bit-identical to quant_i8 on each value.
__device__ __forceinline__ uint32_t quant4(const float* v, float s, float inv) {
  uint32_t u[4];
  if (quant_scale_normal(s) && quant_fast<4>(v, inv, u)) return pack4_biased(u);
  return pack4_i8(quant_i8(v[0], s), quant_i8(v[1], s), quant_i8(v[2], s), quant_i8(v[3], s));
}

// max |x| over 8 bf16 values packed in 16 bytes
__device__ __forceinline__ float bf16x8_absmax(const uint4 u) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a = fmaxf(a, fabsf(__uint_as_float(w[i] << 16)));
    a = fmaxf(a, fabsf(__uint_as_float(w[i] & 0xFFFF0000u)));
  }
  return a;
}

// INT8 codes of 8 bf16 values (16 bytes) -> 8 bytes
__device__ __forceinline__ uint2 quant8_bf16(const uint4 u, float s, float inv) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float v[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  return quant8(v, s, inv);
}

// Fixed-sequence f32 exp: n = rint(x*log2e); r = (x - n*ln2_hi) - n*ln2_lo;
// p = Horner of the degree-7 Taylor polynomial (coefficients 1/k! rounded to f32);
// result p * 2^n rounded once.  Every step is one correctly rounded f32 operation.
__device__ __forceinline__ float exp_fixed(float x) {
  const float kLog2e = 1.44269502162933349609375f;    // f32(log2 e)
  const float kLn2Hi = 0.693359375f;                   // 355/512
  const float kLn2Lo = -2.12194440e-4f;                // f32(ln2 - 355/512)
  float n = rintf(__fmul_rn(x, kLog2e));
  if (n > 128.0f) return __int_as_float(0x7F800000);
  if (n < -151.0f) return 0.0f;
  float r = __fsub_rn(__fsub_rn(x, __fmul_rn(n, kLn2Hi)), __fmul_rn(n, kLn2Lo));
  float p = 1.98412701e-4f;                            // 1/5040
  p = __fadd_rn(__fmul_rn(p, r), 1.38888892e-3f);      // 1/720
  p = __fadd_rn(__fmul_rn(p, r), 8.33333377e-3f);      // 1/120
  p = __fadd_rn(__fmul_rn(p, r), 4.16666679e-2f);      // 1/24
  p = __fadd_rn(__fmul_rn(p, r), 1.66666672e-1f);      // 1/6
  p = __fadd_rn(__fmul_rn(p, r), 0.5f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  p = __fadd_rn(__fmul_rn(p, r), 1.0f);
  return ldexpf(p, (int)n);
}

}  // namespace wq
