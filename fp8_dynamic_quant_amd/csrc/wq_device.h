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

// The same code as quant_i8, usually without the division.  With inv = RN(1/s),
// t = RN(v * inv) lies within |v/s| * 1.5 * 2^-23 of RN(v/s) (three roundings of 2^-24
// each).  When t is farther than that from every half-integer, RN(v/s) and t share the
// integer they round to, so rint(t) is the answer; otherwise (ties and near-ties, or a
// non-finite t when s is subnormal) the correctly rounded division decides.
__device__ __forceinline__ int quant_i8_fast(float v, float s, float inv) {
  if (s == 0.0f) return 0;
  const float tq = __fmul_rn(v, inv);
  float r = rintf(tq);
  const float d = fabsf(__fsub_rn(tq, r));
  const float margin = __fmul_rn(fmaxf(fabsf(tq), 1.0f), 4.8e-7f);
  if (!(__fsub_rn(0.5f, d) > margin)) r = rintf(__fdiv_rn(v, s));
  r = fminf(fmaxf(r, -127.0f), 127.0f);
  return (int)r;
}

__device__ __forceinline__ uint32_t pack4_i8(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xFF) | ((uint32_t)(b & 0xFF) << 8) | ((uint32_t)(c & 0xFF) << 16) |
         ((uint32_t)(d & 0xFF) << 24);
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
  int q[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    q[2 * i] = quant_i8_fast(__uint_as_float(w[i] << 16), s, inv);
    q[2 * i + 1] = quant_i8_fast(__uint_as_float(w[i] & 0xFFFF0000u), s, inv);
  }
  return uint2{pack4_i8(q[0], q[1], q[2], q[3]), pack4_i8(q[4], q[5], q[6], q[7])};
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
