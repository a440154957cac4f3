// Fused decode linear in one launch: per-token INT8 quant of the bf16 rows, INT8 GEMM and
// the bf16 scale epilogue, for M <= 64 rows and K <= 4096.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (BF16 X -> per-token dynamic quant ->
// INT8 GEMM -> BF16 Y, and the fused form that skips the standalone quant launch and the
// HBM round trip of the INT8 payload); section 三 (small M: the weight stream bounds the
// run, so the launch shape follows N, not M).
//
// Why this shape on MI355X: the 4 MiB weight of a 4096 x 1024 linear streams in ~0.5 us,
// a dependent second launch costs several us, and a cross-workgroup handoff (fence + flag)
// costs more than that.  So each workgroup quantises the few activation rows itself, from
// L2, while its slice of the weights is still in flight from HBM:
//  * 512 threads = 8 waves per workgroup, NT output columns per workgroup (N / NT
//    workgroups, e.g. 256 for N = 1024), and wave w owns K range [w K/8, (w+1) K/8);
//  * every global load is issued up front: first the wave's activation chunks (one 16-byte
//    chunk of 8 bf16 per lane per row, so the rows are waited on first), then its weights
//    straight into registers in the v_mfma_i32_16x16x64_i8 B layout;
//  * rows go in groups of 16 (one MFMA row tile): the per-row absmax is reduced inside the
//    wave with DPP (no LDS round trips) and across the 8 waves through LDS, then each lane
//    quantises its own 8 values per row (quant8: one exactness check per 8 values) into the
//    wave's private, XOR-swizzled LDS tile, which feeds the MFMA A operand;
//  * the 8 waves' int32 16 x 16 tiles are summed exactly in LDS and the epilogue writes
//    bf16((f32(acc) * s_m) * sw_n).
// Every workgroup quantises all M rows (M K values); at M <= 16 that costs less VALU time
// than the weight stream takes to arrive.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

namespace {

constexpr int kFW = 8;            // waves per workgroup
constexpr int kFMaxKW = 512;      // K per wave: one 8-value chunk per lane per row
constexpr int kFMaxSteps = kFMaxKW / 64;
constexpr int kFMaxGroups = 4;    // 16-row groups: M <= 64

typedef __attribute__((address_space(3))) void* lds_ptr_f;

// byte offset of 16-byte chunk c of row r (r < 16) in a tile of rows of `rowb` bytes;
// chunks XOR-swizzled by the row within aligned groups of g chunks so the MFMA A reads
// (16 rows at one chunk) spread over the banks
__device__ __forceinline__ int fswz(int r, int c, int rowb) {
  const int chunks = rowb >> 4;
  const int g = min(16, chunks & -chunks);
  return r * rowb + ((c ^ (r & (g - 1))) << 4);
}

// max over the 64 lanes of a wave of non-negative values held as uint bit patterns; the
// result is wave-uniform.  Quad swaps, then half-row and row mirrors (each lane ends with
// the max of its row of 16), then the four rows through readlane.
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));   // quad [1,0,3,2]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));   // quad [2,3,0,1]
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));  // row half mirror
  v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));  // row mirror
  const uint32_t a = max((uint32_t)__builtin_amdgcn_readlane((int)v, 0), (uint32_t)__builtin_amdgcn_readlane((int)v, 16));
  const uint32_t b = max((uint32_t)__builtin_amdgcn_readlane((int)v, 32), (uint32_t)__builtin_amdgcn_readlane((int)v, 48));
  return max(a, b);
}

// max |x| of 8 bf16 values as the bit pattern of a non-negative bf16 (finite inputs)
__device__ __forceinline__ uint32_t bf16x8_absmax_bits(const uint4 u) {
  typedef unsigned short us2 __attribute__((ext_vector_type(2)));
  const uint32_t m = 0x7FFF7FFFu;
  const us2 a = __builtin_bit_cast(us2, u.x & m), b = __builtin_bit_cast(us2, u.y & m);
  const us2 c = __builtin_bit_cast(us2, u.z & m), d = __builtin_bit_cast(us2, u.w & m);
  const us2 e = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
  return max((uint32_t)e.x, (uint32_t)e.y);
}

}  // namespace

__global__ __launch_bounds__(512) void k_fused_decode(DecodeArgs p, int nt) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int KW = K / kFW;           // this wave's K range (a multiple of 64, <= 512)
  const int steps = KW >> 6;
  const int kbase = wv * KW;
  const int n0 = blockIdx.x * nt;
  const int cl = lane & 15, kg = lane >> 4;
  const int col = n0 + cl;
  const bool bvalid = cl < nt && col < N;
  const int G = (M + 15) >> 4;
  const bool xlane = lane * 8 < KW;  // this lane holds a chunk of every row

  // LDS: [8 wave tiles of 16 x KW][red 8 x G x 4 x 64 ints][wmax G x 16 x 8][s_lds 64][wsc 16]
  int8_t* tile = smem + wv * 16 * KW;
  int* red = reinterpret_cast<int*>(smem + kFW * 16 * KW);
  uint32_t* wmax = reinterpret_cast<uint32_t*>(red + kFW * kFMaxGroups * 4 * 64);
  float* s_lds = reinterpret_cast<float*>(wmax + kFMaxGroups * 16 * kFW);
  float* wsc_lds = s_lds + 64;

  // ---- loads: this wave's chunks of the first row group, then its weights ----------------
  uint4 xr[16];
  auto load_rows = [&](int g) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = g * 16 + r;
      xr[r] = (row < M && xlane) ? *reinterpret_cast<const uint4*>(p.x + (int64_t)row * p.ldx + kbase + lane * 8)
                                 : uint4{0u, 0u, 0u, 0u};
    }
  };
  load_rows(0);
  v4i b[kFMaxSteps];
  const int8_t* wcol = p.w + (int64_t)col * K + kbase + 16 * kg;
#pragma unroll
  for (int j = 0; j < kFMaxSteps; ++j)
    b[j] = (bvalid && j < steps) ? *reinterpret_cast<const v4i*>(wcol + j * 64) : v4i{0, 0, 0, 0};
  if (t < nt) wsc_lds[t] = (n0 + t < N) ? p.w_scale[n0 + t] : 0.0f;

  v4i acc[kFMaxGroups];
#pragma unroll
  for (int g = 0; g < kFMaxGroups; ++g) acc[g] = v4i{0, 0, 0, 0};

#pragma unroll
  for (int g = 0; g < kFMaxGroups; ++g) {
    if (g < G) {  // uniform
      if (g > 0) load_rows(g);
      // ---- per-row absmax: in-wave DPP reduction, then across waves through LDS ---------
      uint32_t* wm = wmax + g * 16 * kFW;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t a = (g * 16 + r < M) ? wave_umax(bf16x8_absmax_bits(xr[r])) : 0u;  // uniform
        if (lane == 0) wm[r * kFW + wv] = a;
      }
      __syncthreads();
      // lane r < 16 combines row r's 8 wave maxima and derives s = RN(a/127), inv = RN(1/s)
      float s_l = 0.0f, inv_l = 0.0f;
      if (lane < 16) {
        const uint4 q0 = *reinterpret_cast<const uint4*>(wm + lane * kFW);
        const uint4 q1 = *reinterpret_cast<const uint4*>(wm + lane * kFW + 4);
        const uint32_t a = max(max(max(q0.x, q0.y), max(q0.z, q0.w)), max(max(q1.x, q1.y), max(q1.z, q1.w)));
        s_l = __fdiv_rn(__uint_as_float(a << 16), 127.0f);
        inv_l = __fdiv_rn(1.0f, s_l);
        if (wv == 0) s_lds[g * 16 + lane] = s_l;
        if (p.xs_out && blockIdx.x == 0 && wv == 0 && g * 16 + lane < M) p.xs_out[g * 16 + lane] = s_l;
      }
      // ---- quantise this lane's 8 values of each row into the wave's tile ----------------
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_l), r));
        const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_l), r));
        if (xlane) {
          // rows past M quantise to zero (their accumulator rows are not stored)
          const uint2 q = (g * 16 + r < M) ? quant8_bf16(xr[r], s, inv) : uint2{0u, 0u};
          *reinterpret_cast<uint2*>(tile + fswz(r, lane >> 1, KW) + (lane & 1) * 8) = q;
          const int row = g * 16 + r;
          if (p.xq_out && blockIdx.x == 0 && row < M)
            *reinterpret_cast<uint2*>(p.xq_out + (int64_t)row * K + kbase + lane * 8) = q;
        }
      }
      // ---- MFMA over this wave's K range (the tile is private to the wave) ---------------
#pragma unroll
      for (int j = 0; j < kFMaxSteps; ++j) {
        if (j < steps) {
          const v4i a = *reinterpret_cast<const v4i*>(tile + fswz(cl, j * 4 + kg, KW));
          acc[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[j], acc[g], 0, 0, 0);
        }
      }
    }
  }

  // ---- sum the 8 waves' tiles, epilogue -----------------------------------------------------
#pragma unroll
  for (int g = 0; g < kFMaxGroups; ++g)
    if (g < G)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wv * kFMaxGroups + g) * 4 + i) * 64 + lane] = acc[g][i];
  __syncthreads();
  for (int o = t; o < M * nt; o += kFW * 64) {
    const int row = o / nt, c = o - row * nt;
    const int n = n0 + c;
    if (n < N) {
      const int g = row >> 4, rr = row & 15;
      const int ln = c + 16 * (rr >> 2), i = rr & 3;  // MFMA 16x16 output: col = lane % 16, row = 4 (lane / 16) + i
      int v = 0;
#pragma unroll
      for (int w = 0; w < kFW; ++w) v += red[((w * kFMaxGroups + g) * 4 + i) * 64 + ln];
      p.y[(int64_t)row * p.ldy + n] = (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)v, s_lds[row]), wsc_lds[c]));
      if (p.acc_out) p.acc_out[(int64_t)row * N + n] = v;
    }
  }
}

size_t fused_decode_lds_bytes(int K) {
  return (size_t)kFW * 16 * (K / kFW) + (size_t)kFW * kFMaxGroups * 4 * 64 * 4 + (size_t)kFMaxGroups * 16 * kFW * 4 +
         64 * 4 + 16 * 4;
}

bool fused_decode_fits(int M, int K) {
  return M >= 1 && M <= 16 * kFMaxGroups && K % (kFW * 64) == 0 && K / kFW <= kFMaxKW;
}

hipError_t launch_fused_decode(const DecodeArgs& a, int nt, hipStream_t st) {
  if (!fused_decode_fits(a.M, a.K) || a.x == nullptr || !(nt == 4 || nt == 8 || nt == 16)) return hipErrorInvalidValue;
  const size_t lds = fused_decode_lds_bytes(a.K);
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(k_fused_decode),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  hipLaunchKernelGGL(k_fused_decode, dim3((unsigned)((a.N + nt - 1) / nt)), dim3(kFW * 64), lds, st, a, nt);
  return hipGetLastError();
}

}  // namespace wq
