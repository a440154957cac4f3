// Fused decode linear in one launch: per-token INT8 quant of the bf16 rows, INT8 GEMM and
// the bf16 scale epilogue, for M < 256 rows and K <= 4096.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (BF16 X -> per-token dynamic quant ->
// INT8 GEMM -> BF16 Y, and the fused form that skips the standalone quant launch and the
// HBM round trip of the INT8 payload); section 三 (small M: the weight stream bounds the
// run, and the tiling follows the real M and N).
//
// Why this shape on MI355X: the 4 MiB weight of a 4096 x 1024 linear streams in ~0.5 us,
// a dependent second launch costs several us, and a cross-workgroup handoff (fence + flag)
// costs more than that.  So no workgroup waits on another: each one quantises the rows it
// needs itself, from L2, while its slice of the weights is in flight from HBM.
//  * The grid is (column slices of nt columns) x (row tiles of R rows).  Quantising costs
//    ~90 VALU instructions per 8 values per wave, so a workgroup that quantised all M rows
//    would spend most of the call on VALU work every other workgroup repeats; a row tile
//    of R rows bounds that, and the R-row tiles of one column slice run on one XCD
//    (workgroups are dispatched to the 8 XCDs round robin), whose L2 then fetches the
//    slice's weights from HBM once for all of them.
//  * 512 threads = 8 waves, wave w owns K range [w K/8, (w+1) K/8).  Every global load is
//    issued up front: the wave's chunk of each of its rows (16 bytes of 8 bf16 per lane),
//    then its weights straight into registers in the v_mfma_i32_16x16x64_i8 B layout
//    (CT = nt / 16 column tiles, or one partly used tile for nt < 16).
//  * The per-row absmax is reduced inside the wave with DPP and across the 8 waves through
//    LDS; each lane quantises its 8 values per row into the wave's private XOR-swizzled
//    LDS tile (the MFMA A operand) by the fast path (one fma per value with 1/s, whose bit
//    pattern holds both the code and a near-tie flag); a row where some lane meets a
//    near-tie, or whose scale is zero or not normal, is redone by the whole wave with the
//    exact quant_i8 behind a uniform branch, from the chunk still in registers.
//  * The 8 waves' int32 16 x 16 tiles are summed exactly in LDS and the epilogue writes
//    bf16((f32(acc) * s_m) * sw_n).
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

namespace {

constexpr int kFW = 8;            // waves per workgroup
constexpr int kFMaxKW = 512;      // K per wave: one 8-value chunk per lane per row
constexpr int kFMaxSteps = kFMaxKW / 64;

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

// INT8 codes of 8 bf16 values by the fast path of quant_i8 (one fma with inv ~ 1/s); *l is
// 0 when a value lies near a rounding tie (the codes are then not used)
__device__ __forceinline__ uint2 quant8_bf16_fast(const uint4 u, float inv, uint16_t* l) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  float v[8];
  uint32_t b[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    v[2 * i] = __uint_as_float(w[i] << 16);
    v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
  *l = quant_fast_lmin<8>(v, inv, b);
  return uint2{pack4_codes(b), pack4_codes(b + 4)};
}

// INT8 codes of 8 bf16 values by the exact quant_i8 (correctly rounded division)
__device__ __forceinline__ uint2 quant8_bf16_exact(const uint4 u, float s) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
  int c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = quant_i8(__uint_as_float(w[i] << 16), s);
    c[2 * i + 1] = quant_i8(__uint_as_float(w[i] & 0xFFFF0000u), s);
  }
  return uint2{pack4_i8(c[0], c[1], c[2], c[3]), pack4_i8(c[4], c[5], c[6], c[7])};
}

}  // namespace

// PREQ: the rows arrive quantised (p.a int8 with p.a_scale, the decode GEMM of
// wq_quant_matmul): the same kernel without the quantisation.
// PK: p.w holds the weights in fragment order (wq_pack_weight_i8): byte (n, k) at
// ((k/64 * N/4 + n/4) * 4 + (k%64)/16) * 64 + (n%4) * 16 + k%16, so the 16 columns x 64 K
// bytes of one MFMA B fragment are 1 KiB contiguous, in lane order.
template <int R, int CT, bool PREQ, bool PK>
__global__ __launch_bounds__(512) void k_fused_decode(DecodeArgs p, int nt, int slices, int rtiles) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int M = p.M, N = p.N, K = p.K;
  const int KW = K / kFW;           // this wave's K range (a multiple of 64, <= 512)
  const int steps = KW >> 6;
  const int kbase = wv * KW;

  // block -> (column slice, row tile): with slices % 8 == 0, XCD x (blocks b with b % 8 == x)
  // gets slices [x S/8, (x+1) S/8) with all their row tiles
  int slice, rt;
  if ((slices & 7) == 0) {
    const int x = blockIdx.x & 7, i = blockIdx.x >> 3;
    slice = x * (slices >> 3) + i / rtiles;
    rt = i - (i / rtiles) * rtiles;
  } else {
    slice = blockIdx.x / rtiles;
    rt = blockIdx.x - slice * rtiles;
  }
  const int n0 = slice * nt, row0 = rt * R;
  const int rows = min(R, M - row0);  // >= 1
  const int cl = lane & 15, kg = lane >> 4;
  const bool xlane = lane * 8 < KW;  // this lane holds a chunk of every row

  // LDS: [8 wave tiles of R x KW][red 8 x CT x 4 x 64 ints][wmax R x 8][s_lds R][wsc nt]
  int8_t* tile = smem + wv * R * KW;
  int* red = reinterpret_cast<int*>(smem + kFW * R * KW);
  uint32_t* wmax = reinterpret_cast<uint32_t*>(red + kFW * CT * 4 * 64);
  float* s_lds = reinterpret_cast<float*>(wmax + R * kFW);
  float* wsc_lds = s_lds + R;

  // ---- loads, all issued before the first wait: this wave's chunk of each row, the slice's
  // column scales, then the weights.  No load sits under a branch: lanes, rows and K steps
  // out of range read a clamped in-range address and their values go unused (a load under
  // a per-lane branch let the compiler wait for the first loads before issuing the rest,
  // which cost a second memory round trip).
  const int xl = min(lane, (KW >> 3) - 1);
  uint4 xr[PREQ ? 1 : R];   // bf16 rows: 8 values per lane
  uint2 xq8[PREQ ? R : 1];  // quantised rows: 8 codes per lane
  float s_pre = 0.0f;       // quantised rows: lane r < R holds row r's scale
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (PREQ)
      xq8[r] = *reinterpret_cast<const uint2*>(p.a + (int64_t)(row0 + min(r, rows - 1)) * p.lda + kbase + xl * 8);
    else
      xr[r] = *reinterpret_cast<const uint4*>(p.x + (int64_t)(row0 + min(r, rows - 1)) * p.ldx + kbase + xl * 8);
  }
  if constexpr (PREQ) s_pre = p.a_scale[row0 + min(lane, rows - 1)];
  const float wsc_v = p.w_scale[min(n0 + min(t, nt - 1), N - 1)];
  v4i b[CT][kFMaxSteps];
  // weight fragment idx = ct * kFMaxSteps + j
  auto load_w = [&](int idx) {
    const int ct = idx % CT, j = idx / CT;  // K-step-major: the order the MFMA loop takes them
    // B column cl of tile ct is output column ct * 16 + cl; columns past nt or N read a
    // column in range and are not stored
    const int c = CT == 1 ? (cl & (nt - 1)) : ct * 16 + cl;
    const int n = min(n0 + c, N - 1);
    if constexpr (PK) {
      // fragment j of this wave: K step kbase/64 + j, a (N/4) x 256-byte row of 4-column blocks.
      // Streaming loads: the weights are read once per call in whole 1 KiB pieces and need
      // no place in L2, which keeps it for the activation rows every workgroup re-reads
      // (measured 3.80 -> 3.44 us at M = 1, 9.41 -> 9.13 us at M = 64).  The plain layout
      // below reads half a 128-byte line per step and the other half one step later, so it
      // keeps ordinary loads.
      const int8_t* wfr = p.w + ((int64_t)(kbase >> 6) * (N >> 2) + (n >> 2)) * 256 + kg * 64 + (n & 3) * 16;
      b[ct][j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(wfr + (int64_t)min(j, steps - 1) * (N >> 2) * 256));
    } else {
      const int8_t* wcol = p.w + (int64_t)n * K + kbase + 16 * kg;
      b[ct][j] = *reinterpret_cast<const v4i*>(wcol + min(j, steps - 1) * 64);
    }
  };
  // With several rows to quantise the weights are requested only once the rows have landed,
  // a few fragments per quantised row: issued up front they queued ahead of the rows at the
  // address unit (which takes ~64 bytes a cycle per CU) and held back the absmax and the
  // quantisation, whose VALU work then covers their flight instead.  The first kEarly K
  // steps of every column tile still go out with the rows where that measured faster
  // (graph replays, cold weights): fragment order, R = 4 with two column tiles (the M = 32
  // shape): 6.00 -> 5.59 us; plain weights, R = 4 with one tile (M = 16): 5.43 -> 5.21 us,
  // and R = 8 with two (M = 64): 8.15 -> 8.00 us.  The other shapes measured slower with
  // them (fragment order M = 16: 4.84 -> 4.95 us, M = 64: 7.52 -> 7.75 us).  Fragments go
  // out K-step-major in the order the MFMA loop consumes them (M = 64: 7.59 -> 7.52 us).
  constexpr bool kLateW = !PREQ && R >= 4;  // at R = 2 the late weights were measured slower (5.08 -> 5.21 us)
  constexpr int kWLoads = CT * kFMaxSteps;
  constexpr int kEarlySteps = PK ? ((R == 4 && CT == 2) ? 2 : 0) : (((R == 4 && CT == 1) || (R == 8 && CT == 2)) ? 2 : 0);
  constexpr int kEarly = kLateW ? kEarlySteps * CT : kWLoads;
#pragma unroll
  for (int idx = 0; idx < kEarly; ++idx) load_w(idx);

  if constexpr (PREQ) {
    // ---- the given codes into the wave's tile, the given scales into LDS ----------------
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (r < rows && xlane) *reinterpret_cast<uint2*>(tile + fswz(r, lane >> 1, KW) + (lane & 1) * 8) = xq8[r];
    if (wv == 0 && lane < R) s_lds[lane] = s_pre;
  } else {
  // ---- per-row absmax: in-wave DPP reduction, then across waves through LDS ---------------
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const uint32_t a = r < rows ? wave_umax(bf16x8_absmax_bits(xr[r])) : 0u;  // uniform
    if (lane == 0) wmax[r * kFW + wv] = a;
  }
  lds_barrier();  // the weight loads stay in flight through the quantisation
  // lane r < R combines row r's 8 wave maxima and derives s = RN(a/127), inv = RN(1/s)
  float s_l = 0.0f, inv_l = 0.0f;
  if (lane < R) {
    const uint4 q0 = *reinterpret_cast<const uint4*>(wmax + lane * kFW);
    const uint4 q1 = *reinterpret_cast<const uint4*>(wmax + lane * kFW + 4);
    const uint32_t a = max(max(max(q0.x, q0.y), max(q0.z, q0.w)), max(max(q1.x, q1.y), max(q1.z, q1.w)));
    s_l = div127_bf16(__uint_as_float(a << 16));
    inv_l = recip_refined(s_l);
    if (wv == 0) s_lds[lane] = s_l;
    if (p.xs_out && slice == 0 && wv == 0 && lane < rows) p.xs_out[row0 + lane] = s_l;
  }

  // ---- quantise this lane's 8 values of each row into the wave's tile ----------------------
  // Per row, the fast codes (one fma per value, quant_fast_lmin); where some lane's chunk
  // holds a near-tie, or the row's scale is zero, subnormal or infinite, the whole wave
  // replaces them with the exact codes of that row at once, from the chunk still in its
  // registers.  The branch is uniform (a ballot), so a row without a near-tie costs one
  // compare and a few scalar instructions.  Only a few rows per call meet a near-tie, but
  // their workgroups set the call's time: a marked-row loop after all rows either kept every
  // row's chunk live through the whole quantisation (R = 16: 158 VGPRs against 101) or
  // re-read it from L2 (a round trip per marked row; M = 64: 8.68 -> 9.49 us on plain
  // weights).  Rows past `rows` (the last tile) are quantised from their clamped copies into
  // tile rows the MFMA never reads, and never re-done.  The tile offset of chunk c of row r
  // is r KW + ((c ^ (r % g)) << 4): the XOR with a per-row constant applies to this lane's
  // fixed chunk offset.
  const bool export_q = p.xq_out != nullptr && slice == 0;
  const int chunks = KW >> 4;
  const int gmask = min(16, chunks & -chunks) - 1;
  const int lane_off = ((lane >> 1) << 4) + (lane & 1) * 8;
  const uint32_t abnormal = (uint32_t)__builtin_amdgcn_ballot_w64(lane < R && !quant_scale_normal(s_l));
  const uint64_t xmask = __builtin_amdgcn_ballot_w64(xlane);
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if constexpr (kLateW) {  // this row's share of the weight fragments, outside any branch
#pragma unroll
      for (int idx = kEarly + r * (kWLoads - kEarly) / R; idx < kEarly + (r + 1) * (kWLoads - kEarly) / R; ++idx)
        load_w(idx);
    }
    const float inv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(inv_l), r));
    uint16_t l;
    uint2 q = quant8_bf16_fast(xr[r], inv, &l);
    const bool tie = (__builtin_amdgcn_ballot_w64(l == 0) & xmask) != 0;
    if (r < rows && (tie || ((abnormal >> r) & 1u))) {  // uniform
      const float s = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s_l), r));
      q = quant8_bf16_exact(xr[r], s);
    }
    if (xlane) {
      *reinterpret_cast<uint2*>(tile + r * KW + (lane_off ^ ((r & gmask) << 4))) = q;
      if (export_q && r < rows) *reinterpret_cast<uint2*>(p.xq_out + (int64_t)(row0 + r) * K + kbase + lane * 8) = q;
    }
  }
  }  // quantisation

  // ---- MFMA over this wave's K range (the tile is private to the wave); MFMA rows past
  // the tile's rows repeat its last row and are not stored -----------------------------------
  v4i acc[CT];
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) acc[ct] = v4i{0, 0, 0, 0};
  const int ar = min(cl, rows - 1);
#pragma unroll
  for (int j = 0; j < kFMaxSteps; ++j) {
    if (j < steps) {
      const v4i a = *reinterpret_cast<const v4i*>(tile + fswz(ar, j * 4 + kg, KW));
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) acc[ct] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[ct][j], acc[ct], 0, 0, 0);
    }
  }

  // ---- sum the 8 waves' tiles, epilogue -----------------------------------------------------
  // (the column scales go to LDS only now: storing them earlier would wait for every load
  // issued before them, the weights included, ahead of the quantisation)
  if (t < nt) wsc_lds[t] = n0 + t < N ? wsc_v : 0.0f;
#pragma unroll
  for (int ct = 0; ct < CT; ++ct)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wv * CT + ct) * 4 + i) * 64 + lane] = acc[ct][i];
  __syncthreads();
  for (int o = t; o < rows * nt; o += kFW * 64) {
    const int r = o / nt, c = o - r * nt;
    const int n = n0 + c;
    if (n < N) {
      const int ct = c >> 4;
      const int ln = (c & 15) + 16 * (r >> 2), i = r & 3;  // MFMA 16x16 output: col = lane % 16, row = 4 (lane / 16) + i
      int v = 0;
#pragma unroll
      for (int w = 0; w < kFW; ++w) v += red[((w * CT + ct) * 4 + i) * 64 + ln];
      const int64_t m = row0 + r;
      p.y[m * p.ldy + n] = (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)v, s_lds[r]), wsc_lds[c]));
      if (p.acc_out) p.acc_out[m * N + n] = v;
    }
  }
}

namespace {

size_t fused_lds_bytes(int R, int CT, int K) {
  return (size_t)kFW * R * (K / kFW) + (size_t)kFW * CT * 4 * 64 * 4 + (size_t)R * kFW * 4 + (size_t)R * 4 + 32 * 4;
}

template <int R, int CT, bool PREQ, bool PK>
hipError_t launch_fused_rt(const DecodeArgs& a, int nt, hipStream_t st) {
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(k_fused_decode<R, CT, PREQ, PK>), 160 * 1024);
  if (e != hipSuccess) return e;
  const int slices = (a.N + nt - 1) / nt, rtiles = (a.M + R - 1) / R;
  hipLaunchKernelGGL((k_fused_decode<R, CT, PREQ, PK>), dim3((unsigned)(slices * rtiles)), dim3(kFW * 64),
                     fused_lds_bytes(R, CT, a.K), st, a, nt, slices, rtiles);
  return hipGetLastError();
}

template <int R>
hipError_t launch_fused_r(const DecodeArgs& a, int nt, bool packed, hipStream_t st) {
  if (a.x == nullptr && packed)
    return nt > 16 ? launch_fused_rt<R, 2, true, true>(a, nt, st) : launch_fused_rt<R, 1, true, true>(a, nt, st);
  if (a.x == nullptr)
    return nt > 16 ? launch_fused_rt<R, 2, true, false>(a, nt, st) : launch_fused_rt<R, 1, true, false>(a, nt, st);
  if (packed)
    return nt > 16 ? launch_fused_rt<R, 2, false, true>(a, nt, st) : launch_fused_rt<R, 1, false, true>(a, nt, st);
  return nt > 16 ? launch_fused_rt<R, 2, false, false>(a, nt, st) : launch_fused_rt<R, 1, false, false>(a, nt, st);
}

// fragment-order weights: thread i writes the i-th 16-byte piece of wp, read from row
// n = 4 (i / 16 % (N/4)) + i % 4, bytes 64 (i / (4 N)) + 16 (i / 4 % 4) of w
__global__ __launch_bounds__(256) void k_pack_weight_i8(const int8_t* __restrict__ w, int64_t ldw, int N, int K,
                                                        int8_t* __restrict__ wp) {
  const int64_t pieces = (int64_t)N * (K / 16);
  for (int64_t i = blockIdx.x * 256ll + threadIdx.x; i < pieces; i += (int64_t)gridDim.x * 256) {
    const int c = (int)(i & 3), kg = (int)((i >> 2) & 3);
    const int64_t blk = i >> 4;  // ks * (N/4) + nb4
    const int nb4 = (int)(blk % (N >> 2));
    const int64_t ks = blk / (N >> 2);
    const int n = nb4 * 4 + c;
    const int64_t k = ks * 64 + kg * 16;
    *reinterpret_cast<uint4*>(wp + i * 16) = *reinterpret_cast<const uint4*>(w + (int64_t)n * ldw + k);
  }
}

}  // namespace

bool fused_decode_fits(int M, int K) {
  return M >= 1 && M < 256 && K % (kFW * 64) == 0 && K / kFW <= kFMaxKW;
}

bool given_decode_fits(int M, int K) {
  return M >= 1 && M < 256 && K % (kFW * 64) == 0 && K / kFW <= kFMaxKW;
}

hipError_t launch_fused_decode(const DecodeArgs& a, int nt, int rows_per_wg, hipStream_t st, bool packed) {
  if (!(a.x != nullptr ? fused_decode_fits(a.M, a.K) : given_decode_fits(a.M, a.K)) ||
      (a.x == nullptr && (a.a == nullptr || a.a_scale == nullptr)) ||
      !(nt == 4 || nt == 8 || nt == 16 || nt == 32) || (packed && a.N % 4 != 0))
    return hipErrorInvalidValue;
  switch (rows_per_wg) {
    case 1: return launch_fused_r<1>(a, nt, packed, st);
    case 2: return launch_fused_r<2>(a, nt, packed, st);
    case 4: return launch_fused_r<4>(a, nt, packed, st);
    case 8: return launch_fused_r<8>(a, nt, packed, st);
    case 16: return launch_fused_r<16>(a, nt, packed, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_pack_weight_i8(const int8_t* w, int64_t ldw, int N, int K, int8_t* wp, hipStream_t st) {
  if (N % 4 != 0 || K % 64 != 0 || ldw < K || ldw % 16 != 0) return hipErrorInvalidValue;
  const int64_t pieces = (int64_t)N * (K / 16);
  if (pieces == 0) return hipSuccess;
  const int64_t blocks = min((pieces + 255) / 256, (int64_t)65536);
  hipLaunchKernelGGL(k_pack_weight_i8, dim3((unsigned)blocks), dim3(256), 0, st, w, ldw, N, K, wp);
  return hipGetLastError();
}

}  // namespace wq
