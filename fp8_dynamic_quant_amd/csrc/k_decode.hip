// Decode-sized INT8 W8A8 linear (M <= 64): weight streaming with no inter-workgroup traffic.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (per-token quant, INT8 GEMM, BF16
// epilogue; a Linear may take the (INT8, scale) tuple instead of quantising) and section
// 三 (small M: the launch shape comes from the real M, N, K).
//
// Why this shape on MI355X: at decode M the whole weight (4 MiB for 4096x1024) streams
// in ~0.5 us at HBM rate, while a kernel dispatch costs ~1.7 us and device-scope atomics
// or fences between workgroups cost several us more.  So each workgroup owns NT output
// columns and the WHOLE K range and never talks to another workgroup, and every global
// load it needs is issued before it waits on any of them (one memory round trip):
//  * its four waves split K in quarters; each wave loads its weights (16 bytes per lane
//    per 64-deep step) straight into registers in the MFMA B layout;
//  * the activations go global -> LDS with global_load_lds_dwordx4 (no VGPR staging),
//    each wave fetching the rows of its own K quarter, in rounds when M rows do not fit;
//    the 16-byte chunks of a row are XOR-swizzled by the row index so the MFMA A reads
//    (16 rows, same chunk) hit 16 different bank groups;
//  * v_mfma_i32_16x16x64_i8 accumulates; the four waves' int32 tiles are summed in LDS
//    (exact) and the scale epilogue writes bf16.
// NT < 16 leaves MFMA column slots empty (their lanes load nothing): compute is cheap here
// and the narrower tile puts N/NT workgroups on the chip, e.g. 256 for N = 1024.
// Above 16 rows the grid's second dimension splits the rows into tiles of 16*MT: every
// workgroup reads all its rows' activations from L2, so at M = 64 a workgroup per 16 rows
// with 16 columns moves 128 KiB per CU instead of 272 KiB for all 64 rows and 4 columns.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

constexpr int kDecodeChunk = 16;      // 64-deep k-steps of weights held in registers per wave
constexpr int kDecodeRoundBytes = 128 * 1024;  // LDS for one round of staged activations

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ uint16_t epi_bf16_d(int acc, float s, float sw) {
  return (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)acc, s), sw));
}

// Byte offset of 16-byte chunk c of row m in rows of `rowb` bytes, XOR-swizzled within
// aligned groups of G chunks (G = the largest power of two <= 16 dividing the row's chunk
// count; rows here always hold a multiple of 4 chunks).
__device__ __forceinline__ int swz(int m, int c, int rowb) {
  const int chunks = rowb >> 4;
  const int g = min(16, chunks & -chunks);
  return m * rowb + ((c ^ (m & (g - 1))) << 4);
}

__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// 64-deep k-steps per staging round: a power of two in [4, 64] (so rounds and the
// 16-step weight chunks nest), no larger than needed for `per` steps, with M rows of
// every wave fitting in the round buffer
__host__ __device__ inline int decode_round_steps(int M, int per) {
  int cap = 4;
  while (cap < per && cap < 64) cap <<= 1;
  int rs = cap;
  while (rs > 4 && 4 * M * rs * 64 > kDecodeRoundBytes) rs >>= 1;
  return rs;
}

template <int MT, int NT>
__global__ __launch_bounds__(256) void k_decode(DecodeArgs p) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int N = p.N, K = p.K;
  // this workgroup's rows: [row0, row0 + M)
  const int row0 = blockIdx.y * 16 * MT;
  const int M = min(p.M - row0, 16 * MT);
  p.a += (int64_t)row0 * p.lda;
  p.a_scale += row0;
  p.y += (int64_t)row0 * p.ldy;
  if (p.acc_out) p.acc_out += (int64_t)row0 * N;
  const int n0 = blockIdx.x * NT;
  const int cl = lane & 15, kg = lane >> 4;
  const int col = n0 + cl;
  const bool bvalid = (cl < NT) && (col < N);
  const int KST = (K + 63) >> 6;  // 64-deep steps over all K
  const int per = (KST + 3) >> 2; // steps per wave
  const int ks0 = min(KST, wv * per), ks1 = min(KST, ks0 + per);
  const int nsteps = ks1 - ks0;

  // LDS layout: [A staging rounds][s_lds 64][wsc_lds 16][red]
  int8_t* a_s = smem;
  float* s_lds = reinterpret_cast<float*>(smem + kDecodeRoundBytes);
  float* wsc_lds = s_lds + 64;
  int* red = reinterpret_cast<int*>(wsc_lds + 16);

  // ---- 1. every global load first --------------------------------------------------------
  v4i b[kDecodeChunk];
  const int8_t* wcol = p.w + (int64_t)col * K + 16 * kg;
#pragma unroll
  for (int j = 0; j < kDecodeChunk; ++j) {
    const int ks = ks0 + j;
    b[j] = (bvalid && ks < ks1 && ks * 64 + 16 * kg < K) ? *reinterpret_cast<const v4i*>(wcol + ks * 64)
                                                         : v4i{0, 0, 0, 0};
  }
  float wsc = 0.0f, asc = 0.0f;
  if (t < NT && n0 + t < N) wsc = p.w_scale[n0 + t];
  if (t < M) asc = p.a_scale[t];

  // ---- 2. activations --------------------------------------------------------------------
  const int rs = decode_round_steps(M, per);               // steps per staging round
  int8_t* my_a = a_s + wv * (kDecodeRoundBytes / 4);      // this wave's staging region
  auto stage_round = [&](int r0) {
    // rows [0, M) x steps [r0, r0 + rs) of this wave's quarter -> my_a, swizzled rows of rs*64 B
    const int rowb = rs * 64;    // a power of two (rs is)
    const int lg_rowb = __builtin_ctz(rowb);
    const int total = M * rowb;  // bytes
    const int chunks = rowb >> 4;
    const int g = min(16, chunks & -chunks);
    for (int off = 0; off < total; off += 1024) {
      const int o = off + lane * 16;
      const int m = o >> lg_rowb;
      const int pc = (o & (rowb - 1)) >> 4;   // position of this lane's chunk in the row
      const int c = pc ^ (m & (g - 1));       // the chunk that position holds (swz inverse)
      int k = (ks0 + r0) * 64 + c * 16;
      if (m >= M || k >= K) k = 0;            // in bounds; the bytes meet zero B or are unused
      const int mm = m < M ? m : 0;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(p.a + (int64_t)mm * p.lda + k),
                                       (lds_ptr_t)(my_a + off), 16, 0, 0);
    }
  };
  if (nsteps > 0) stage_round(0);
  if (t < M) s_lds[t] = asc;
  if (t < NT) wsc_lds[t] = wsc;

  // ---- 3. MFMA over this wave's K quarter -------------------------------------------------
  v4i acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = v4i{0, 0, 0, 0};

  // Rows >= M only feed accumulator rows the epilogue drops, so they read a valid row
  // (row M-1) instead of branching: the LDS reads and MFMAs then schedule freely.
  int arow[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) arow[mt] = min(mt * 16 + cl, M - 1);

  // MFMA over k-steps s_lo + j, j in [j0, j0 + cnt), weights b[j]; A chunk (s - b_lo)*4 + kg
  auto mfma_steps = [&](const int8_t* abase, int rowb, int s_lo, int j0, int cnt, int b_lo) {
    if (j0 == 0 && cnt == kDecodeChunk) {  // the common full chunk: no per-step branch
#pragma unroll
      for (int j = 0; j < kDecodeChunk; ++j) {
        const int s = s_lo + j;
        v4i af[MT];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
          af[mt] = *reinterpret_cast<const v4i*>(abase + swz(arow[mt], (s - b_lo) * 4 + kg, rowb));
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], b[j], acc[mt], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int j = 0; j < kDecodeChunk; ++j) {
        if (j >= j0 && j < j0 + cnt) {  // uniform
          const int s = s_lo + j;
          v4i af[MT];
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            af[mt] = *reinterpret_cast<const v4i*>(abase + swz(arow[mt], (s - b_lo) * 4 + kg, rowb));
#pragma unroll
          for (int mt = 0; mt < MT; ++mt)
            acc[mt] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[mt], b[j], acc[mt], 0, 0, 0);
        }
      }
    }
  };

  {
    // rounds of rs steps staged in this wave's region and weight chunks of 16 steps nest:
    // walk in pieces of min(rs, 16) steps
    const int piece = min(rs, kDecodeChunk);
    for (int s0 = 0; s0 < nsteps; s0 += piece) {
      const int cb = s0 - (s0 % kDecodeChunk);  // first step held in b[]
      const int r0 = s0 - (s0 % rs);            // first step of the staged round
      if (s0 == cb && s0 != 0) {
#pragma unroll
        for (int j = 0; j < kDecodeChunk; ++j) {
          const int ks = ks0 + cb + j;
          b[j] = (bvalid && ks < ks1 && ks * 64 + 16 * kg < K) ? *reinterpret_cast<const v4i*>(wcol + ks * 64)
                                                               : v4i{0, 0, 0, 0};
        }
      }
      if (s0 == r0) {
        if (s0 != 0) {
          asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // reads of the last round done
          stage_round(r0);
        }
        wait_vm_all();
      }
      const int s1 = min(nsteps, s0 + piece);
      mfma_steps(my_a, rs * 64, cb, s0 - cb, s1 - s0, r0);
    }
    __syncthreads();  // s_lds / wsc_lds written by other threads
  }

  // ---- 4. sum the four waves' tiles in LDS, then the epilogue -------------------------------
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[((wv * MT + mt) * 4 + i) * 64 + lane] = acc[mt][i];
  __syncthreads();
  for (int e = t; e < MT * 4 * 64; e += 256) {
    const int ln = e & 63, mi = e >> 6;  // mi = mt*4 + i
    const int mt = mi >> 2, i = mi & 3;
    const int row = mt * 16 + 4 * (ln >> 4) + i;
    const int c = ln & 15;
    const int n = n0 + c;
    if (row < M && c < NT && n < N) {
      const int v = red[(0 * MT * 4 + mi) * 64 + ln] + red[(1 * MT * 4 + mi) * 64 + ln] +
                    red[(2 * MT * 4 + mi) * 64 + ln] + red[(3 * MT * 4 + mi) * 64 + ln];
      p.y[(int64_t)row * p.ldy + n] = epi_bf16_d(v, s_lds[row], wsc_lds[c]);
      if (p.acc_out) p.acc_out[(int64_t)row * N + n] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------
// k_gemv: M <= 8.  Here even the MFMA's 16-row granularity is wasted, and the decode
// kernel's B layout (a load instruction spread over 16 weight rows) costs more than the
// arithmetic.  Instead a workgroup owns RW weight rows (output columns) and every thread
// one 16-byte K chunk per row: each load instruction of a wave reads 1 KiB of ONE row,
// contiguous.  v_dot4_i32_i8 does the products; the 256 per-thread partial sums of each
// (row, token) are reduced exactly through LDS.  The fused variant holds its 16 bf16
// inputs per token in registers, takes the per-token absmax over the workgroup and
// quantises them itself (same arithmetic as k_quant).
// ------------------------------------------------------------------------------------------
constexpr int kGemvRows = 4;   // weight rows per workgroup
constexpr int kGemvIters = 2;  // 16-byte K chunks per thread held at once (K <= 8192 in one pass)

__device__ __forceinline__ int dot16_i8(const v4i a, const v4i b, int acc) {
  acc = __builtin_amdgcn_sdot4(a[0], b[0], acc, false);
  acc = __builtin_amdgcn_sdot4(a[1], b[1], acc, false);
  acc = __builtin_amdgcn_sdot4(a[2], b[2], acc, false);
  return __builtin_amdgcn_sdot4(a[3], b[3], acc, false);
}

template <int MR, bool FUSED>
__global__ __launch_bounds__(256) void k_gemv(DecodeArgs p) {
  constexpr int RW = kGemvRows;
  constexpr int NO = RW * MR;  // outputs per workgroup
  __shared__ int part[NO][257];
  __shared__ float s_lds[MR], inv_lds[MR], wsc_lds[RW];
  __shared__ unsigned amax[MR];
  const int t = threadIdx.x, lane = t & 63;
  const int M = p.M, N = p.N, K = p.K;
  const int n0 = blockIdx.x * RW;
  const int C = K >> 4;  // 16-byte chunks per row
  if (t < MR) amax[t] = 0u;
  if (t < RW) wsc_lds[t] = (n0 + t < N) ? p.w_scale[n0 + t] : 0.0f;
  if (!FUSED && t < MR) s_lds[t] = (t < M) ? p.a_scale[t] : 0.0f;

  int acc[RW][MR];
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[r][m] = 0;

  for (int c0 = 0; c0 < C; c0 += 256 * kGemvIters) {
    // all loads of this pass first
    v4i wv[kGemvIters][RW];
#pragma unroll
    for (int i = 0; i < kGemvIters; ++i) {
      const int c = c0 + t + 256 * i;
#pragma unroll
      for (int r = 0; r < RW; ++r)
        wv[i][r] = (c < C && n0 + r < N) ? *reinterpret_cast<const v4i*>(p.w + (int64_t)(n0 + r) * K + c * 16)
                                         : v4i{0, 0, 0, 0};
    }
    v4i xq[kGemvIters][MR];
    if constexpr (FUSED) {
      uint4 xb[kGemvIters][MR][2];
#pragma unroll
      for (int i = 0; i < kGemvIters; ++i) {
        const int c = c0 + t + 256 * i;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          if (c < C && m < M) {
            const uint16_t* src = p.x + (int64_t)m * p.ldx + c * 16;
            xb[i][m][0] = *reinterpret_cast<const uint4*>(src);
            xb[i][m][1] = *reinterpret_cast<const uint4*>(src + 8);
          } else {
            xb[i][m][0] = uint4{0u, 0u, 0u, 0u};
            xb[i][m][1] = uint4{0u, 0u, 0u, 0u};
          }
        }
      }
      // per-token absmax over the workgroup (the host guarantees one pass covers all K)
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float a = 0.0f;
#pragma unroll
        for (int i = 0; i < kGemvIters; ++i) a = fmaxf(a, fmaxf(bf16x8_absmax(xb[i][m][0]), bf16x8_absmax(xb[i][m][1])));
        a = wave_max(a);
        if (lane == 0) atomicMax(&amax[m], __float_as_uint(a));
      }
      __syncthreads();
      if (t < MR) {
        const float s = __fdiv_rn(__uint_as_float(amax[t]), 127.0f);
        s_lds[t] = s;
        inv_lds[t] = __fdiv_rn(1.0f, s);
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kGemvIters; ++i) {
        const int c = c0 + t + 256 * i;
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          const uint2 lo = quant8_bf16(xb[i][m][0], s_lds[m], inv_lds[m]);
          const uint2 hi = quant8_bf16(xb[i][m][1], s_lds[m], inv_lds[m]);
          xq[i][m] = v4i{(int)lo.x, (int)lo.y, (int)hi.x, (int)hi.y};
          if (p.xq_out && blockIdx.x == 0 && c < C && m < M)
            *reinterpret_cast<v4i*>(p.xq_out + (int64_t)m * K + c * 16) = xq[i][m];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < kGemvIters; ++i) {
        const int c = c0 + t + 256 * i;
#pragma unroll
        for (int m = 0; m < MR; ++m)
          xq[i][m] = (c < C && m < M) ? *reinterpret_cast<const v4i*>(p.a + (int64_t)m * p.lda + c * 16)
                                      : v4i{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int i = 0; i < kGemvIters; ++i)
#pragma unroll
      for (int r = 0; r < RW; ++r)
#pragma unroll
        for (int m = 0; m < MR; ++m) acc[r][m] = dot16_i8(wv[i][r], xq[i][m], acc[r][m]);
  }

  // exact reduction of the 256 partials of each output through LDS
#pragma unroll
  for (int r = 0; r < RW; ++r)
#pragma unroll
    for (int m = 0; m < MR; ++m) part[r * MR + m][t] = acc[r][m];
  __syncthreads();
  constexpr int TPO = 256 / NO;  // threads per output (power of two)
  const int o = t / TPO, q = t % TPO;
  int v = 0;
  for (int j = q; j < 256; j += TPO) v += part[o][j];
#pragma unroll
  for (int off = TPO / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  if (q == 0) {
    const int r = o / MR, m = o % MR;
    const int n = n0 + r;
    if (m < M && n < N) {
      p.y[(int64_t)m * p.ldy + n] = epi_bf16_d(v, s_lds[m], wsc_lds[r]);
      if (p.acc_out) p.acc_out[(int64_t)m * N + n] = v;
    }
  }
  if (FUSED && p.xs_out && blockIdx.x == 0 && t < M) p.xs_out[t] = s_lds[t];
}

bool gemv_fits(int M, int K, bool fused) {
  if (M < 1 || M > 8) return false;
  return !fused || ((K >> 4) <= 256 * kGemvIters && M <= 4);
}

template <int MR>
static hipError_t gemv_mr(const DecodeArgs& a, bool fused, hipStream_t st) {
  dim3 grid((unsigned)((a.N + kGemvRows - 1) / kGemvRows)), block(256);
  if (fused)
    hipLaunchKernelGGL((k_gemv<MR, true>), grid, block, 0, st, a);
  else
    hipLaunchKernelGGL((k_gemv<MR, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

hipError_t launch_gemv(const DecodeArgs& a, hipStream_t st) {
  const bool fused = a.x != nullptr;
  if (!gemv_fits(a.M, a.K, fused)) return hipErrorInvalidValue;
  if (a.M <= 1) return gemv_mr<1>(a, fused, st);
  if (a.M <= 2) return gemv_mr<2>(a, fused, st);
  if (a.M <= 4) return gemv_mr<4>(a, fused, st);
  if (fused) return hipErrorInvalidValue;
  return gemv_mr<8>(a, false, st);
}

size_t decode_lds_bytes(int mt) { return (size_t)kDecodeRoundBytes + (64 + 16) * 4 + (size_t)4 * mt * 4 * 64 * 4; }

template <int MT, int NT>
static hipError_t decode_launch(const DecodeArgs& a, hipStream_t st) {
  const size_t lds = decode_lds_bytes(MT);
  auto kfn = k_decode<MT, NT>;
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kfn), 160 * 1024);
  if (e != hipSuccess) return e;
  dim3 grid((unsigned)((a.N + NT - 1) / NT), (unsigned)((a.M + 16 * MT - 1) / (16 * MT))), block(256);
  hipLaunchKernelGGL(kfn, grid, block, lds, st, a);
  return hipGetLastError();
}

template <int MT>
static hipError_t decode_mt(const DecodeArgs& a, int nt, hipStream_t st) {
  switch (nt) {
    case 4: return decode_launch<MT, 4>(a, st);
    case 8: return decode_launch<MT, 8>(a, st);
    case 16: return decode_launch<MT, 16>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs& a, int nt, int mt, hipStream_t st) {
  if (a.x != nullptr || a.M < 1 || a.M > 64) return hipErrorInvalidValue;
  switch (mt) {
    case 1: return decode_mt<1>(a, nt, st);
    case 2: return decode_mt<2>(a, nt, st);
    case 4: return decode_mt<4>(a, nt, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace wq
