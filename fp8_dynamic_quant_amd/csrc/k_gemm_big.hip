// Large-M INT8 W8A8 GEMM (prefill): persistent 256 x 256 tiles.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (quant matmul: INT8 X and per-token
// scale times pre-quantised per-channel-scaled weights, BF16 Y), at prefill M where the
// MFMA units, not HBM, bound the run (e.g. M = 8192, K = 1024, N = 32768: 550 Gop, 587 MB).
//
// Shape of the kernel (MI355X):
//  * one workgroup per CU, persistent: 512 threads = 8 waves in a 2 x 4 grid, each wave a
//    128 x 64 block of the 256 x 256 tile as 4 x 2 v_mfma_i32_32x32x32_i8 tiles (128 int32
//    accumulators per lane).  The 256 x 256 tile halves the L2 traffic per MAC of a 128 x 128
//    tile; two waves per SIMD hide each other's LDS latency;
//  * operands move global -> LDS with global_load_lds_dwordx4 in 128-byte K slices through
//    two 64 KiB stages (A 256 x 128 and B 256 x 128 bytes, XOR-swizzled chunks): one slice
//    loads while the other is multiplied.  The slice sequence runs across tile boundaries:
//    the next tile's first slice loads during the current tile's last slice and epilogue;
//  * tile order: workgroup b sits on XCD b % 8 (round robin dispatch); each XCD owns a
//    contiguous range of tiles, walked in groups of 4 tile rows so the A rows and B columns
//    its 32 CUs work on at the same time stay in that XCD's 4 MB L2;
//  * epilogue straight from the accumulators: bf16((f32(acc) * s_m) * sw_n); neighbouring
//    lanes swap one value so each lane stores two adjacent columns as one 32-bit word, with
//    nontemporal stores.
// K must be a multiple of 128; rows and columns past the edges read clamped rows and are
// not stored.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

constexpr int kBT = 256;                   // tile edge
constexpr int kBKb = 128;                  // K bytes per slice
constexpr int kStages = 2;                 // LDS ring depth: kStages - 1 slices in flight
constexpr int kSliceB = kBT * kBKb;        // bytes per operand per slice
constexpr int kStageB = 2 * kSliceB;       // A + B
constexpr int kChunks = kBKb / 16;         // 16-byte chunks per row
constexpr int kRowsPerBankRow = 256 / kBKb;  // rows sharing one sweep of the 64 4-byte banks
constexpr int kRowsPerDma = 1024 / kBKb;   // rows one 64-lane x 16-byte DMA instruction covers
constexpr int kDmaPerWave = kBT / 8 / kRowsPerDma;  // DMA instructions per operand per wave
constexpr int kGroupRows = 4;              // tile rows per group in the tile order
static_assert(kBKb == 64 || kBKb == 128, "slice width");
static_assert(kStages >= 2 && kStages <= 4 && kStages * kStageB <= 160 * 1024, "LDS ring");

typedef __attribute__((address_space(3))) void* lds_ptr_b;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Chunk swizzle: kRowsPerBankRow consecutive rows fill the 64 banks once, so the rows that
// land on the same banks (r, r + kRowsPerBankRow, ...) get different chunk positions; 16
// consecutive rows read at one logical chunk (a ds_read_b128 pass) then touch every bank once.
__device__ __forceinline__ int swz_of(int r) { return (r / kRowsPerBankRow) % kChunks; }
__device__ __forceinline__ int bswz(int r, int c) { return r * kBKb + ((c ^ swz_of(r)) << 4); }

// DMA a 256-row x kBKb-byte slice (rows clamped to < rows) into `dst`, swizzled; 8 waves,
// kDmaPerWave instructions each.  Instruction i of wave wv fills LDS rows
// wv*32 + i*kRowsPerDma + l/kChunks (lane l writes dst + 16 l), so lane l fetches the
// logical chunk whose swizzled position is l % kChunks.
__device__ __forceinline__ void dma256(const int8_t* src, int64_t ld, int r0, int rows, int k0, int8_t* dst, int wv,
                                       int lane) {
  const bool interior = r0 + kBT <= rows;
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int rl = wv * 32 + i * kRowsPerDma + lane / kChunks;
    const int c = (lane % kChunks) ^ swz_of(rl);
    const int gr = interior ? r0 + rl : min(r0 + rl, rows - 1);
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + (int64_t)gr * ld + k0 + c * 16),
                                     (lds_ptr_b)(dst + (wv * kDmaPerWave + i) * 1024), 16, 0, 0);
  }
}

// s_waitcnt needs an immediate: n later slices of 2 * kDmaPerWave loads each
__device__ __forceinline__ void wait_vm_slices(int n) {
  static_assert(2 * kDmaPerWave * 2 <= 63, "vmcnt range");
  if (n <= 0) {
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  } else if (n == 1) {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * kDmaPerWave) : "memory");
  } else {
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * kDmaPerWave) : "memory");
  }
}

__device__ __forceinline__ void sc_store_now(float* dst, int t, float v) { dst[t] = v; }

struct BigTiles {
  int tiles_m, tiles_n, per_xcd, nt;
  __device__ void tile(int lin, int& tm, int& tn) const {
    const int group = lin / (kGroupRows * tiles_n);
    const int gm0 = group * kGroupRows;
    const int gsz = min(kGroupRows, tiles_m - gm0);
    const int in = lin - group * kGroupRows * tiles_n;
    tm = gm0 + in % gsz;
    tn = in / gsz;
  }
};

__global__ __launch_bounds__(512, 1) void k_gemm_i8_big(TileArgs p, BigTiles bt, int wgs_per_xcd) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  // the row (0..255) and column (256..511) scales of two tiles, by tile parity
  __shared__ __attribute__((aligned(16))) float scl[2][512];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 2, wn = wv & 3;  // 2 x 4 waves of 128 x 64
  const int M = p.M, N = p.N, K = p.K;
  const int KT = K / kBKb;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int lin0 = xcd * bt.per_xcd;
  const int lin_end = min(bt.nt, lin0 + bt.per_xcd);
  // this workgroup's tiles: lin0 + local, + wgs_per_xcd, ...
  const int my_tiles = lin0 + local < lin_end ? (lin_end - lin0 - local + wgs_per_xcd - 1) / wgs_per_xcd : 0;
  const int total = my_tiles * KT;  // slices
  if (total == 0) return;

  auto tile_of = [&](int s, int& m0, int& n0) {
    int tm, tn;
    bt.tile(lin0 + local + (s / KT) * wgs_per_xcd, tm, tn);
    m0 = tm * kBT;
    n0 = tn * kBT;
  };
  auto issue = [&](int s) {
    int m0, n0;
    tile_of(s, m0, n0);
    const int k0 = (s % KT) * kBKb;
    int8_t* st = smem + (s % kStages) * kStageB;
    dma256(p.a, p.lda, m0, M, k0, st, wv, lane);
    dma256(p.w, K, n0, N, k0, st + kSliceB, wv, lane);
  };

  v16i acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;

  const int ar = wm * 128 + (lane & 31), br = wn * 64 + (lane & 31);
  const int kh = lane >> 5;
  // Each thread fetches one of the current tile's 512 scales with its first slice and
  // stores it to LDS one slice later, after the slice wait has covered it, so the epilogue
  // reads no global memory: a scale load there waited for the stores issued before it.
  float scale_v = 0.0f;
  auto load_scale = [&](int s) {
    int m0, n0;
    tile_of(s, m0, n0);
    scale_v = t < 256 ? p.a_scale[min(m0 + t, M - 1)] : p.w_scale[min(n0 + t - 256, N - 1)];
  };
  for (int s = 0; s < kStages - 1 && s < total; ++s) issue(s);
  for (int s = 0; s < total; ++s) {
    // wait for this wave's DMA of slice s while the later slices already issued (up to
    // kStages - 2 of them, 2 * kDmaPerWave instructions each) stay in flight.  Loads
    // complete in order among themselves, so "at most n operations outstanding" with n the
    // later slices' instruction count means slice s has landed, whatever epilogue stores
    // are also counted.
    {
      const int later = min(kStages - 2, total - 1 - s);
      wait_vm_slices(later);
    }
    lds_barrier();  // slice s is in LDS everywhere; the stage of slice s-1 is free
    if (KT > 1 && s % KT == 1) scl[(s / KT) & 1][t] = scale_v;  // loaded with slice s - 1, now waited for
    if (s % KT == 0) load_scale(s);
    if (s + kStages - 1 < total) issue(s + kStages - 1);
    const int8_t* sa = smem + (s % kStages) * kStageB;
    const int8_t* sb = sa + kSliceB;
    // operand fragments double-buffered in registers: step ks+1 is read from LDS while the
    // 16 MFMAs of step ks issue (the barriers keep the compiler from hoisting every read)
    v4i af[2][4], bf[2][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) af[0][i] = *reinterpret_cast<const v4i*>(sa + bswz(ar + i * 32, kh));
#pragma unroll
    for (int j = 0; j < 2; ++j) bf[0][j] = *reinterpret_cast<const v4i*>(sb + bswz(br + j * 32, kh));
#pragma unroll
    for (int ks = 0; ks < kBKb / 32; ++ks) {
      const int cb = ks & 1, nb = cb ^ 1;
      if (ks < kBKb / 32 - 1) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
          af[nb][i] = *reinterpret_cast<const v4i*>(sa + bswz(ar + i * 32, 2 * (ks + 1) + kh));
#pragma unroll
        for (int j = 0; j < 2; ++j)
          bf[nb][j] = *reinterpret_cast<const v4i*>(sb + bswz(br + j * 32, 2 * (ks + 1) + kh));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(af[cb][i], bf[cb][j], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if ((s % KT) == KT - 1) {
      // ---- epilogue of this tile ----
      int m0, n0;
      tile_of(s, m0, n0);
      const bool odd = lane & 1;
      const float* sc = scl[(s / KT) & 1];
      if (KT <= 2) {  // the scales were stored in this iteration (KT = 2) or are still in registers
        if (KT == 1) sc_store_now(scl[(s / KT) & 1], t, scale_v);
        __syncthreads();
      }
      float swv[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) swv[j] = sc[256 + wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int mrow = m0 + wm * 128 + i * 32 + 4 * kh;
        // row scales of the 16 rows this lane holds in the i-th 32-row block: rows
        // mrow + 8q + 0..3, four consecutive floats per q
        float rs[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float4 r4 = *reinterpret_cast<const float4*>(sc + (mrow - m0) + 8 * q);
          rs[4 * q] = r4.x;
          rs[4 * q + 1] = r4.y;
          rs[4 * q + 2] = r4.z;
          rs[4 * q + 3] = r4.w;
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          __builtin_amdgcn_sched_barrier(0);  // one 32 x 32 block at a time: bounded live registers
          const int n = n0 + wn * 64 + j * 32 + (lane & 31);
          const float sw = swv[j];
          const int nbase = n - (odd ? 1 : 0);  // the even column of the pair
          // this lane's first output row (r0 for even lanes, r0 + 1 for odd) and its stride
          // of two rows: the 8 stores below are at fixed multiples of the stride
          uint16_t* rowp = reinterpret_cast<uint16_t*>(p.y) + (int64_t)(mrow + (odd ? 1 : 0)) * p.ldy + nbase;
          const int64_t ld2 = 2 * p.ldy;
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            // registers e = 4q + 0..3 hold rows mrow + 8q + 0..3 of column n
#pragma unroll
            for (int hp = 0; hp < 2; ++hp) {
              const int e0 = 4 * q + 2 * hp;  // rows r0 = mrow + 8q + 2hp and r1 = r0 + 1
              const int r0 = mrow + 8 * q + 2 * hp;
              const float s0 = rs[e0];
              const float s1 = rs[e0 + 1];
              const float f0 = __fmul_rn(__fmul_rn((float)acc[i][j][e0], s0), sw);
              const float f1 = __fmul_rn(__fmul_rn((float)acc[i][j][e0 + 1], s1), sw);
              // even lane keeps row r0 and takes its neighbour's (r0, n+1); odd lane keeps
              // row r1 and takes its neighbour's (r1, n-1): a quad-permute DPP move swaps
              // lanes 2k and 2k+1 without the LDS crossbar
              const float give = odd ? f0 : f1;
              const float got = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(give), 0xB1, 0xF, 0xF, false));
              // two f32 -> one word of two bf16, round to nearest even (v_cvt_pk_bf16_f32)
              const f32x2 pair = odd ? f32x2{got, f1} : f32x2{f0, got};
              const uint32_t word = __builtin_bit_cast(uint32_t, __builtin_convertvector(pair, bf16x2));
              const int row = odd ? r0 + 1 : r0;
              if (row < M && nbase < N) {
                uint16_t* dst = rowp + (4 * q + hp) * ld2;
                // streaming store: the output is not read again here, and keeping it out of
                // the L2's reuse set leaves room for the A and B tiles (measured ~15% faster)
                __builtin_nontemporal_store(word, reinterpret_cast<uint32_t*>(dst));  // N even: nbase + 1 < N
              }
              if (p.acc_out) {  // raw accumulators, same pairing
                const int a0 = acc[i][j][e0], a1 = acc[i][j][e0 + 1];
                const int ag = __builtin_amdgcn_mov_dpp(odd ? a0 : a1, 0xB1, 0xF, 0xF, false);
                if (row < M && nbase < N) {
                  int2 pr = odd ? int2{ag, a1} : int2{a0, ag};
                  *reinterpret_cast<int2*>(p.acc_out + (int64_t)row * N + nbase) = pr;
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
    }
  }
}

bool big_fits(int M, int N, int K, int64_t lda, int64_t ldy) {
  return K % kBKb == 0 && M >= kBT && N >= kBT && N % 2 == 0 && ldy % 2 == 0 && lda % 16 == 0;
}

hipError_t launch_gemm_i8_big(const TileArgs& a, int num_cu, hipStream_t st) {
  if (!big_fits(a.M, a.N, a.K, a.lda, a.ldy)) return hipErrorInvalidValue;
  BigTiles bt;
  bt.tiles_m = (a.M + kBT - 1) / kBT;
  bt.tiles_n = (a.N + kBT - 1) / kBT;
  bt.nt = bt.tiles_m * bt.tiles_n;
  bt.per_xcd = (bt.nt + 7) / 8;
  const int wgs_per_xcd = num_cu / 8;
  const size_t lds = kStages * (size_t)kStageB;
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(k_gemm_i8_big), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gemm_i8_big, dim3((unsigned)(wgs_per_xcd * 8)), dim3(512), lds, st, a, bt, wgs_per_xcd);
  return hipGetLastError();
}

}  // namespace wq
