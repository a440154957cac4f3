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
//    loads while the other is multiplied.  The next slice's eight DMA instructions per wave
//    are spread over the first half of the current slice's MFMAs (issued in one burst they
//    held every wave at the address unit for 1300-3000 cycles a slice); the slice sequence
//    runs across tile boundaries, so the next tile's first slice loads during the current
//    tile's last slice;
//  * tile order: workgroup b sits on XCD b % 8 (round robin dispatch); each XCD owns a
//    contiguous range of tiles.  When the tile grid allows, an XCD owns an N-range of W (an
//    eighth of the columns, for every row) walked in blocks of 4 tile rows x 8 tile columns,
//    so W is fetched from HBM once per call rather than once per XCD; otherwise it walks
//    groups of 4 tile rows over all columns;
//  * the MFMA takes the W fragment as its first operand, so each lane ends a tile with four
//    consecutive output columns of one row.  Epilogue: bf16((f32(acc) * s_m) * sw_n), four
//    values per 8-byte LDS write into the ring stage the last slice used (144-byte row pitch),
//    read back so that each nontemporal 16-byte-per-lane store writes eight whole 128-byte
//    rows of Y; the next tile's first slice waits only for its DMA, not for these stores.
// K must be a multiple of 128, N of 8; rows and columns past the edges read clamped rows and
// are not stored.

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
constexpr int kStgPitch = 144;             // epilogue staging: bytes per 128-byte row (bank spread)
constexpr int kStgWave = 32 * kStgPitch;   // staging bytes per wave: one 32-row block
static_assert(kBKb == 128 && kDmaPerWave == 4, "slice width: 4 K steps, 8 DMA instructions per wave");
static_assert(kStages == 2 && kStages * kStageB <= 160 * 1024, "LDS ring: one slice in flight");
static_assert(8 * kStgWave <= kStageB, "epilogue staging fits in one ring stage");

typedef __attribute__((address_space(3))) void* lds_ptr_b;
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Chunk swizzle: kRowsPerBankRow consecutive rows fill the 64 banks once, so the rows that
// land on the same banks (r, r + kRowsPerBankRow, ...) get different chunk positions; 16
// consecutive rows read at one logical chunk (a ds_read_b128 pass) then touch every bank once.
__device__ __forceinline__ int swz_of(int r) { return (r / kRowsPerBankRow) % kChunks; }
__device__ __forceinline__ int bswz(int r, int c) { return r * kBKb + ((c ^ swz_of(r)) << 4); }

struct BigTiles {
  int tiles_m, tiles_n, per_xcd, nt;
  int ncol;  // 0: row groups over all columns; else each XCD owns ncol tile columns (N-range order)
  __device__ void tile(int lin, int& tm, int& tn) const {
    if (ncol) {
      // XCD x = lin / per_xcd owns tile columns [x ncol, (x+1) ncol) for every tile row; it
      // walks them in blocks of 4 tile rows x 8 tile columns (one tile per CU of the XCD),
      // row blocks first, so each 8-column block of W stays in the XCD's L2 while the A rows
      // stream past it
      const int x = lin / per_xcd, idx = lin - x * per_xcd;
      const int per_cb = tiles_m * 8;  // tiles per 8-column block
      const int cb = idx / per_cb, in = idx - cb * per_cb;
      const int rb = in / 32, l = in - rb * 32;
      tm = rb * 4 + (l & 3);
      tn = x * ncol + cb * 8 + (l >> 2);
      return;
    }
    const int group = lin / (kGroupRows * tiles_n);
    const int gm0 = group * kGroupRows;
    const int gsz = min(kGroupRows, tiles_m - gm0);
    const int in = lin - group * kGroupRows * tiles_n;
    tm = gm0 + in % gsz;
    tn = in / gsz;
  }
};

// Per-lane byte offsets of one operand's DMA: instruction i (0..3) of wave wv fills LDS rows
// wv*32 + 8i + lane/8 with 16-byte chunks at position lane % 8, which hold the logical chunk
// (lane % 8) ^ swz_of(row).  swz_of(row) = (row / 2) % 8 = (4i + lane / 16) % 8, i.e.
// lane / 16 for even i and that plus 4 for odd i, so two offsets per lane (even and odd
// instructions) serve all four next to a wave-uniform row base.
__device__ __forceinline__ void dma_lane_offsets(int64_t ld, int lane, uint32_t off[2]) {
  const int c0 = (lane % kChunks) ^ (lane / 16);
  off[0] = (uint32_t)((lane / kChunks) * ld + c0 * 16);
  off[1] = (uint32_t)((lane / kChunks) * ld + (c0 ^ 4) * 16);
}

// One DMA instruction (i of 4) of a 256-row x 128-byte operand slice into `dst`: a
// wave-uniform base (row r0, byte k0) plus a 32-bit lane offset (ld < 2^23).  Edge slices
// clamp rows to < rows.
__device__ __forceinline__ void dma_one(const int8_t* src, int64_t ld, int r0, int rows, int k0, int8_t* dst, int wv,
                                        int lane, int i, bool interior, const uint32_t off[2]) {
  const int8_t* base = src + (int64_t)r0 * ld + k0;
  uint32_t o;
  if (interior) {
    o = (uint32_t)((wv * 32 + i * kRowsPerDma) * (int)ld) + off[i & 1];
  } else {
    const int rl = wv * 32 + i * kRowsPerDma + lane / kChunks;
    const int c = (lane % kChunks) ^ swz_of(rl);
    o = (uint32_t)(min(rl, rows - 1 - r0) * (int)ld + c * 16);
  }
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(base + o),
                                   (lds_ptr_b)(dst + (wv * kDmaPerWave + i) * 1024), 16, 0, 0);
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

__global__ __launch_bounds__(512, 1) void k_gemm_i8_big(TileArgs p, BigTiles bt, int wgs_per_xcd) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  // the row (0..255) and column (256..511) scales of two tiles, by tile parity
  __shared__ __attribute__((aligned(16))) float scl[2][512];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wv >> 2, wn = wv & 3;  // 2 x 4 waves of 128 x 64
  const int M = p.M, N = p.N, K = p.K;
  const int KT = K / kBKb;
  const int xcd = blockIdx.x & 7, local = blockIdx.x >> 3;
  const int lin0 = xcd * bt.per_xcd;
  const int lin_end = min(bt.nt, lin0 + bt.per_xcd);
  // this workgroup's tiles: lin0 + local, + wgs_per_xcd, ...
  const int my_tiles = lin0 + local < lin_end ? (lin_end - lin0 - local + wgs_per_xcd - 1) / wgs_per_xcd : 0;
  if (my_tiles == 0) return;

  uint32_t aoff[2], boff[2];
  dma_lane_offsets(p.lda, lane, aoff);
  dma_lane_offsets(K, lane, boff);
  auto tile_at = [&](int ti, int& m0, int& n0) {
    int tm, tn;
    bt.tile(lin0 + local + ti * wgs_per_xcd, tm, tn);
    m0 = tm * kBT;
    n0 = tn * kBT;
  };
  // DMA instruction d (0..7: A 0-3, B 4-7) of the slice at (ma, nb, k0) into stage st
  auto dma = [&](int d, int ma, int nb, int k0, int8_t* st) {
    if (d < kDmaPerWave)
      dma_one(p.a, p.lda, ma, M, k0, st, wv, lane, d, ma + kBT <= M, aoff);
    else
      dma_one(p.w, K, nb, N, k0, st + kSliceB, wv, lane, d - kDmaPerWave, nb + kBT <= N, boff);
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
  int m0, n0, nm0 = 0, nn0 = 0;
  tile_at(0, m0, n0);
  if (my_tiles > 1) tile_at(1, nm0, nn0);
#pragma unroll
  for (int d = 0; d < 2 * kDmaPerWave; ++d) dma(d, m0, n0, 0, smem);
  // Each thread fetches one of the current tile's 512 scales with its first slice and
  // stores it to LDS one slice later, after the slice wait has covered it, so the epilogue
  // reads no global memory.
  float scale_v = 0.0f;
  bool stores_pending = false;  // the previous tile's 16 output stores per wave may be in flight
  for (int ti = 0; ti < my_tiles; ++ti) {
    const int par = ti & 1;
    for (int kt = 0; kt < KT; ++kt) {
      const int s = ti * KT + kt;
      // This wave's DMA of slice s (and any scale load) has landed.  VMEM operations retire
      // in issue order, and the previous tile's output stores were issued after this slice's
      // DMA, so those 16 may stay in flight.  The barrier makes every wave's slice visible and
      // frees the stage of slice s-1 for slice s+1.
      if (stores_pending)
        asm volatile("s_waitcnt vmcnt(16)" ::: "memory");
      else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      stores_pending = false;
      lds_barrier();
      if (kt == 1) scl[par][t] = scale_v;  // loaded with slice s - 1, now waited for
      if (kt == 0) scale_v = t < 256 ? p.a_scale[min(m0 + t, M - 1)] : p.w_scale[min(n0 + t - 256, N - 1)];
      // the next slice: the same tile's next K slice, else the next tile's first
      const bool has_next = kt + 1 < KT || ti + 1 < my_tiles;
      const int xa = kt + 1 < KT ? m0 : nm0, xb = kt + 1 < KT ? n0 : nn0;
      const int xk = kt + 1 < KT ? (kt + 1) * kBKb : 0;
      int8_t* xst = smem + ((s + 1) % kStages) * kStageB;
      const int8_t* sa = smem + (s % kStages) * kStageB;
      const int8_t* sb = sa + kSliceB;
      // Operand fragments double-buffered in registers.  With LDS-DMA loads in flight the
      // compiler waits for every outstanding LDS read at once, so the reads of step ks+1 are
      // issued after the first MFMA of step ks: the wait in front of step ks+1 then covers
      // reads issued seven MFMAs earlier.  The next slice's eight DMA instructions go out one
      // per two MFMAs in the first half of the slice: the MFMA pipe keeps running while the
      // address unit accepts them, and they have the second half to land.
      // The MFMA takes the W fragment as its first operand: each lane then holds four
      // consecutive output columns of one row (register 4q + r: column 8q + 4(lane/32) + r
      // of the 32-column block, row lane % 32).
      v4i af[2][4], bf[2][2];
      auto read_frags = [&](int ks, v4i* a4, v4i* b2) {
#pragma unroll
        for (int i = 0; i < 4; ++i) a4[i] = *reinterpret_cast<const v4i*>(sa + bswz(ar + i * 32, 2 * ks + kh));
#pragma unroll
        for (int j = 0; j < 2; ++j) b2[j] = *reinterpret_cast<const v4i*>(sb + bswz(br + j * 32, 2 * ks + kh));
      };
      read_frags(0, af[0], bf[0]);
#pragma unroll
      for (int ks = 0; ks < kBKb / 32; ++ks) {
        const int cb = ks & 1, nb = cb ^ 1;
        acc[0][0] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[cb][0], af[cb][0], acc[0][0], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if (ks < kBKb / 32 - 1) read_frags(ks + 1, af[nb], bf[nb]);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int q = 1; q < 8; ++q) {
          const int i = q >> 1, j = q & 1;
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bf[cb][j], af[cb][i], acc[i][j], 0, 0, 0);
          if (ks < 2 && (q & 1)) {
            __builtin_amdgcn_sched_barrier(0);
            if (has_next) dma(4 * ks + (q >> 1), xa, xb, xk, xst);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      if (kt == KT - 1) {
        // ---- epilogue of this tile: bf16((f32(acc) * s_m) * sw_n) ----
        if (KT == 1) scl[par][t] = scale_v;
        // every wave is done with this slice's ring stage (and, for KT <= 2, the scales are
        // in LDS): the stage becomes the staging area of the output, 8 KiB per wave
        lds_barrier();
        const float* sc = scl[par];
        int8_t* stg = smem + (s % kStages) * kStageB + wv * kStgWave;
        const bool interior = m0 + kBT <= M && n0 + kBT <= N;
        // Four rounds, one per 32-row block: each lane converts its four consecutive columns
        // to bf16 and writes them as 8 bytes to its row of the staging area (144-byte pitch,
        // so the 32 rows of one write instruction fall on different banks); reading back,
        // eight lanes take one row, and each store instruction writes eight whole 128-byte
        // rows of Y.  Staging offsets and the store's lane offset are per-lane constants.
        int8_t* wr = stg + (lane & 31) * kStgPitch + kh * 8;
        const int8_t* rd = stg + (lane / 8) * kStgPitch + (lane % 8) * 16;
        const uint32_t yoff = (uint32_t)((lane / 8) * p.ldy * 2 + (lane % 8) * 16);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float rs = sc[wm * 128 + i * 32 + (lane & 31)];
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            float4 cs[4];  // column scales of this lane's 4 x 4 columns of the 32-column block
#pragma unroll
            for (int q = 0; q < 4; ++q)
              cs[q] = *reinterpret_cast<const float4*>(sc + 256 + wn * 64 + j * 32 + 8 * q + 4 * kh);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const v16i& a = acc[i][j];
              const float f0 = __fmul_rn(__fmul_rn((float)a[4 * q + 0], rs), cs[q].x);
              const float f1 = __fmul_rn(__fmul_rn((float)a[4 * q + 1], rs), cs[q].y);
              const float f2 = __fmul_rn(__fmul_rn((float)a[4 * q + 2], rs), cs[q].z);
              const float f3 = __fmul_rn(__fmul_rn((float)a[4 * q + 3], rs), cs[q].w);
              // two f32 -> one word of two bf16, round to nearest even (v_cvt_pk_bf16_f32)
              const v2u w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f0, f1}, bf16x2)),
                             __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f2, f3}, bf16x2))};
              *reinterpret_cast<v2u*>(wr + j * 64 + q * 16) = w;
            }
          }
          v4i rows[4];
#pragma unroll
          for (int k = 0; k < 4; ++k) rows[k] = *reinterpret_cast<const v4i*>(rd + k * 8 * kStgPitch);
          __builtin_amdgcn_sched_barrier(0);  // the four reads in flight before the first store
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            const int mr = m0 + wm * 128 + i * 32 + k * 8;  // first of the 8 rows of this store
            int8_t* yb = reinterpret_cast<int8_t*>(p.y) + ((int64_t)mr * p.ldy + n0 + wn * 64) * 2;  // wave-uniform
            // streaming store: the output is not read again here, and keeping it out of the
            // L2's reuse set leaves room for the A and B tiles.  N % 8 == 0: a lane's eight
            // columns are in or out together
            if (interior || (mr + lane / 8 < M && n0 + wn * 64 + (lane % 8) * 8 < N))
              __builtin_nontemporal_store(rows[k], reinterpret_cast<v4i*>(yb + yoff));
          }
        }
        if (p.acc_out) {  // raw accumulators (a parity hook): four consecutive columns per store
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 2; ++j)
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const int m = m0 + wm * 128 + i * 32 + (lane & 31);
                const int n = n0 + wn * 64 + j * 32 + 8 * q + 4 * kh;
                if (m < M && n < N)
                  *reinterpret_cast<v4i*>(p.acc_out + (int64_t)m * N + n) =
                      v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
              }
        }
        stores_pending = interior && !p.acc_out && ti + 1 < my_tiles;  // 16 stores per wave
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0;
        m0 = nm0;
        n0 = nn0;
        if (ti + 2 < my_tiles) tile_at(ti + 2, nm0, nn0);
      }
    }
  }
}

// Eight consecutive bf16 columns per store: y 16-byte aligned, N and ldy multiples of 8;
// acc_out (when given) 16-byte aligned; 32-bit DMA lane offsets: lda, K < 2^23.
bool big_fits(int M, int N, int K, int64_t lda, int64_t ldy, const void* y, const void* acc_out) {
  return K % kBKb == 0 && M >= kBT && N >= kBT && N % 8 == 0 && ldy % 8 == 0 && lda % 16 == 0 && lda < (1 << 23) &&
         K < (1 << 23) && reinterpret_cast<uintptr_t>(y) % 16 == 0 && reinterpret_cast<uintptr_t>(acc_out) % 16 == 0;
}

hipError_t launch_gemm_i8_big(const TileArgs& a, int num_cu, hipStream_t st) {
  if (!big_fits(a.M, a.N, a.K, a.lda, a.ldy, a.y, a.acc_out)) return hipErrorInvalidValue;
  BigTiles bt;
  bt.tiles_m = (a.M + kBT - 1) / kBT;
  bt.tiles_n = (a.N + kBT - 1) / kBT;
  bt.nt = bt.tiles_m * bt.tiles_n;
  bt.per_xcd = (bt.nt + 7) / 8;
  // N-range order when the grid splits evenly: per_xcd = tiles_m * tiles_n / 8 exactly
  bt.ncol = bt.tiles_n % 64 == 0 && bt.tiles_m % 4 == 0 ? bt.tiles_n / 8 : 0;
  const int wgs_per_xcd = num_cu / 8;
  const size_t lds = kStages * (size_t)kStageB;
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(k_gemm_i8_big), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_gemm_i8_big, dim3((unsigned)(wgs_per_xcd * 8)), dim3(512), lds, st, a, bt, wgs_per_xcd);
  return hipGetLastError();
}

}  // namespace wq
