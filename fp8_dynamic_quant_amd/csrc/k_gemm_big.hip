// Large-M INT8 W8A8 GEMM (prefill): persistent 256 x 256 tiles.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (quant matmul: INT8 X and per-token
// scale times pre-quantised per-channel-scaled weights, BF16 Y), at prefill M where the
// MFMA units, not HBM, bound the run (e.g. M = 8192, K = 1024, N = 32768: 550 Gop, 587 MB).
//
// Shape of the kernel (MI355X):
//  * one workgroup per CU, persistent: 512 threads = 8 waves in a 2 x 4 grid, each wave 128
//    rows by two 32-column blocks of the 256 x 256 tile as 4 x 2 v_mfma_i32_32x32x32_i8 tiles
//    (128 int32 accumulators per lane).  The 256 x 256 tile halves the L2 traffic per MAC of
//    a 128 x 128 tile; two waves per SIMD hide each other's LDS latency;
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
//    consecutive output columns of one row.  Epilogue: bf16((f32(acc) * s_m) * sw_n), carried
//    into the next tile's first K slice, which runs block by block: each 32 x 32 block's
//    accumulators are converted during the previous block's MFMAs, staged through a private
//    LDS area (four values per 8-byte write) and read back so that each 16-byte-per-lane
//    store writes 16 rows of 64 bytes; the conversion, staging and stores run beside the MFMA
//    pipe.  The last tile's epilogue runs on its own.  Output stores are nontemporal in the
//    N-range order and cached otherwise;
//  * M, N >= 256; the last tile row and column are shifted back to end at M and N, so every
//    DMA and store is inside the operands.
// K must be a multiple of 128, N of 8.

#include <type_traits>

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
constexpr int kStgWave = 32 * 64;          // epilogue staging per wave: one 32 x 32 block of bf16
static_assert(kBKb == 128 && kDmaPerWave == 4, "slice width: 4 K steps, 8 DMA instructions per wave");
static_assert(kStages == 2 && kStages * kStageB <= 160 * 1024, "LDS ring: one slice in flight");
static_assert(kStages * kStageB + 8 * kStgWave + 2 * 512 * 4 <= 160 * 1024, "ring, output staging and scales fit in LDS");

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

// Raw buffer resource over `base` (no stride, no format conversion; word 3 as CDNA3/4 raw
// buffers take it).  Buffer instructions take a scalar base and soffset plus a 32-bit lane
// offset, so no 64-bit lane address is formed in the loop.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t raw_rsrc(const void* base) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, 0x7FFFFFFF, kRsrcWord3);
}

// One DMA instruction (i of 4) of a 256-row x 128-byte operand slice into `dst`: a
// wave-uniform base (row r0 + this instruction's first row, byte k0) in scalar registers plus
// a 32-bit lane offset (ld < 2^23).  Every tile lies inside the operands (the last tile row
// and column are shifted back to end at M and N), so no row is clamped.
//
// The instruction is written out (global_load_lds_dwordx4 with its LDS address in M0): given
// the builtin, the compiler makes every later LDS read whose address it cannot separate from
// the DMA's target wait for all DMAs in flight (vmcnt(0) in the middle of the slice).  Here the
// kernel orders them itself: each slice waits for its own DMA (vmcnt) and a barrier before
// reading the stage, and nothing else reads a stage a DMA is filling.  The instruction has no
// register result.  The compiler cannot see the hazards inside the statement, so it keeps its
// own wait states: six between the statement's start and the load (a VALU write of an SGPR
// the load reads, e.g. a readfirstlane just ahead, needs five; the M0 write needs one).
__device__ __forceinline__ void dma_one(const int8_t* src, int64_t ld, int r0, int k0, int8_t* dst, int wv, int i,
                                        const uint32_t off[2]) {
  const int8_t* base = src + (int64_t)(r0 + wv * 32 + i * kRowsPerDma) * ld + k0;
  const uint32_t o = off[i & 1];
  const uint32_t la = (uint32_t)(uintptr_t)(lds_ptr_b)(dst + (wv * kDmaPerWave + i) * 1024);
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(o), "s"(base), "s"(la)
               : "memory", "m0");
#pragma clang diagnostic pop
}

typedef unsigned v2u __attribute__((ext_vector_type(2)));

// ACC: the raw accumulators are exported too (a parity hook; its own instantiation keeps the
// export's registers out of the production kernel).  NT: the output stores are nontemporal.
template <bool ACC, bool NT>
__global__ __launch_bounds__(512, 1) void k_gemm_i8_big(TileArgs p, BigTiles bt, int wgs_per_xcd) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  // the row (0..255) and column (256..511) scales of two tiles, by tile parity
  __shared__ __attribute__((aligned(16))) float scl[2][512];
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wv >> 2, wn = wv & 3;  // 2 x 4 waves of 128 rows x two 32-column blocks
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
  // tile origins; the last tile row and column end at M and N (M, N >= 256), so their first
  // rows or columns are also another tile's: computed twice and stored twice, with the same
  // bytes
  auto tile_at = [&](int ti, int& m0, int& n0) __attribute__((always_inline)) {
    int tm, tn;
    bt.tile(lin0 + local + ti * wgs_per_xcd, tm, tn);
    m0 = min(tm * kBT, M - kBT);
    n0 = min(tn * kBT, N - kBT);
  };
  // DMA instruction d (0..7: A 0-3, B 4-7) of the slice at (ma, nb, k0) into stage st
  auto dma = [&](int d, int ma, int nb, int k0, int8_t* st) __attribute__((always_inline)) {
    // wave-uniform operands (scalar registers: a scalar base plus the 32-bit lane offset)
    ma = __builtin_amdgcn_readfirstlane(ma);
    nb = __builtin_amdgcn_readfirstlane(nb);
    k0 = __builtin_amdgcn_readfirstlane(k0);
    if (d < kDmaPerWave)
      dma_one(p.a, p.lda, ma, k0, st, wv, d, aoff);
    else
      dma_one(p.w, K, nb, k0, st + kSliceB, wv, d - kDmaPerWave, boff);
  };

  v16i acc[4][2];  // set by each tile's first K step (an MFMA with a zero accumulator)
  const v16i zero16 = {};

  // Wave (wm, wn) computes rows wm*128 + [0, 128) and two 32-column blocks j = 0, 1 at tile
  // column col0(j).  With cached output stores they are j*128 + wn*32: the four waves of a
  // row half cover 128 consecutive columns with each block, so the two 64-byte halves of a
  // line are stored by two waves at about the same point and meet in the L2.  With
  // nontemporal stores (written back early, so halves from two waves often reach memory
  // apart) they are wn*64 + j*32: one wave stores both halves of its lines.
  auto col0 = [&](int j) __attribute__((always_inline)) { return NT ? wn * 64 + j * 32 : j * 128 + wn * 32; };
  const int ar = wm * 128 + (lane & 31);
  auto brow = [&](int j) __attribute__((always_inline)) { return col0(j) + (lane & 31); };  // W row of block j
  const int kh = lane >> 5;
  // This wave's output staging: one 32 x 32 block, row r (64 bytes) at 64 r, its 16-byte
  // chunk c at position c ^ ((r / 4) % 4) and, for r >= 16, the two 8-byte halves of each
  // chunk swapped.  Then the 32 lanes of a half-wave writing 8 bytes each (rows 0..31, one
  // half of one chunk) cover the 64 banks once, and the 16 lanes of a quarter-wave reading
  // 16 bytes each (four rows, four chunks) do too.
  int8_t* const stg = smem + kStages * kStageB + wv * kStgWave;
  const int sr = lane & 31, sw = (sr >> 2) & 3;
  int8_t* const stg_wr = stg + sr * 64 + 8 * (kh ^ (sr >> 4));
  const int8_t* const stg_rd = stg + (lane / 4) * 64 + 16 * ((lane % 4) ^ ((lane >> 4) & 3));
  const uint32_t yoff = (uint32_t)((lane / 4) * p.ldy * 2 + (lane % 4) * 16);
  int m0, n0, nm0 = 0, nn0 = 0, om0 = 0, on0 = 0;
  tile_at(0, m0, n0);
  if (my_tiles > 1) tile_at(1, nm0, nn0);
#pragma unroll
  for (int d = 0; d < 2 * kDmaPerWave; ++d) dma(d, m0, n0, 0, smem);

  // ---- epilogue pieces for the finished tile at (om0, on0): bf16((f32(acc) * s_m) * sw_n) ----
  // A lane holds, for block (i, j), row i*32 + lane % 32 of the wave's 128 rows and tile
  // columns j*128 + wn*32 + 8q + 4(lane/32) + r (register 4q + r).  Four values become two
  // words of two bf16 each (round to nearest even, v_cvt_pk_bf16_f32).
  auto col_scales = [&](const float* sc, int j, int q) __attribute__((always_inline)) {
    return *reinterpret_cast<const float4*>(sc + 256 + col0(j) + 8 * q + 4 * kh);
  };
  auto conv = [&](const float4 cs, int i, int j, int q, float rs, v2u& w) __attribute__((always_inline)) {
    const v16i& a = acc[i][j];
    const float f0 = __fmul_rn(__fmul_rn((float)a[4 * q + 0], rs), cs.x);
    const float f1 = __fmul_rn(__fmul_rn((float)a[4 * q + 1], rs), cs.y);
    const float f2 = __fmul_rn(__fmul_rn((float)a[4 * q + 2], rs), cs.z);
    const float f3 = __fmul_rn(__fmul_rn((float)a[4 * q + 3], rs), cs.w);
    w = v2u{__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f0, f1}, bf16x2)),
            __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{f2, f3}, bf16x2))};
  };
  auto row_scale = [&](const float* sc, int i) __attribute__((always_inline)) { return sc[wm * 128 + i * 32 + (lane & 31)]; };
  // raw accumulators of the finished tile (a parity hook): four consecutive columns per store
  auto export_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int m = om0 + wm * 128 + i * 32 + (lane & 31);
          const int n = on0 + col0(j) + 8 * q + 4 * kh;
          *reinterpret_cast<v4i*>(p.acc_out + (int64_t)m * N + n) =
              v4i{acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
        }
  };
  // Staging of one block: every lane writes its four 8-byte pieces (one row, 16 columns);
  // read back, four lanes take one 64-byte row, and each store writes 16 rows of 64 bytes
  // (an aligned half of each 128-byte line; col0 above says who writes the other half).  A
  // wave's LDS operations run in order, so the next block's writes may follow this block's
  // reads without a wait.
  auto stage_write = [&](const v2u (&w)[4]) __attribute__((always_inline)) {
#pragma unroll
    for (int q = 0; q < 4; ++q) *reinterpret_cast<v2u*>(stg_wr + 16 * (q ^ sw)) = w[q];
  };
  auto stage_read = [&](v4i (&rows)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k) rows[k] = *reinterpret_cast<const v4i*>(stg_rd + k * 16 * 64);
    rows[1] = v4i{rows[1][2], rows[1][3], rows[1][0], rows[1][1]};  // rows 16..31: halves swapped back
  };
  auto stage_store = [&](int i, int j, const v4i (&rows)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int rr = wm * 128 + i * 32 + k * 16;  // first of the 16 rows of this store, in the tile
      const int cc = col0(j);                     // first of the 32 columns, in the tile
      // Scalar tile base, 32-bit lane offset (256 ldy < 2^30).  Nontemporal (streaming) when
      // each XCD keeps a block of W resident in its L2 across many row blocks (the N-range
      // tile order): the output then stays out of the L2's reuse set.  Otherwise the stores
      // are cached, and the two halves of a line meet in the L2 before it is written back.
      // The whole offset is in the lane offset and soffset is the constant 0: the compiler
      // then keeps a wait state between the 16-byte store and a VALU write of its data
      // registers, which it leaves out when soffset is a register; without it the store sent
      // some dwords of the registers' next values (seen with the register reused at once).
      __builtin_amdgcn_raw_buffer_store_b128(rows[k], raw_rsrc(reinterpret_cast<int8_t*>(p.y) + ((int64_t)om0 * p.ldy + on0) * 2),
                                             (int)(yoff + (uint32_t)((rr * p.ldy + cc) * 2)), 0, NT ? 2 : 0);
    }
  };

  // Each thread fetches one of the tile's 512 scales (row scales 0..255, column scales
  // 256..511) with the tile's first slice and stores it to LDS at the next slice's wait,
  // before its barrier, so the epilogue (in the next tile's first slice, or after the last
  // tile) reads no global memory.
  float scale_v = 0.0f;
  int scale_par = -1;  // the tile parity scale_v belongs to, while it waits to be stored
  int after_dma = 0;   // output stores issued after the last DMA of the previous slice
  // The start of slice s: this wave's DMA of slice s (and any scale load) has landed.  VMEM
  // operations retire in issue order, so the output stores issued after the last DMA may stay
  // in flight.  The barrier makes every wave's slice visible and frees the stage of slice s-1
  // for slice s+1.
  auto slice_wait = [&]() __attribute__((always_inline)) {
    if (after_dma == 10)
      asm volatile("s_waitcnt vmcnt(10)" ::: "memory");
    else
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    after_dma = 0;
    if (scale_par >= 0) {
      scl[scale_par][t] = scale_v;
      scale_par = -1;
    }
    lds_barrier();
  };

  // A slice after a tile's first: operand fragments double-buffered in registers.  With
  // LDS-DMA loads in flight the compiler waits for every outstanding LDS read at once, so the
  // reads of step ks+1 are issued after the first MFMA of step ks: the wait in front of step
  // ks+1 then covers reads issued seven MFMAs earlier.  The next slice's eight DMA
  // instructions go out one per two MFMAs in the first half of the slice: the MFMA pipe keeps
  // running while the address unit accepts them, and they have the second half to land.
  // The MFMA takes the W fragment as its first operand: each lane then holds four
  // consecutive output columns of one row (register 4q + r: column 8q + 4(lane/32) + r of the
  // 32-column block, row lane % 32).
  auto next_slice = [&](const int8_t* sa, int xa, int xb, int xk, int8_t* xst) __attribute__((always_inline)) {
    const int8_t* sb = sa + kSliceB;
    v4i af[2][4], bf[2][2];
    auto read_frags = [&](int ks, v4i* a4, v4i* b2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) a4[i] = *reinterpret_cast<const v4i*>(sa + bswz(ar + i * 32, 2 * ks + kh));
#pragma unroll
      for (int j = 0; j < 2; ++j) b2[j] = *reinterpret_cast<const v4i*>(sb + bswz(brow(j), 2 * ks + kh));
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
          dma(4 * ks + (q >> 1), xa, xb, xk, xst);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // A tile's first slice, block by block (block b = (i, j) = (b % 4, b / 4), its four K steps
  // in a row), carrying the previous tile's epilogue (OLD): block b's accumulators have become
  // bf16 words before its first MFMA (converted during block b-1's MFMAs), and those words are
  // staged and stored during block b's MFMAs, so the epilogue's VALU, LDS and store work runs
  // beside the MFMA pipe instead of after it.  The fragments of one A row block and one W
  // column block (four K steps each) are in registers; K step ks of the next block's is
  // reloaded once this block's MFMA at ks is issued.
  auto first_slice = [&](auto OLD, const int8_t* sa, const float* sc, int xa, int xb, int xk,
                         int8_t* xst) __attribute__((always_inline)) {
    constexpr bool kOld = decltype(OLD)::value;
    const int8_t* sb = sa + kSliceB;
    v4i bfr[4], afr[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      bfr[ks] = *reinterpret_cast<const v4i*>(sb + bswz(brow(0), 2 * ks + kh));
      afr[ks] = *reinterpret_cast<const v4i*>(sa + bswz(ar, 2 * ks + kh));
    }
    v2u w[4];  // the words of the block being staged, then of the next block
    // the previous tile's scales in registers ahead of their use (an LDS read next to its
    // conversion would stall the wave for the LDS latency): the four row scales of this
    // lane, and the column scales of one 32-column block (the same for the four blocks of a
    // column), reloaded for the second column block once the first is done
    float rsr[4];
    float4 csr[4];
    if constexpr (kOld) {
#pragma unroll
      for (int i = 0; i < 4; ++i) rsr[i] = row_scale(sc, i);
#pragma unroll
      for (int q = 0; q < 4; ++q) csr[q] = col_scales(sc, 0, q);
#pragma unroll
      for (int q = 0; q < 4; ++q) conv(csr[q], 0, 0, q, rsr[0], w[q]);
    }
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = b & 3, j = b >> 2, ni = (b + 1) & 3, nj = (b + 1) >> 2;
      v4i rows[2];
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(bfr[ks], afr[ks], ks == 0 ? zero16 : acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        if ((ks & 1) && b < 4) dma(2 * b + (ks >> 1), xa, xb, xk, xst);
        if constexpr (kOld) {
          // block b: written (ks 0), read (ks 1), stored (ks 3); the words are free for
          // block b + 1 from ks 1
          if (ks == 0) stage_write(w);
          if (ks == 0 && b == 3) {
#pragma unroll
            for (int q = 0; q < 4; ++q) csr[q] = col_scales(sc, 1, q);
          }
          if (ks == 1) stage_read(rows);
          if (b < 7) {
            if (ks == 1) conv(csr[0], ni, nj, 0, rsr[ni], w[0]);
            if (ks == 2) {
              conv(csr[1], ni, nj, 1, rsr[ni], w[1]);
              conv(csr[2], ni, nj, 2, rsr[ni], w[2]);
            }
            if (ks == 3) conv(csr[3], ni, nj, 3, rsr[ni], w[3]);
          }
          if (ks == 3) stage_store(i, j, rows);
        }
        if (b < 7) {
          if (ni != i) afr[ks] = *reinterpret_cast<const v4i*>(sa + bswz(ar + ni * 32, 2 * ks + kh));
          if (nj != j) bfr[ks] = *reinterpret_cast<const v4i*>(sb + bswz(brow(nj), 2 * ks + kh));
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // one tile: its first slice (carrying the previous tile's epilogue when OLD), then the rest
  auto run_tile = [&](int ti, auto OLD) __attribute__((always_inline)) {
    constexpr bool kOld = decltype(OLD)::value;
    const int s0 = ti * KT;
    {
      slice_wait();
      scale_v = t < 256 ? p.a_scale[min(m0 + t, M - 1)] : p.w_scale[min(n0 + t - 256, N - 1)];
      scale_par = ti & 1;
      // the next slice: the same tile's next K slice, else the next tile's first (after the
      // last tile: the last tile again, into a stage nothing reads, so every slice issues
      // the same eight DMA instructions)
      const int xa = KT > 1 ? m0 : nm0, xb = KT > 1 ? n0 : nn0, xk = KT > 1 ? kBKb : 0;
      const int8_t* sa = smem + (s0 % kStages) * kStageB;
      int8_t* xst = smem + ((s0 + 1) % kStages) * kStageB;
      if constexpr (!kOld) {
        first_slice(std::false_type{}, sa, nullptr, xa, xb, xk, xst);
      } else {
        if constexpr (ACC) export_acc();
        first_slice(std::true_type{}, sa, scl[(ti - 1) & 1], xa, xb, xk, xst);
        // stores after the last DMA (block 3, K step 3): blocks 3..7, two each
        if constexpr (!ACC) after_dma = 10;
      }
    }
    for (int kt = 1; kt < KT; ++kt) {
      const int s = s0 + kt;
      slice_wait();
      const int xa = kt + 1 < KT ? m0 : nm0, xb = kt + 1 < KT ? n0 : nn0;
      const int xk = kt + 1 < KT ? (kt + 1) * kBKb : 0;
      next_slice(smem + (s % kStages) * kStageB, xa, xb, xk, smem + ((s + 1) % kStages) * kStageB);
    }
    om0 = m0;
    on0 = n0;
    m0 = nm0;
    n0 = nn0;
    if (ti + 2 < my_tiles) tile_at(ti + 2, nm0, nn0);
  };

  run_tile(0, std::false_type{});
  for (int ti = 1; ti < my_tiles; ++ti) run_tile(ti, std::true_type{});
  // the last tile's epilogue, on its own
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  if (scale_par >= 0) scl[scale_par][t] = scale_v;
  lds_barrier();
  {
    const float* sc = scl[(my_tiles - 1) & 1];
    if constexpr (ACC) export_acc();
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int i = b & 3, j = b >> 2;
      const float rs = row_scale(sc, i);
      v2u w[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) conv(col_scales(sc, j, q), i, j, q, rs, w[q]);
      v4i rows[2];
      stage_write(w);
      stage_read(rows);
      stage_store(i, j, rows);
    }
  }
}

// Eight consecutive bf16 columns per store: y 16-byte aligned, N and ldy multiples of 8;
// acc_out (when given) 16-byte aligned; 32-bit DMA lane offsets: lda, K < 2^23; 32-bit
// output offsets within a tile: ldy < 2^22.
bool big_fits(int M, int N, int K, int64_t lda, int64_t ldy, const void* y, const void* acc_out) {
  return K >= kBKb && K % kBKb == 0 && M >= kBT && N >= kBT && N % 8 == 0 && ldy % 8 == 0 && lda % 16 == 0 &&
         lda < (1 << 23) && K < (1 << 23) && ldy < (1 << 22) && reinterpret_cast<uintptr_t>(y) % 16 == 0 &&
         reinterpret_cast<uintptr_t>(acc_out) % 16 == 0;
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
  const size_t lds = kStages * (size_t)kStageB + 8 * kStgWave;
  const dim3 grid((unsigned)(wgs_per_xcd * 8));
  const bool acc = a.acc_out != nullptr, nt = bt.ncol != 0;
  auto go = [&](auto kern) {
    hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kern), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kern, grid, dim3(512), lds, st, a, bt, wgs_per_xcd);
    return hipGetLastError();
  };
  if (acc) return nt ? go(k_gemm_i8_big<true, true>) : go(k_gemm_i8_big<true, false>);
  return nt ? go(k_gemm_i8_big<false, true>) : go(k_gemm_i8_big<false, false>);
}

}  // namespace wq
