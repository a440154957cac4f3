// Tiled MFMA GEMM for prefill-sized M: INT8 (per-token x per-channel scales) and FP8 E4M3
// with power-of-two block scales, over strided groups or expert segments.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 一 (quant matmul with the scale
// epilogue to BF16) and section 五 (grouped matmul over the expert segments given by
// group_list); "DeepSeek V4 950 低精度优化全复盘" section 2.3 (SwiGLU fused behind the
// gate/up matmul); the SGLang PR #34277 summary (the FP8 contraction that reads the
// packed UE8M0 activation scales as written, with 128x128 power-of-two weight block
// scales).
//
// Tile: 128 x 128 outputs per workgroup, 128-byte K slices, four waves in a 2 x 2 grid of
// 64 x 64 wave tiles (2 x 2 MFMA tiles of 32 x 32).  Operand slices move global -> LDS with
// global_load_lds_dwordx4 (no VGPR staging) into a ring of LDS stages (4, or 3 with the
// SwiGLU pair of B tiles), so several slices are in flight while one feeds the MFMAs.  Rows
// of a slice are 128 bytes = 8 chunks of 16 bytes, XOR-swizzled by bits 1..3 of the row so
// the MFMA operand reads hit distinct banks.  FP8 slices carry their 128 rows' packed scale
// words in the same stage.
//  * INT8: v_mfma_i32_32x32x32_i8, 4 per slice per tile; exact int32 accumulation; the
//    epilogue computes bf16((f32(acc) * s_m) * sw_n).
//  * FP8: v_mfma_scale_f32_32x32x64_f8f6f4, 2 per slice per tile.  A 128-byte K slice is
//    exactly one scale block, so the block scales ride in the MFMA's E8M0 scale operands:
//    the activation byte is the packed UE8M0 byte itself, the weight byte is the exponent
//    field of its f32 power-of-two scale.  f32 accumulation.
//  * Segments (MoE): the grid is persistent; each workgroup builds the list of non-empty
//    (expert, 128-row tile) pairs from the segment offsets once, then walks the
//    (pair, column tile) work items with a grid stride, so empty experts cost nothing.
//  * SwiGLU: the workgroup computes the gate tile (columns n) and the up tile (columns
//    n + I) of the same rows together and writes f32 silu(g) * u.
// Rows or columns past the edge read a clamped valid row (they only feed outputs that
// are not stored); K must be a multiple of 128 here (the host routes other K elsewhere).
#include <type_traits>

#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

constexpr int kBM = 128, kBN = 128, kBK = 128;
constexpr int kSlice = kBM * kBK;  // bytes of one operand slice in LDS
constexpr int kScaleB = 1024;      // FP8: the slice's packed activation-scale words (4 waves x 256 B)
// LDS ring: STAGES - 1 slices in flight while one is multiplied (bytes per stage: A + B
// [+ B2] [+ scales]).  Dense tiles use 4 stages (128 KiB); the persistent segment kernels
// keep 16 KiB of static LDS for their work list (SegRing below).
// MT (INT8 only): 128-row A tiles per workgroup tile (1, or 2 for the 256-row tiles of large
// experts).
// KB (INT8 only): the slice's depth in bytes, 128 or 64 (a 64-deep slice keeps twice as
// many slices in flight in the same LDS).
template <bool FP8, bool DUAL, int STAGES, int MT = 1, int KB = 128>
struct TileRing {
  static constexpr int kOperands = MT + (DUAL ? 2 : 1);  // A slices (MT) + B (+ B2)
  static constexpr int kOpB = kBM * KB;                  // bytes of one 128-row operand slice
  static constexpr int kStageB = kOperands * kOpB + (FP8 ? kScaleB : 0);
  static constexpr int kStages = STAGES;
  static constexpr int kDmaPerSlice = (KB / 32) * kOperands + (FP8 ? 1 : 0);  // per wave
  static constexpr int kBytes = kStages * kStageB;
  static_assert(STAGES >= 2 && STAGES <= 6, "ring depth");
  static_assert(KB == 128 || (KB == 64 && !FP8), "64-deep slices are INT8 only");
  static_assert(MT == 1 || (MT == 2 && !FP8), "256-row tiles are INT8 only");
};
constexpr int kDenseStages = 4;
// Segment kernels (at most 144 KiB of ring next to the 16 KiB work list): slice depth and
// ring depth per epilogue and tile height.
template <int EPI, int MT>
struct SegRing {
  static constexpr int kKB = (EPI == 2 && MT == 2) ? 64 : 128;
  // 128-row tiles: 4 stages of 32 KiB (SwiGLU: 3 of 48 KiB; 6 of 24 KiB with 64-deep slices
  // measured no faster); 256-row tiles: 3 of 48 KiB (SwiGLU: 4 of 32 KiB with 64-deep
  // slices; 2 of 64 KiB left one slice in flight)
  static constexpr int kStages = MT == 1 ? (EPI == 2 ? 3 : 4) : (EPI == 2 ? 4 : 3);
  using Ring = TileRing<false, EPI == 2, kStages, MT, kKB>;
};
static_assert(SegRing<2, 2>::Ring::kBytes <= 144 * 1024 && SegRing<1, 2>::Ring::kBytes <= 144 * 1024 &&
                  SegRing<2, 1>::Ring::kBytes <= 144 * 1024 && SegRing<1, 1>::Ring::kBytes <= 144 * 1024,
              "segment rings fit next to the 16 KiB work list");
constexpr int kGroupM = 8;         // tile rows per group in the L2-friendly tile order
constexpr int kMaxSegTiles = kSegMaxPairs;  // (expert, row tile) pairs a persistent workgroup lists

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// A 128-byte row covers half of the 64 LDS banks, so rows r and r+2 share banks: the
// chunk is XORed with bits 1..3 of the row, and the 16 rows a ds_read_b128 pass reads at
// one logical chunk then land on distinct banks.
__device__ __forceinline__ int tswz_of(int r) { return (r >> 1) & 7; }
__device__ __forceinline__ int tswz(int r, int c) { return r * kBK + ((c ^ tswz_of(r)) << 4); }

// A slice is 128 rows x 128 bytes (rows of the operand, bytes [k0, k0 + 128)), written to
// LDS swizzled (tswz) by 16 DMA instructions of 64 lanes x 16 bytes: instruction w * 4 + i
// (wave w) carries the slice's 16-byte positions (w * 4 + i) * 64 + lane, position q being
// row q / 8, chunk (q % 8) ^ tswz_of(row), and lands at byte (w * 4 + i) * 1024.
// INT8 weights in fragment order (launch_pack_weight_i8, for N columns): chunk c (bytes
// 16c .. of the slice at k0) of column n sits at ((k0/64 + c/4) N/4 + n/4) 256 + 64 (c%4) + 16 (n%4).

// One INT8 tile of 128 MT rows x 128 columns (two B tiles when DUAL): acc[i][j] (and acc2)
// over all K.  a: rows [m0, row_hi) clamped; b: columns [n0, ..) of w (row stride K), b2 at
// n0 + dual_off.  Four waves in a 2 x 2 grid; wave (wm, wn) holds the 32-row blocks
// 2 i + wm (i < 2 MT) of the tile, so that a partly filled tile spreads its rows over both
// wave rows, and columns wn * 64 .. + 63: (2 MT) x 2 MFMA tiles of 32 x 32.  The MT A
// slices sit back to back in the stage, so A row r of the tile (0 .. 128 MT - 1) is at
// tswz(r, c) of the stage's first slice.
//
// Schedule, per slice kt (the FP8 tiles below follow the same plan):
//  * the slice's D DMA instructions per wave (for slice kt + STAGES - 1, into the stage of
//    slice kt - 1) are issued one at a time between the MFMAs of its first three K steps,
//    not in one burst: a burst held each wave at the address unit, MFMA pipe idle, for
//    about as long as the slice's MFMAs take;
//  * the LDS fragments of each K step are read one step ahead, into a second register set;
//    after the first MFMA of the last K step come the wait and the barrier that make slice
//    kt + 1 visible, and its first step's fragments are read there;
//  * the body is straight-line code: past the last slice, the DMA copies the last slice
//    into the stage no later slice uses, so every wait counts the same STAGES - 2 later
//    slices.  The next tile's opening __syncthreads() waits for those copies.
// With two stages only one slice is in flight, and its DMA goes out in the slice's first
// K step, to leave the others for the latency.
// NV (<= 2 MT): the wave's row blocks that hold a valid row, i < NV (the caller counts them):
// the MFMAs and fragment reads of the others are skipped; their accumulators stay zero and
// their rows are never stored.  Every wave still issues its whole share of the slices' DMA
// and meets every barrier, whatever its NV.
// KB: slice depth in bytes.  A 128-deep slice keeps operand row r at tswz(r, chunk); in a
// 64-deep slice rows 2R and 2R + 1 share the 128-byte LDS row R, as its chunks 0..3 and
// 4..7 (same swizzle, also free of bank conflicts for the fragment reads).
__device__ __forceinline__ int slice_off(int r, int c, int kb) {
  return kb == 128 ? tswz(r, c) : tswz(r >> 1, c + ((r & 1) << 2));
}

template <bool DUAL, int STAGES, int MT, int NV = 2 * MT, int KB = 128>
__device__ __forceinline__ void tile_mainloop(const TileArgs& p, int8_t* smem, const int8_t* A, int m0, int row_hi,
                                              const int8_t* B, int n0, int dual_off, v16i (&acc)[2 * MT][2],
                                              v16i (&acc2)[2 * MT][2]) {
  using Ring = TileRing<false, DUAL, STAGES, MT, KB>;
  constexpr int S = Ring::kStages, D = Ring::kDmaPerSlice, OPB = Ring::kOpB;
  constexpr int NB = DUAL ? 2 : 1;
  constexpr int KS = KB / 32;   // K steps (32 deep) per slice
  constexpr int DPO = KB / 32;  // DMA instructions per wave per 128-row operand slice
  static_assert(NV >= 1 && NV <= 2 * MT, "valid row blocks");
  constexpr int Q = NV * 2 * NB;              // MFMAs per K step
  // MFMA slots that carry the slice's DMA: those of the slice's K steps before the last
  // (several instructions share a slot when there are fewer slots than instructions); with
  // two stages, as early as the address unit allows, to leave the rest for the latency
  constexpr int kMaxWin = (KS - 1) * Q;
  constexpr int kWin = S == 2 ? (Q >= D ? Q : (2 * Q >= D ? 2 * Q : kMaxWin)) : kMaxWin;
  static_assert(kWin <= kMaxWin, "DMA window");
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = p.K, N = p.N;
  const int KT = K / KB;
#pragma unroll
  for (int i = 0; i < 2 * MT; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        acc[i][j][e] = 0;
        acc2[i][j][e] = 0;
      }

  // Every DMA instruction is a wave-uniform base plus a 32-bit lane offset.  The offsets
  // (rows clamped to the tile's valid range, chunks swizzled as slice_off places them) are
  // fixed for the tile; the bases step one slice at a time.  Weights in fragment order:
  // column n0 + g, chunk c of the 128-deep slice at k0 sits at byte
  // k0 N + 64 n0 + (c / 4) 64 N + (g / 4) 256 + (c % 4) 64 + (g % 4) 16 (n0 % 4 = 0).
  // The second B tile's columns (n0 + dual_off + g) never need the clamp: SwiGLU tiles have
  // n0 + 127 < N / 2 = dual_off.
  const bool frag = p.b_frag != 0;
  uint32_t aoff[MT][DPO], boff[DPO];
#pragma unroll
  for (int i = 0; i < DPO; ++i) {
    // 16-byte position in the operand slice; its LDS row, the chunk it holds there, and
    // the operand row and chunk that is
    const int pos = (wv * DPO + i) * 64 + lane;
    const int R = pos >> 3, cp = (pos & 7) ^ tswz_of(R);
    const int r = KB == 128 ? R : 2 * R + (cp >> 2), c = KB == 128 ? cp : (cp & 3);
#pragma unroll
    for (int h = 0; h < MT; ++h) aoff[h][i] = (uint32_t)(min(h * kBM + r, row_hi - 1 - m0) * (int)p.lda + c * 16);
    const int gr = min(r, N - 1 - n0);
    boff[i] = frag ? (uint32_t)((c >> 2) * (N >> 2) * 256 + (gr >> 2) * 256 + (c & 3) * 64 + (gr & 3) * 16)
                   : (uint32_t)(gr * K + c * 16);
  }
  const int8_t* a_base = A + (int64_t)m0 * p.lda;
  const int8_t* b_base = B + (int64_t)n0 * (frag ? 64 : K);
  const int64_t b_step = frag ? (int64_t)KB * N : KB;
  const int64_t b2_shift = (int64_t)dual_off * (frag ? 64 : K);

  // DMA instruction d of slice kt into ring slot `slot`: A (slice h = d / DPO) for
  // d < DPO MT, then B, then B2
  auto issue_one = [&](int kt, int d, int slot) {
    int8_t* st = smem + (slot % S) * Ring::kStageB + wv * (DPO * 1024);
    const int8_t* bk = b_base + kt * b_step;
    const int8_t* src;
    int8_t* dst;
    if (d < DPO * MT) {
      src = a_base + kt * KB + aoff[d / DPO][d % DPO];
      dst = st + (d / DPO) * OPB + (d % DPO) * 1024;
    } else if (d < DPO * (MT + 1)) {
      src = bk + boff[d - DPO * MT];
      dst = st + MT * OPB + (d - DPO * MT) * 1024;
    } else {
      src = bk + b2_shift + boff[d - DPO * (MT + 1)];
      dst = st + (MT + 1) * OPB + (d - DPO * (MT + 1)) * 1024;
    }
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), (lds_ptr_t)dst, 16, 0, 0);
  };

  const int ar = wm * 32 + (lane & 31), br = wn * 64 + (lane & 31);
  const int kh = lane >> 5;  // which half of the K step this lane carries: chunk 2 ks + kh
  struct Frags {
    v4i a[NV], b[2], b2[2];
  };
  auto read_step = [&](int slot, int ks, Frags& f) {
    const int8_t* sa = smem + (slot % S) * Ring::kStageB;
    const int8_t* sb = sa + MT * OPB;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int r = ar + i * 64;  // tile row; a 256-row tile's second A slice follows the first
      f.a[i] = *reinterpret_cast<const v4i*>(sa + (r >> 7) * OPB + slice_off(r & 127, 2 * ks + kh, KB));
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      f.b[j] = *reinterpret_cast<const v4i*>(sb + slice_off(br + j * 32, 2 * ks + kh, KB));
      if constexpr (DUAL) f.b2[j] = *reinterpret_cast<const v4i*>(sb + OPB + slice_off(br + j * 32, 2 * ks + kh, KB));
    }
  };
  auto wait_slice = [&]() { asm volatile("s_waitcnt vmcnt(%0)" ::"n"(D * (S - 2)) : "memory"); };

  // K step ks of slice kt on `cur`; `nxt` receives the following step's fragments
  auto step = [&](int kt, int ks, const Frags& cur, Frags& nxt) {
    const int nk = min(kt + S - 1, KT - 1);
#pragma unroll
    for (int q = 0; q < Q; ++q) {
      const int i = q / (2 * NB), j = (q / NB) & 1;
      if (NB == 1 || (q & 1) == 0)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[i], cur.b[j], acc[i][j], 0, 0, 0);
      else
        acc2[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(cur.a[i], cur.b2[j], acc2[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
      if (q == 0) {
        if (ks < KS - 1) {
          read_step(kt, ks + 1, nxt);
        } else {
          wait_slice();
          lds_barrier();  // slice kt + 1 is in LDS for everyone; every wave has read slice kt
          read_step(kt + 1, 0, nxt);
        }
      }
      const int g = ks * Q + q;  // MFMA slot in the slice
#pragma unroll
      for (int d = 0; d < D; ++d)
        if (((2 * d + 1) * kWin) / (2 * D) == g) issue_one(nk, d, kt + S - 1);
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  __syncthreads();  // the previous tile's LDS reads (and its copies past the end) are done
#pragma unroll
  for (int s = 0; s < S - 1; ++s)
#pragma unroll
    for (int d = 0; d < D; ++d) issue_one(min(s, KT - 1), d, s);
  wait_slice();  // slice 0 has landed once only slices 1 .. S-2 may be outstanding
  lds_barrier();
  Frags f0, f1;
  read_step(0, 0, f0);
  for (int kt = 0; kt < KT; ++kt) {
#pragma unroll
    for (int ks = 0; ks < KS; ks += 2) {
      step(kt, ks, f0, f1);
      step(kt, ks + 1, f1, f0);
    }
  }
}

// INT8 epilogue.  The lane holds column (lane & 31) and rows 8*(e/4) + 4*(lane>>5) + e%4 of
// each 32 x 32 MFMA tile (row blocks as in tile_mainloop), two MFMA row tiles at a time.
template <int EPI, int MT>
__device__ __forceinline__ void tile_epilogue(const TileArgs& p, int m0, int row_hi, int n0, int g, const float* wsc,
                                              v16i (&acc)[2 * MT][2], v16i (&acc2)[2 * MT][2]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int N = p.N;
  const int mb = m0 + wm * 32 + 4 * (lane >> 5);  // this lane's rows: mb + 64 i + 8 (e / 4) + e % 4
  float sw[2] = {1.0f, 1.0f}, sw2[2] = {0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + j * 32 + (lane & 31);
    if constexpr (EPI == 2) {
      const int I = N / 2;
      sw[j] = wsc[min(n, I - 1)];
      sw2[j] = wsc[min(n, I - 1) + I];
    } else {
      sw[j] = wsc[min(n, N - 1)];
    }
  }
#pragma unroll
  for (int hh = 0; hh < MT; ++hh) {
    // Every scale this half needs is loaded first, at clamped in-range indices, with no
    // branch between the loads: a scale loaded next to each store made every store group
    // wait for the stores before it.
    float rs[2][16];
#pragma unroll
    for (int ii = 0; ii < 2; ++ii)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        rs[ii][e] = p.a_scale[min(mb + (2 * hh + ii) * 64 + 8 * (e >> 2) + (e & 3), row_hi - 1)];
    // one wait for all of them, as a real s_waitcnt (vmcnt(0)) that the compiler's wait
    // accounting sees: without it, the per-row store branches made it wait again before
    // each scale's use, and so for every store issued before
    __builtin_amdgcn_s_waitcnt(0x0F70);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int n = n0 + wn * 64 + j * 32 + (lane & 31);
      if constexpr (EPI == 2) {
        const int I = N / 2;
        if (n >= I) continue;
        float* H = reinterpret_cast<float*>(p.y);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = 2 * hh + ii;
            const int m = mb + i * 64 + 8 * (e >> 2) + (e & 3);
            if (m < row_hi) {
              const float s = rs[ii][e];
              const float gv = __fmul_rn(__fmul_rn((float)acc[i][j][e], s), sw[j]);
              const float uv = __fmul_rn(__fmul_rn((float)acc2[i][j][e], s), sw2[j]);
              const float sg = __fdiv_rn(gv, __fadd_rn(1.0f, exp_fixed(-gv)));
              H[(int64_t)m * p.ldy + n] = __fmul_rn(sg, uv);
            }
          }
      } else {
        if (n >= N) continue;
        uint16_t* Y = reinterpret_cast<uint16_t*>(p.y) + (p.seg_offsets ? 0 : (int64_t)g * p.y_batch_stride);
#pragma unroll
        for (int ii = 0; ii < 2; ++ii)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int i = 2 * hh + ii;
            const int m = mb + i * 64 + 8 * (e >> 2) + (e & 3);
            if (m < row_hi) {
              Y[(int64_t)m * p.ldy + n] =
                  (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)acc[i][j][e], rs[ii][e]), sw[j]));
              if (p.acc_out) p.acc_out[(int64_t)m * N + n] = acc[i][j][e];
            }
          }
      }
    }
  }
}

// FP8 (and MX) dense tiles: the same 128 x 128 tile and LDS ring, scheduled for one wave
// per SIMD.  Per 128-byte slice each wave runs 8 block-scaled MFMAs; the schedule keeps the
// MFMA pipe fed across the slice boundary:
//  * the slice's nine DMA instructions per wave (A, B, the scale words) are issued one per
//    MFMA instead of in one burst, which held the wave at the address unit for ~600 cycles a
//    slice with the MFMA pipe idle;
//  * LDS operand reads run a whole slice ahead, into a second register set: after slice
//    kt's first MFMA comes the wait and barrier that make slice kt+1 visible, then slice
//    kt+1's fragments and scale words are read while slice kt's other seven MFMAs run.
//    (Under the DMA traffic an LDS read takes ~700 cycles to return, and with LDS-DMA loads
//    in flight the compiler waits for all outstanding LDS reads at once, so a read must be
//    issued well before the MFMA that needs it.)
//  * the MFMA takes the W fragment as its first operand, so each lane ends with four
//    consecutive output columns of one row; the epilogue stages bf16 rows through LDS and
//    each store instruction writes eight whole 128-byte rows of Y.
// The DMA issued during slice kt fills the stage of slice kt-1, whose reads every wave
// finished (and waited for) before the barrier of slice kt-1.

// DMA instruction i (0..3) of a 128-row x 128-byte operand slice (this wave's i-th, as above)
__device__ __forceinline__ void dma_slice_one(const int8_t* src, int64_t ld, int r0, int rows, int k0, int8_t* dst,
                                              int wv, int lane, int i) {
  const int pos = (wv * 4 + i) * 64 + lane;
  const int r = pos >> 3, pc = pos & 7;
  const int c = pc ^ tswz_of(r);
  const int gr = min(r0 + r, rows - 1);
  __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src + (int64_t)gr * ld + k0 + c * 16),
                                   (lds_ptr_t)(dst + (wv * 4 + i) * 1024), 16, 0, 0);
}

template <int STAGES, bool MX>
__device__ __forceinline__ void fp8_tile_mainloop(const TileArgs& p, int8_t* smem, const int8_t* A, int m0, int row_hi,
                                                  const int8_t* B, int n0, int g, v16f (&acc)[2][2]) {
  using Ring = TileRing<true, false, STAGES>;
  static_assert(Ring::kDmaPerSlice == 9, "A 4 + B 4 + scales 1 per wave");
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int K = p.K, N = p.N;
  const int KT = K / kBK;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
  constexpr bool mx = MX;  // a template parameter: a runtime flag put branches in the loop body
  const int PH = mx ? KT : (KT + 3) >> 2;
  const int32_t* xs_g = p.a_scale_packed + (int64_t)g * PH * p.a_scale_tokens;
  const float* ws_g = !mx ? p.w_scale + ((int64_t)g * (N / 128) + (n0 >> 7)) * KT : nullptr;
  const uint32_t* wsw_g = mx ? reinterpret_cast<const uint32_t*>(p.w_scale) + (int64_t)g * N * KT : nullptr;

  // DMA instruction d (0..8) of slice kt: A 0-3, B 4-7, the scale words 8 (as tile_mainloop)
  auto issue_one = [&](int kt, int d, int slot) {
    int8_t* st = smem + (slot % Ring::kStages) * Ring::kStageB;
    if (d < 4) {
      dma_slice_one(A, p.lda, m0, row_hi, kt * kBK, st, wv, lane, d);
    } else if (d < 8) {
      dma_slice_one(B, K, n0, N, kt * kBK, st + kSlice, wv, lane, d - 4);
    } else {
      // both addresses computed on every lane and one picked by a select (a conditional
      // address computation became a branch that split the loop body)
      const int r = min(m0 + wv * 32 + (lane & 31), row_hi - 1);
      const char* xa = reinterpret_cast<const char*>(xs_g + (int64_t)(mx ? kt : kt >> 2) * p.a_scale_tokens + r);
      const char* wa = mx ? reinterpret_cast<const char*>(wsw_g + (int64_t)min(n0 + wv * 32 + (lane & 31), N - 1) * KT + kt)
                          : reinterpret_cast<const char*>(ws_g + kt);
      const bool w_lane = mx ? lane >= 32 : lane == 32;
      const int64_t dw = wa - xa;
      __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(xa + (w_lane ? dw : (int64_t)0)),
                                       (lds_ptr_t)(st + 2 * kSlice + wv * 256), 4, 0, 0);
    }
  };
  // The loop body is straight-line code (a branch lets the compiler sink the MFMAs below
  // it): every iteration issues the DMA of slice kt + STAGES - 1, past the last slice a copy
  // of the last slice into the stage no later slice uses, so exactly STAGES - 2 later slices
  // of 9 instructions each are in flight at every wait (loads complete in order), and the
  // final iteration reads fragments it does not use.  __syncthreads() before the epilogue
  // waits for those copies.
  static_assert(Ring::kStages == 4, "the waits count the later slices in flight");
  // at the wait for slice kt+1 (in slice kt, before slice kt+3's DMA goes out) only slice
  // kt+2's nine instructions are in flight after it
  auto wait_slice = [&]() { asm volatile("s_waitcnt vmcnt(9)" ::: "memory"); };

  const int ar = wm * 64 + (lane & 31), br = wn * 64 + (lane & 31);
  const int kh = lane >> 5;
  // fragments of K step ks (0, 1) of the slice at sa: lane group h holds K bytes 16h..16h+15
  // of the step in registers 0-3 and 32+16h.. in 4-7 (128-block scales: any shared K order
  // gives the same sum, so those keep 32 contiguous bytes per lane); row and column scale words
  // one slice's operands in registers: both K steps' fragments and the scale words
  struct Frags {
    v8i a[2][2], b[2][2];  // [ks][i]
    int rw[2], cw[2], scb;
  };
  auto read_slice = [&](const int8_t* sa, Frags& f) {
    const int8_t* sb = sa + kSlice;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c0 = mx ? 4 * ks + kh : 4 * ks + 2 * kh, c1 = mx ? 4 * ks + 2 + kh : 4 * ks + 2 * kh + 1;
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const v4i lo = *reinterpret_cast<const v4i*>(sa + tswz(ar + i * 32, c0));
        const v4i hi = *reinterpret_cast<const v4i*>(sa + tswz(ar + i * 32, c1));
        f.a[ks][i] = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        const v4i blo = *reinterpret_cast<const v4i*>(sb + tswz(br + i * 32, c0));
        const v4i bhi = *reinterpret_cast<const v4i*>(sb + tswz(br + i * 32, c1));
        f.b[ks][i] = v8i{blo[0], blo[1], blo[2], blo[3], bhi[0], bhi[1], bhi[2], bhi[3]};
      }
    }
    const int32_t* scw = reinterpret_cast<const int32_t*>(sa + 2 * kSlice);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int r = ar + i * 32;  // row in the tile; its word sits at (r / 32) * 64 + r % 32
      f.rw[i] = scw[(r >> 5) * 64 + (r & 31)];
      const int c = br + i * 32;  // column in the tile (MX): at (c / 32) * 64 + 32 + c % 32
      f.cw[i] = mx ? scw[(c >> 5) * 64 + 32 + (c & 31)] : 0;
    }
    f.scb = (scw[32] >> 23) & 0xFF;  // exponent field of the f32 power-of-two block scale
  };

  // Slice kt on the operands in `cur` (read one slice earlier).  After its first MFMA: the
  // wait for this wave's DMA of slice kt+1 and the barrier that makes slice kt+1 visible
  // (every wave read slice kt-1 one slice ago, so the DMA issued below into its stage is
  // safe), then slice kt+1's operands are read into `nxt`, a whole slice ahead of their use.
  // The slice's other seven MFMAs carry the nine DMA instructions of slice kt+3.
  auto step = [&](int kt, const Frags& cur, Frags& nxt) {
    const int nk = min(kt + Ring::kStages - 1, KT - 1);
    const int nst = kt + Ring::kStages - 1;  // the stage slot of slice nk (its copy past the end)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int sub = 2 * ks + kh;  // MX: this lane group's 32-element block of the slice
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int i = q >> 1, j = q & 1;
        const int sca = mx ? (cur.rw[i] >> (8 * sub)) & 0xFF : (cur.rw[i] >> (8 * (kt & 3))) & 0xFF;
        const int scb = mx ? (cur.cw[j] >> (8 * sub)) & 0xFF : cur.scb;
        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(cur.b[ks][j], cur.a[ks][i], acc[i][j], 0, 0, 0, scb, 0, sca);
        __builtin_amdgcn_sched_barrier(0);
        if (ks == 0 && q == 0) {
          wait_slice();
          lds_barrier();
          read_slice(smem + ((kt + 1) % Ring::kStages) * Ring::kStageB, nxt);
        } else {
          const int d = 4 * ks + q - 1;  // 0..6; the last two instructions go behind the final MFMA
          issue_one(nk, d, nst);
          if (ks == 1 && q == 3) {
            issue_one(nk, 7, nst);
            issue_one(nk, 8, nst);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  __syncthreads();  // the previous tile's LDS reads are done before the new DMA lands
  for (int kt = 0; kt < Ring::kStages - 1; ++kt)
    for (int d = 0; d < Ring::kDmaPerSlice; ++d) issue_one(min(kt, KT - 1), d, kt);
  // slice 0 has landed once slices 1 and 2 alone may be outstanding
  asm volatile("s_waitcnt vmcnt(18)" ::: "memory");
  lds_barrier();
  Frags f0, f1;
  read_slice(smem, f0);
  // two slices per trip with the operand sets swapped, so no register copies; an odd last
  // slice after the loop
  int kt = 0;
  for (; kt + 1 < KT; kt += 2) {
    step(kt, f0, f1);
    step(kt + 1, f1, f0);
  }
  if (kt < KT) step(kt, f0, f1);
}

// FP8 epilogue: acc (W-first MFMA: lane holds row lane % 32 of each 32-row block and columns
// 8q + 4(lane/32) + r of each 32-column block) -> bf16 rows staged through LDS (144-byte
// pitch) -> 16-byte stores of whole 128-byte rows
__device__ __forceinline__ void fp8_tile_epilogue(const TileArgs& p, int8_t* smem, int m0, int row_hi, int n0, int g,
                                                  v16f (&acc)[2][2]) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int wm = wv >> 1, wn = wv & 1, kh = lane >> 5;
  constexpr int kPitch = 144;
  __syncthreads();  // every wave is done with the ring: it becomes the staging area
  int8_t* stg = smem + wv * 64 * kPitch;
  int8_t* wr = stg + (lane & 31) * kPitch + kh * 8;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef unsigned v2u __attribute__((ext_vector_type(2)));
        const v16f& a = acc[i][j];
        // round to nearest even (v_cvt_pk_bf16_f32), as f32_to_bf16_rn for finite values
        const v2u w = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a[4 * q], a[4 * q + 1]}, bf16x2)),
                       __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a[4 * q + 2], a[4 * q + 3]}, bf16x2))};
        *reinterpret_cast<v2u*>(wr + i * 32 * kPitch + j * 64 + q * 16) = w;
      }
  uint16_t* Y = reinterpret_cast<uint16_t*>(p.y) + (int64_t)g * p.y_batch_stride;
  const int8_t* rd = stg + (lane / 8) * kPitch + (lane % 8) * 16;
  v4i rows[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) rows[k] = *reinterpret_cast<const v4i*>(rd + k * 8 * kPitch);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const int m = m0 + wm * 64 + k * 8 + lane / 8;
    if (m < row_hi)
      __builtin_nontemporal_store(rows[k], reinterpret_cast<v4i*>(Y + (int64_t)m * p.ldy + n0 + wn * 64 + (lane % 8) * 8));
  }
}

// Dense or strided groups: one tile per workgroup, (group, tile) items on a 1-D grid.
template <bool FP8>
__global__ __launch_bounds__(256) void k_gemm_tile(TileArgs p, int tiles_m, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  // XCD-aware order over all (group, tile) items: consecutive workgroups land on different
  // XCDs (round robin), so each XCD gets a contiguous run of items, whole groups first
  // (8 groups of 32 tiles: one group per XCD, whose L2 then fetches that group's
  // activations and weights from HBM once); within a group, tiles go in groups of kGroupM
  // tile rows sweeping the tile columns, so the A rows and B columns a CU group works on
  // at once stay in that XCD's L2
  const int nt = tiles_m * tiles_n;
  const int total = nt * p.batch;
  const int bid = blockIdx.x;
  const int xcd = bid & 7, slot = bid >> 3;
  const int per_xcd = (total + 7) >> 3;
  const int item = xcd * per_xcd + slot;
  if (slot >= per_xcd || item >= total) return;
  const int g = item / nt;
  const int lin = item - g * nt;
  const int8_t* A = p.a + (int64_t)g * p.a_batch_stride;
  const int8_t* B = p.w + (int64_t)g * p.w_batch_stride;
  const int group = lin / (kGroupM * tiles_n);
  const int gm0 = group * kGroupM;
  const int gsz = min(kGroupM, tiles_m - gm0);
  const int in = lin - group * kGroupM * tiles_n;
  const int tm = gm0 + in % gsz, tn = in / gsz;
  const int m0 = tm * kBM, n0 = tn * kBN;
  if constexpr (FP8) {
    v16f acc[2][2];
    if (p.mx)
      fp8_tile_mainloop<kDenseStages, true>(p, smem, A, m0, p.M, B, n0, g, acc);
    else
      fp8_tile_mainloop<kDenseStages, false>(p, smem, A, m0, p.M, B, n0, g, acc);
    fp8_tile_epilogue(p, smem, m0, p.M, n0, g, acc);
  } else {
    v16i acc[2][2], acc2[2][2];
    tile_mainloop<false, kDenseStages, 1>(p, smem, A, m0, p.M, B, n0, 0, acc, acc2);
    tile_epilogue<1, 1>(p, m0, p.M, n0, g, p.w_scale + (int64_t)g * p.N, acc, acc2);
  }
}

// Expert segments (INT8), persistent.  EPI 1: bf16 [rows, N]; EPI 2: f32 silu(gate)*up [rows, N/2].
// With seg_tall, an expert's rows go in units of 256: a unit of more than 128 rows is one
// tall tile (256 rows, MT = 2), so that each column tile of the expert's weights is streamed
// once for it; a unit of at most 128 rows (only an expert's last unit can be one) is a
// 128-row tile (MT = 1).  Without it every 128-row block is a 128-row tile.  One launch
// takes both kinds, tall tiles first (a launch of its own left the few tall tiles of a
// typical routing alone on a few CUs).
template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_seg(TileArgs p, int tiles_n) {
  extern __shared__ __attribute__((aligned(16))) int8_t smem[];
  // one word per tile: expert << 16 | first 128-row block << 1 | tall (16 KiB, so that with
  // the largest ring of 144 KiB the workgroup holds 160 KiB)
  __shared__ int pair_list[kMaxSegTiles];
  const int t = threadIdx.x;
  // list the tiles in expert order, the tall ones first (one wave, scan by shuffles)
  if (t < 64) {
    int base = 0;
    for (int pass = 0; pass < 2; ++pass) {
      const bool tall_pass = pass == 0;
      if (tall_pass && !p.seg_tall) continue;
      for (int e0 = 0; e0 < p.batch; e0 += 64) {
        const int e = e0 + t;
        int cnt = 0, b0 = 0, bstep = 1;
        if (e < p.batch) {
          const int64_t rows = p.seg_offsets[e + 1] - p.seg_offsets[e];
          const bool take = rows > 0 && rows >= p.seg_min_rows;
          if (p.seg_tall) {
            const int units = take ? (int)((rows + 2 * kBM - 1) / (2 * kBM)) : 0;
            const bool short_tail = units > 0 && rows - (int64_t)(units - 1) * 2 * kBM <= kBM;
            // tall pass: units 0 .. cnt-1; short pass: the last unit
            cnt = tall_pass ? units - (short_tail ? 1 : 0) : (short_tail ? 1 : 0);
            b0 = tall_pass ? 0 : 2 * (units - 1);
            bstep = 2;
          } else {
            cnt = take ? (int)((rows + kBM - 1) / kBM) : 0;
          }
        }
        int incl = cnt;
#pragma unroll
        for (int o = 1; o < 64; o <<= 1) {
          const int u = __shfl_up(incl, o, 64);
          if (t >= o) incl += u;
        }
        const int start = base + incl - cnt;
        for (int j = 0; j < cnt; ++j)
          if (start + j < kMaxSegTiles) pair_list[start + j] = (e << 16) | ((b0 + bstep * j) << 1) | (tall_pass ? 1 : 0);
        base += __shfl(incl, 63, 64);
      }
    }
    // the count goes through the ring's first word, which no DMA touches before the
    // mainloop's opening barrier
    if (t == 0) *reinterpret_cast<int*>(smem) = base < kMaxSegTiles ? base : kMaxSegTiles;
  }
  __syncthreads();
  const int npair = *reinterpret_cast<const int*>(smem);
  const int nn = (EPI == 2) ? (p.N / 2 + kBN - 1) / kBN : tiles_n;
  // The items of one tile row (its nn column tiles) share item % 8, and so, with the grid a
  // multiple of 8 and workgroups dealt to the 8 XCDs in turn, one XCD: its rows of the
  // activations come into that XCD's L2 once.  Tile rows go in groups of 8, one per XCD;
  // the last group's missing ones are skipped.
  const int total = (npair + 7) / 8 * 8 * nn;
  for (int item = blockIdx.x; item < total; item += gridDim.x) {
    const int rest = item >> 3, grp = rest / nn, tn = rest - grp * nn;
    const int pi = grp * 8 + (item & 7);
    if (pi >= npair) continue;
    const int pw = pair_list[pi];
    const int e = pw >> 16;
    const int m0 = (int)p.seg_offsets[e] + ((pw & 0xFFFF) >> 1) * kBM;
    const int row_hi = (int)p.seg_offsets[e + 1];
    const int8_t* B = p.w + (int64_t)e * p.w_batch_stride;
    const float* wsc = p.w_scale + (int64_t)e * p.N;
    const int n0 = tn * kBN;
    // this wave's row blocks 2 i + wm with a valid row: i < nv (wave-uniform)
    const int wm = (int)threadIdx.x >> 7;
    const int nblk = (row_hi - m0 + 31) >> 5;
    const int nv = __builtin_amdgcn_readfirstlane((nblk - wm + 1) >> 1);
    constexpr bool DU = EPI == 2;
    if (pw & 1) {
      v16i acc[4][2], acc2[4][2];
      constexpr int S2 = SegRing<EPI, 2>::kStages, KB2 = SegRing<EPI, 2>::kKB;
      if (nv <= 2)  // a tall tile holds at least 129 rows: every wave has two blocks or more
        tile_mainloop<DU, S2, 2, 2, KB2>(p, smem, p.a, m0, row_hi, B, n0, p.N / 2, acc, acc2);
      else if (nv == 3)
        tile_mainloop<DU, S2, 2, 3, KB2>(p, smem, p.a, m0, row_hi, B, n0, p.N / 2, acc, acc2);
      else
        tile_mainloop<DU, S2, 2, 4, KB2>(p, smem, p.a, m0, row_hi, B, n0, p.N / 2, acc, acc2);
      tile_epilogue<EPI, 2>(p, m0, row_hi, n0, 0, wsc, acc, acc2);
    } else {
      v16i acc[2][2], acc2[2][2];
      constexpr int S1 = SegRing<EPI, 1>::kStages, KB1 = SegRing<EPI, 1>::kKB;
      if (nv <= 1)  // (a wave with no valid block multiplies its padding rows)
        tile_mainloop<DU, S1, 1, 1, KB1>(p, smem, p.a, m0, row_hi, B, n0, p.N / 2, acc, acc2);
      else
        tile_mainloop<DU, S1, 1, 2, KB1>(p, smem, p.a, m0, row_hi, B, n0, p.N / 2, acc, acc2);
      tile_epilogue<EPI, 1>(p, m0, row_hi, n0, 0, wsc, acc, acc2);
    }
  }
}

template <bool DUAL>
constexpr size_t seg_ring_bytes() {
  constexpr size_t a = SegRing<DUAL ? 2 : 1, 1>::Ring::kBytes;
  constexpr size_t b = SegRing<DUAL ? 2 : 1, 2>::Ring::kBytes;
  return a > b ? a : b;
}

bool tile_fits(int K, int64_t lda) { return K % kBK == 0 && lda < (1 << 23); }

hipError_t launch_gemm_tile(const TileArgs& a, bool fp8, hipStream_t st) {
  if (!tile_fits(a.K, a.lda)) return hipErrorInvalidValue;
  const int tiles_n = (a.N + kBN - 1) / kBN;
  if (a.seg_offsets) {
    if (fp8) return hipErrorInvalidValue;
    if (a.epilogue == 2 && (a.N % 256) != 0) return hipErrorInvalidValue;
    const bool dual = a.epilogue == 2;
    int dev = 0, cus = 256;
    (void)hipGetDevice(&dev);
    (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const size_t lds = dual ? seg_ring_bytes<true>() : seg_ring_bytes<false>();
    auto kfn = dual ? k_gemm_seg<2> : k_gemm_seg<1>;
    hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kfn), (int)lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(kfn, dim3((unsigned)(2 * cus)), dim3(256), lds, st, a, tiles_n);
    return hipGetLastError();
  }
  const int tiles_m = (a.M + kBM - 1) / kBM;
  const int nt = tiles_m * tiles_n;
  const int64_t total = (int64_t)nt * a.batch;
  dim3 grid((unsigned)(((total + 7) / 8) * 8)), block(256);
  const size_t lds = fp8 ? (size_t)TileRing<true, false, kDenseStages>::kBytes
                          : (size_t)TileRing<false, false, kDenseStages>::kBytes;
  auto kfn = fp8 ? k_gemm_tile<true> : k_gemm_tile<false>;
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kfn), (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kfn, grid, block, lds, st, a, tiles_m, tiles_n);
  return hipGetLastError();
}

}  // namespace wq
