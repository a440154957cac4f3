// Host-side launchers for the wq kernels (internal to libwq).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace wq {

// Raise a kernel's dynamic-LDS limit to `bytes` on the current device, once per (kernel,
// device); safe to call from several host threads (wq_api.hip).
hipError_t set_lds_limit(const void* kernel, int bytes);

// Per-token INT8 quant (k_quant.hip).  S = K-split factor.  *ch_used reports the
// register-cache depth chosen (0 = streamed rows).
hipError_t launch_dynamic_quant(const void* x, bool x_f32, int64_t M, int K, int64_t ldx,
                                const uint16_t* gamma, float eps, const int32_t* row_index, int8_t* xq,
                                float* xs, int S, hipStream_t st, int* ch_used);

// Decode-sized INT8 GEMM, M <= 64 (k_decode.hip); also the argument block of the fused
// decode kernels (x non-null: they quantise the bf16 rows themselves).
struct DecodeArgs {
  const int8_t* a;        // int8 [M, lda]
  int64_t lda;
  const float* a_scale;   // f32 [M]
  const uint16_t* x;      // bf16 [M, ldx] (fused) or null
  int64_t ldx;
  const int8_t* w;        // int8 [N, K]
  const float* w_scale;   // f32 [N]
  int M, N, K;
  uint16_t* y;            // bf16 [M, ldy]
  int64_t ldy;
  int32_t* acc_out;       // optional [M, N]
  int8_t* xq_out;         // optional (fused)
  float* xs_out;          // optional (fused)
};
// nt: output columns per workgroup (4, 8 or 16); mt: 16-row MFMA tiles per workgroup
// (1, 2 or 4), the grid's second dimension covering ceil(M / (16 mt)) row tiles.
hipError_t launch_decode(const DecodeArgs& a, int nt, int mt, hipStream_t st);
// One-launch fused quant + GEMM for M <= 64, K % 512 == 0, K <= 4096 (k_fused.hip);
// nt output columns (4, 8, 16 or 32) and rows_per_wg rows (1, 2, 4, 8 or 16) per
// workgroup, ceil(N / nt) * ceil(M / rows_per_wg) workgroups
// packed: a.w holds the weights in fragment order (launch_pack_weight_i8), N % 4 == 0
hipError_t launch_fused_decode(const DecodeArgs& a, int nt, int rows_per_wg, hipStream_t st, bool packed = false);
// weights int8 [N, K] (row stride ldw) -> fragment order: byte (n, k) at
// ((k/64 * N/4 + n/4) * 4 + (k%64)/16) * 64 + (n%4) * 16 + k%16; N % 4 == 0, K % 64 == 0
hipError_t launch_pack_weight_i8(const int8_t* w, int64_t ldw, int N, int K, int8_t* wp, hipStream_t st);
bool fused_decode_fits(int M, int K);
// the same kernel on given INT8 codes (x null): M < 256 (row tiles of up to 16 rows)
bool given_decode_fits(int M, int K);
// GEMV-style kernel for M <= 8 (k_decode.hip); fused needs M <= 4 and K <= 8192
hipError_t launch_gemv(const DecodeArgs& a, hipStream_t st);
bool gemv_fits(int M, int K, bool fused);

// Tiled INT8 GEMM for large M (k_gemm_i8.hip), optionally over expert segments.
struct TileArgs {
  const int8_t* a;        // int8 rows, row stride lda
  int64_t lda;
  const float* a_scale;   // f32 per row
  const int8_t* w;        // int8 [batch][N][K]
  int64_t w_batch_stride;
  const float* w_scale;   // f32 [batch][N]
  int M, N, K;
  int epilogue;           // 1 = bf16, 2 = swiglu f32
  void* y;
  int64_t ldy;
  int32_t* acc_out;       // optional [M, N] (dense only)
  const int64_t* seg_offsets;  // device [batch+1] or null (dense)
  int batch;
  int64_t a_batch_stride;      // strided groups: bytes between groups of a
  const int32_t* a_scale_packed;  // FP8: packed UE8M0 storage [batch, PH, TA]
  int64_t a_scale_tokens;      // FP8: TA
  int64_t y_batch_stride;      // strided groups: elements between groups of y
  int seg_min_rows;            // segments: experts with fewer rows are left to another kernel
  int b_frag;                  // INT8 segments: each expert's w in the fragment order of launch_pack_weight_i8
  int mx;                      // FP8: MX-like 32-element blocks (storage [G, K/128, TA]; w_scale bytes [G][N][K/32])
  int seg_tall;                // INT8 segments: 256-row tiles for experts' units of 129..256 rows (else 128-row tiles only)
};
hipError_t launch_gemm_i8_tile(const TileArgs& a, hipStream_t st);
// 128x128 tiles with DMA-fed LDS (k_gemm_tile.hip); K % 128 == 0
hipError_t launch_gemm_tile(const TileArgs& a, bool fp8, hipStream_t st);
bool tile_fits(int K, int64_t lda);  // K % 128 == 0, lda < 2^23 (32-bit DMA lane offsets)
// (expert, 128-row tile) pairs the segmented kernel can hold
constexpr int kSegMaxPairs = 4096;
// Segments: experts with at most this many rows go to the weight-streaming kernel
// (k_seg_decode.hip), the rest to the tiled one
constexpr int kSegSmallRows = 16;
hipError_t launch_seg_decode(const TileArgs& a, int num_cu, hipStream_t st);
bool seg_decode_fits(int N, int K, int epilogue, int64_t batch);
// persistent 256x256 INT8 tiles for large M (k_gemm_big.hip)
hipError_t launch_gemm_i8_big(const TileArgs& a, int num_cu, hipStream_t st);
bool big_fits(int M, int N, int K, int64_t lda, int64_t ldy, const void* y, const void* acc_out);

// FP8 grouped contraction for T <= 64, K % 512 == 0, K <= 4096 (k_fp8_decode.hip):
// 16 output columns of one group and min(rt_per_wg, ceil(T / 16)) 16-token tiles per
// workgroup, grid (N / 16, G, ceil(ceil(T / 16) / that))
// mx: 32-element blocks (activation storage [G, K/128, TA]; w_scale UE8M0 bytes [G][N][K/32])
hipError_t launch_fp8_decode(const TileArgs& a, int rt_per_wg, hipStream_t st, bool mx = false);
bool fp8_decode_fits(int T, int N, int K);
// 32 output columns of one group per workgroup of 8 waves, all token tiles (16 < T <= 64,
// K % 1024 == 0, K <= 4096, N % 32 == 0), grid (N / 32, G); at T <= 16 the 16-column
// kernel is faster (one token tile: the activation re-reads it saves are few)
hipError_t launch_fp8_decode32(const TileArgs& a, hipStream_t st, bool mx = false);
bool fp8_decode32_fits(int T, int N, int K);

// FP8 group quant with packed UE8M0 scales (k_fp8.hip).
hipError_t launch_group_quant_fp8(const uint16_t* x, int64_t T, int G, int D, uint8_t* xq, int32_t* xs,
                                  hipStream_t st, int ppw_force = 0);
// the same with MX-like 32-element blocks (D % 32 == 0; HG = D / 32)
hipError_t launch_group_quant_mx(const uint16_t* x, int64_t T, int G, int D, uint8_t* xq, int32_t* xs,
                                 hipStream_t st);

// Expert sort (k_moe.hip).
hipError_t launch_moe_sort(const int32_t* ids, int64_t T, int topk, int E, int32_t* perm, int32_t* row_token,
                           int64_t* offsets, hipStream_t st);

}  // namespace wq
