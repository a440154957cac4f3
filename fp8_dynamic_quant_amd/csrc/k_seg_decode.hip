// Segmented INT8 GEMM for the experts that hold few rows: weight streaming per expert.
//
// Operation: "DeepSeek-V4 W8A8 性能分析", section 五 (grouped matmul over the expert
// segments of group_list; most experts of a decode-sized batch receive a handful of
// tokens) and "DeepSeek V4 950 低精度优化全复盘" section 2.3 (SwiGLU fused behind the
// gate/up matmul, f32 result kept for the requant).
//
// With 256 tokens routed top-8 over 256 experts, ~90 % of the active experts get at most
// 16 rows, and their weights (16 MiB gate/up + 8 MiB down each) are what the block
// streams.  A 128 x 128 tile would re-read a 128-row activation tile per column tile and
// spend its MFMAs on padding; here a work item is (expert, 16 output columns, whole K):
//  * the persistent grid lists the experts with 1 <= rows <= 16 once, in LDS, and walks
//    the (expert, column tile) items with a grid stride;
//  * 8 waves split K; each wave loads its weight slice (16 bytes per lane per 64-deep step,
//    the v_mfma_i32_16x16x64_i8 B layout) and the expert's activation rows (A layout, rows
//    past the segment read its last row) straight into registers, then runs the MFMAs;
//  * an item carries two 16-column MFMA tiles: the gate columns n and the up columns
//    n + N/2 for SwiGLU, else columns n and n + 16 (32 KiB or more of weights per item);
//  * the 8 waves' int32 tiles are summed exactly in LDS, then the epilogue writes
//    bf16((f32(acc) * s_m) * sw_n), or f32 silu(g) * u with the same operation sequence as
//    the tiled kernel.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

namespace {
constexpr int kSDW = 8;           // waves per workgroup
constexpr int kSDNT = 16;         // columns per MFMA tile (two tiles per item)
constexpr int kSDMaxSteps = 8;    // 64-deep K steps per wave: K <= 4096
constexpr int kSDMaxExperts = 4096;
}  // namespace

template <int EPI>
__global__ __launch_bounds__(512) void k_seg_decode(TileArgs p) {
  __shared__ int exp_list[kSDMaxExperts];
  __shared__ int nexp;
  __shared__ int red[kSDW][2][4][64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int K = p.K, N = p.N;
  const int ncols = EPI == 2 ? N / 2 : N;  // output columns
  const int KW = K / kSDW, steps = KW >> 6, kbase = wv * KW;
  const int cl = lane & 15, kg = lane >> 4;

  // the experts with 1 <= rows <= kSegSmallRows, in expert order (one wave, shuffle scan)
  if (t < 64) {
    int base = 0;
    for (int e0 = 0; e0 < p.batch; e0 += 64) {
      const int e = e0 + t;
      int take = 0;
      if (e < p.batch) {
        const int64_t rows = p.seg_offsets[e + 1] - p.seg_offsets[e];
        take = rows >= 1 && rows <= kSegSmallRows;
      }
      int incl = take;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (t >= o) incl += u;
      }
      if (take) exp_list[base + incl - 1] = e;
      base += __shfl(incl, 63, 64);
    }
    if (t == 0) nexp = base;
  }
  __syncthreads();
  const int tiles = ncols / (EPI == 2 ? kSDNT : 2 * kSDNT);  // items per expert
  const int col2 = EPI == 2 ? ncols : kSDNT;                  // offset of an item's second tile
  const int items = nexp * tiles;

  // Items are software-pipelined in pairs of register buffers: the loads of the next item
  // are issued right after the MFMAs of the current one, so they stream while the current
  // item's cross-wave sum and epilogue run.
  v4i g0[kSDMaxSteps], u0[kSDMaxSteps], a0[kSDMaxSteps];
  v4i g1[kSDMaxSteps], u1[kSDMaxSteps], a1[kSDMaxSteps];
  auto issue = [&](int item, v4i (&bg)[kSDMaxSteps], v4i (&bu)[kSDMaxSteps], v4i (&a)[kSDMaxSteps]) {
    const int e = exp_list[item / tiles];
    const int n0 = (item - (item / tiles) * tiles) * (EPI == 2 ? kSDNT : 2 * kSDNT);
    const int row0 = (int)p.seg_offsets[e];
    const int rows = (int)p.seg_offsets[e + 1] - row0;
    const int8_t* W = p.w + (int64_t)e * p.w_batch_stride + kbase + kg * 16;
    // rows past the segment read its last row: they only feed output rows not stored
    const int8_t* arow = p.a + (int64_t)(row0 + min(cl, rows - 1)) * p.lda + kbase + kg * 16;
#pragma unroll
    for (int j = 0; j < kSDMaxSteps; ++j) {
      if (j < steps) {
        bg[j] = *reinterpret_cast<const v4i*>(W + (int64_t)(n0 + cl) * K + j * 64);
        bu[j] = *reinterpret_cast<const v4i*>(W + (int64_t)(col2 + n0 + cl) * K + j * 64);
      }
    }
#pragma unroll
    for (int j = 0; j < kSDMaxSteps; ++j)
      if (j < steps) a[j] = *reinterpret_cast<const v4i*>(arow + j * 64);
  };
  auto finish = [&](int item, const v4i (&bg)[kSDMaxSteps], const v4i (&bu)[kSDMaxSteps], const v4i (&a)[kSDMaxSteps],
                    int next, v4i (&ng)[kSDMaxSteps], v4i (&nu)[kSDMaxSteps], v4i (&na)[kSDMaxSteps]) {
    v4i accg = v4i{0, 0, 0, 0}, accu = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kSDMaxSteps; ++j) {
      if (j < steps) {
        accg = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], bg[j], accg, 0, 0, 0);
        accu = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], bu[j], accu, 0, 0, 0);
      }
    }
    if (next < items) issue(next, ng, nu, na);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wv][0][i][lane] = accg[i];
      red[wv][1][i][lane] = accu[i];
    }
    __syncthreads();
    if (EPI == 2 ? t < 256 : true) {
      const int e = exp_list[item / tiles];
      const int n0 = (item - (item / tiles) * tiles) * (EPI == 2 ? kSDNT : 2 * kSDNT);
      const int row0 = (int)p.seg_offsets[e];
      const int rows = (int)p.seg_offsets[e + 1] - row0;
      const int ln = t & 63, i = (t >> 6) & 3, tile = t >> 8;  // tile: which of the item's two (bf16 epilogue)
      const int r = 4 * (ln >> 4) + i, c = ln & 15;  // MFMA 16x16 output: col = lane % 16, row = 4 (lane / 16) + i
      if (r < rows) {
        int vg = 0, vu = 0;
#pragma unroll
        for (int w = 0; w < kSDW; ++w) {
          vg += red[w][tile][i][ln];
          if constexpr (EPI == 2) vu += red[w][1][i][ln];
        }
        const int m = row0 + r;
        const float s = p.a_scale[m];
        const float* wsc = p.w_scale + (int64_t)e * N;
        if constexpr (EPI == 2) {
          const int n = n0 + c;
          const float gv = __fmul_rn(__fmul_rn((float)vg, s), wsc[n]);
          const float uv = __fmul_rn(__fmul_rn((float)vu, s), wsc[n + ncols]);
          const float sg = __fdiv_rn(gv, __fadd_rn(1.0f, exp_fixed(-gv)));
          reinterpret_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = __fmul_rn(sg, uv);
        } else {
          const int n = n0 + tile * kSDNT + c;
          reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * p.ldy + n] =
              (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)vg, s), wsc[n]));
        }
      }
    }
    __syncthreads();  // red is reused by the next item
  };

  int item = blockIdx.x;
  const int stride = gridDim.x;
  if (item < items) issue(item, g0, u0, a0);
  while (item < items) {  // uniform
    finish(item, g0, u0, a0, item + stride, g1, u1, a1);
    item += stride;
    if (item >= items) break;
    finish(item, g1, u1, a1, item + stride, g0, u0, a0);
    item += stride;
  }
}

bool seg_decode_fits(int N, int K, int epilogue, int64_t batch) {
  const int ncols = epilogue == 2 ? N / 2 : N;
  return K % (kSDW * 64) == 0 && K / (kSDW * 64) <= kSDMaxSteps && ncols % (epilogue == 2 ? kSDNT : 2 * kSDNT) == 0 &&
         (epilogue != 2 || N % 2 == 0) && batch <= kSDMaxExperts;
}

hipError_t launch_seg_decode(const TileArgs& a, int num_cu, hipStream_t st) {
  if (!seg_decode_fits(a.N, a.K, a.epilogue, a.batch) || !a.seg_offsets) return hipErrorInvalidValue;
  const dim3 grid((unsigned)num_cu), block(kSDW * 64);  // one persistent workgroup per CU
  if (a.epilogue == 2)
    hipLaunchKernelGGL(k_seg_decode<2>, grid, block, 0, st, a);
  else
    hipLaunchKernelGGL(k_seg_decode<1>, grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace wq
