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

// PK: each expert's weights in fragment order (launch_pack_weight_i8): the 16 columns x 64
// K bytes of one B operand are then 1 KiB contiguous
template <int EPI, int STEPS, bool PK>
__global__ __launch_bounds__(512) void k_seg_decode(TileArgs p) {
  __shared__ int exp_list[kSDMaxExperts];  // listed expert: id | rows << 16
  __shared__ int exp_row0[kSDMaxExperts];  // its first row
  __shared__ int nexp;
  __shared__ int red[kSDW][2][4][64];
  const int t = threadIdx.x, lane = t & 63, wv = t >> 6;
  const int K = p.K, N = p.N;
  const int ncols = EPI == 2 ? N / 2 : N;  // output columns
  const int KW = STEPS * 64, kbase = wv * KW;  // K = 8 waves x STEPS 64-deep steps
  const int cl = lane & 15, kg = lane >> 4;

  // the experts with 1 <= rows <= kSegSmallRows, in expert order (one wave, shuffle scan),
  // with their first rows and row counts, so items read them from LDS, not global memory
  if (t < 64) {
    int base = 0;
    for (int e0 = 0; e0 < p.batch; e0 += 64) {
      const int e = e0 + t;
      int take = 0, rows = 0, row0 = 0;
      if (e < p.batch) {
        row0 = (int)p.seg_offsets[e];
        rows = (int)(p.seg_offsets[e + 1] - p.seg_offsets[e]);
        take = rows >= 1 && rows <= kSegSmallRows;
      }
      int incl = take;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (t >= o) incl += u;
      }
      if (take) {
        exp_list[base + incl - 1] = e | (rows << 16);
        exp_row0[base + incl - 1] = row0;
      }
      base += __shfl(incl, 63, 64);
    }
    if (t == 0) nexp = base;
  }
  __syncthreads();
  const int tiles = ncols / (EPI == 2 ? kSDNT : 2 * kSDNT);  // items per expert
  const int col2 = EPI == 2 ? ncols : kSDNT;                  // offset of an item's second tile
  const int items = nexp * tiles;

  // this thread's output in an item's epilogue: MFMA 16x16 output row r, column c of tile
  // `otile` (col = lane % 16, row = 4 (lane / 16) + i)
  const int oi = (t >> 6) & 3, otile = t >> 8;
  const int orow = 4 * (lane >> 4) + oi, ocol = lane & 15;
  struct Item {
    int e, rows, row0, n0;
  };
  auto item_of = [&](int item) {
    const int x = item / tiles;
    const int info = exp_list[x];
    Item it;
    it.e = info & 0xFFFF;
    it.rows = info >> 16;
    it.row0 = exp_row0[x];
    it.n0 = (item - x * tiles) * (EPI == 2 ? kSDNT : 2 * kSDNT);
    return it;
  };

  // Items are software-pipelined in pairs of register buffers: the loads of the next item
  // (weights, activation rows and this thread's epilogue scales) are issued right after the
  // MFMAs of the current one, so they stream while the current item's cross-wave sum and
  // epilogue run.  No load sits under a branch (the step count is a template parameter, and
  // rows past the segment read clamped addresses whose values go unused), and the epilogue
  // reads no global memory: a load waited for there would also wait for the next item's.
  v4i g0[STEPS], u0[STEPS], a0[STEPS];
  v4i g1[STEPS], u1[STEPS], a1[STEPS];
  float sc0[3], sc1[3];  // s_m, sw_n (gate), sw_n (up)
  auto issue = [&](int item, v4i (&bg)[STEPS], v4i (&bu)[STEPS], v4i (&a)[STEPS], float (&sc)[3]) {
    const Item it = item_of(item);
    // rows past the segment read its last row: they only feed output rows not stored
    const int8_t* arow = p.a + (int64_t)(it.row0 + min(cl, it.rows - 1)) * p.lda + kbase + kg * 16;
    if constexpr (PK) {
      // byte (n, k) at ((k/64 * N/4 + n/4) * 4 + (k%64)/16) * 64 + (n%4) * 16 + k%16
      const int8_t* We = p.w + (int64_t)it.e * p.w_batch_stride + (int64_t)(kbase >> 6) * (N >> 2) * 256 + kg * 64;
      const int ngt = it.n0 + cl, nup = col2 + it.n0 + cl;
      const int8_t* Wg = We + (ngt >> 2) * 256 + (ngt & 3) * 16;
      const int8_t* Wu = We + (nup >> 2) * 256 + (nup & 3) * 16;
      // streaming loads: each expert's weights are read once per call, in whole 1 KiB
      // pieces, so they need no place in L2 (the activation rows, read by every item of the
      // expert, keep theirs); measured 574 -> 539 us (gate/up) and 299 -> 277 us (down) per
      // MoE block.  The plain layout below reads 64 of a line's 128 bytes per step and
      // the other 64 one step later, so it keeps ordinary loads
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        bg[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(Wg + (int64_t)j * N * 64));
        bu[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(Wu + (int64_t)j * N * 64));
      }
    } else {
      const int8_t* W = p.w + (int64_t)it.e * p.w_batch_stride + kbase + kg * 16;
#pragma unroll
      for (int j = 0; j < STEPS; ++j) {
        bg[j] = *reinterpret_cast<const v4i*>(W + (int64_t)(it.n0 + cl) * K + j * 64);
        bu[j] = *reinterpret_cast<const v4i*>(W + (int64_t)(col2 + it.n0 + cl) * K + j * 64);
      }
    }
#pragma unroll
    for (int j = 0; j < STEPS; ++j) a[j] = *reinterpret_cast<const v4i*>(arow + j * 64);
    const float* wsc = p.w_scale + (int64_t)it.e * N;
    sc[0] = p.a_scale[it.row0 + min(orow, it.rows - 1)];
    if constexpr (EPI == 2) {
      sc[1] = wsc[it.n0 + ocol];
      sc[2] = wsc[it.n0 + ocol + ncols];
    } else {
      sc[1] = wsc[it.n0 + otile * kSDNT + ocol];
      sc[2] = 0.0f;
    }
  };
  auto finish = [&](int item, const v4i (&bg)[STEPS], const v4i (&bu)[STEPS], const v4i (&a)[STEPS],
                    const float (&sc)[3], int next, v4i (&ng)[STEPS], v4i (&nu)[STEPS], v4i (&na)[STEPS],
                    float (&nsc)[3]) {
    v4i accg = v4i{0, 0, 0, 0}, accu = v4i{0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < STEPS; ++j) {
      accg = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], bg[j], accg, 0, 0, 0);
      accu = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[j], bu[j], accu, 0, 0, 0);
    }
    // unconditional (past the last item it reloads the last one, unused): under a branch,
    // the waits for this item's epilogue scales would also wait for the next item's loads
    issue(min(next, items - 1), ng, nu, na, nsc);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      red[wv][0][i][lane] = accg[i];
      red[wv][1][i][lane] = accu[i];
    }
    lds_barrier();  // the next item's loads stay in flight through the epilogue
    if (EPI == 2 ? t < 256 : true) {
      const Item it = item_of(item);
      if (orow < it.rows) {
        int vg = 0, vu = 0;
#pragma unroll
        for (int w = 0; w < kSDW; ++w) {
          vg += red[w][otile][oi][lane];
          if constexpr (EPI == 2) vu += red[w][1][oi][lane];
        }
        const int m = it.row0 + orow;
        if constexpr (EPI == 2) {
          const int n = it.n0 + ocol;
          const float gv = __fmul_rn(__fmul_rn((float)vg, sc[0]), sc[1]);
          const float uv = __fmul_rn(__fmul_rn((float)vu, sc[0]), sc[2]);
          const float sg = __fdiv_rn(gv, __fadd_rn(1.0f, exp_fixed(-gv)));
          reinterpret_cast<float*>(p.y)[(int64_t)m * p.ldy + n] = __fmul_rn(sg, uv);
        } else {
          const int n = it.n0 + otile * kSDNT + ocol;
          reinterpret_cast<uint16_t*>(p.y)[(int64_t)m * p.ldy + n] =
              (uint16_t)f32_to_bf16_rn(__fmul_rn(__fmul_rn((float)vg, sc[0]), sc[1]));
        }
      }
    }
    lds_barrier();  // red is reused by the next item
  };

  int item = blockIdx.x;
  const int stride = gridDim.x;
  if (item < items) issue(item, g0, u0, a0, sc0);
  while (item < items) {  // uniform
    finish(item, g0, u0, a0, sc0, item + stride, g1, u1, a1, sc1);
    item += stride;
    if (item >= items) break;
    finish(item, g1, u1, a1, sc1, item + stride, g0, u0, a0, sc0);
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
  const int steps = a.K / (kSDW * 64);
  // persistent workgroups, one per CU: with two per CU where the registers allow it (up to
  // 4 steps per wave), the down projection of the MoE block (K = 2048) measured slower,
  // 278.5 against 267.9 us on fragment-order experts
  const dim3 grid((unsigned)num_cu), block(kSDW * 64);
#define WQ_SEG_CASE(S)                                                                         \
  case S:                                                                                      \
    if (a.epilogue == 2 && a.b_frag)                                                           \
      hipLaunchKernelGGL((k_seg_decode<2, S, true>), grid, block, 0, st, a);                   \
    else if (a.epilogue == 2)                                                                  \
      hipLaunchKernelGGL((k_seg_decode<2, S, false>), grid, block, 0, st, a);                  \
    else if (a.b_frag)                                                                         \
      hipLaunchKernelGGL((k_seg_decode<1, S, true>), grid, block, 0, st, a);                   \
    else                                                                                       \
      hipLaunchKernelGGL((k_seg_decode<1, S, false>), grid, block, 0, st, a);                  \
    break;
  switch (steps) {
    WQ_SEG_CASE(1)
    WQ_SEG_CASE(2)
    WQ_SEG_CASE(3)
    WQ_SEG_CASE(4)
    WQ_SEG_CASE(5)
    WQ_SEG_CASE(6)
    WQ_SEG_CASE(7)
    WQ_SEG_CASE(8)
    default: return hipErrorInvalidValue;
  }
#undef WQ_SEG_CASE
  return hipGetLastError();
}

}  // namespace wq
