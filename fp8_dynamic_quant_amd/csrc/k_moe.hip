// Expert sort for the MoE block.
//
// Operation: "DeepSeek V4 950 低精度优化全复盘", section 3.2: sort the (token, slot)
// pairs by expert id before the gather, so each expert's rows are contiguous; the
// per-expert row counts become the group_list of the grouped GEMM ("DeepSeek-V4 W8A8
// 性能分析", section 五).
//
// One workgroup of 16 waves does a stable counting sort.  Wave w owns a contiguous chunk
// of the pairs.  Pass 1: per-wave histograms in LDS.  Pass 2: an exclusive scan over
// (expert, wave) in expert-major order gives each wave the first output slot of each
// expert (each wave scans a block of it, then adds the earlier blocks' totals).  Pass 3:
// each wave walks its chunk 64 pairs at a time in order; lanes holding the same id find
// each other with one ballot per id bit, so a lane's rank among equal ids is the popcount
// of the lower matching lanes - the pair order is kept.
#include "wq_device.h"
#include "wq_kernels.h"

namespace wq {

constexpr int kSortWaves = 16;
constexpr int kSortMaxE = 1024;

__global__ __launch_bounds__(1024) void k_moe_sort(const int32_t* __restrict__ ids, int n, int topk, int E,
                                                   int32_t* __restrict__ perm, int32_t* __restrict__ row_token,
                                                   int64_t* __restrict__ offsets) {
  __shared__ int cnt[kSortMaxE * kSortWaves];  // [e][w]
  __shared__ int blk_total[kSortWaves];         // the scan's per-wave block totals
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  for (int i = t; i < E * kSortWaves; i += 1024) cnt[i] = 0;
  __syncthreads();
  const int chunk = (n + kSortWaves - 1) / kSortWaves;
  const int lo = w * chunk, hi = min(n, lo + chunk);
  for (int i = lo + lane; i < hi; i += 64) {
    const int id = ids[i];
    if (id >= 0 && id < E) atomicAdd(&cnt[id * kSortWaves + w], 1);
  }
  __syncthreads();
  // exclusive scan over cnt in (e, w) order, in two levels: each wave scans its own
  // contiguous block of whole 64-entry chunks (a serial chain of total / 1024 chunks rather
  // than total / 64), then adds the totals of the blocks before it
  {
    const int total = E * kSortWaves;
    const int per = ((total + kSortWaves - 1) / kSortWaves + 63) & ~63;
    const int b0 = w * per, b1 = min(total, b0 + per);
    int carry = 0;
    for (int base = b0; base < b1; base += 64) {
      const int i = base + lane;
      const int v = (i < b1) ? cnt[i] : 0;
      int incl = v;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int u = __shfl_up(incl, o, 64);
        if (lane >= o) incl += u;
      }
      if (i < b1) cnt[i] = carry + incl - v;
      carry += __shfl(incl, 63, 64);
    }
    if (lane == 0) blk_total[w] = carry;
    __syncthreads();
    int off = 0;
    for (int j = 0; j < w; ++j) off += blk_total[j];
    for (int i = b0 + lane; i < b1; i += 64) cnt[i] += off;
  }
  __syncthreads();
  // ids outside [0, E) are dropped: offsets[E] counts the kept rows, and the slots past them
  // get perm = -1 and row_token = 0 (a valid token), so a gather over all T * topk rows reads
  // only valid memory
  int kept = 0;
  for (int j = 0; j < kSortWaves; ++j) kept += blk_total[j];
  for (int e = t; e <= E; e += 1024) offsets[e] = (e < E) ? (int64_t)cnt[e * kSortWaves] : (int64_t)kept;
  for (int i = kept + t; i < n; i += 1024) {
    perm[i] = -1;
    row_token[i] = 0;
  }
  __syncthreads();
  // stable scatter
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  for (int base = lo; base < hi; base += 64) {
    const int i = base + lane;
    int id = i < hi ? ids[i] : -1;
    const bool valid = id >= 0 && id < E;  // out-of-range ids are dropped
    if (!valid) id = 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const uint64_t ones = __ballot(valid && ((id >> b) & 1));
      peers &= ((id >> b) & 1) ? ones : ~ones;
    }
    if (valid) {
      const uint64_t lower = peers & ((1ull << lane) - 1ull);
      const int rank = __popcll(lower);
      const int pos = cnt[id * kSortWaves + w] + rank;
      perm[pos] = i;
      row_token[pos] = i / topk;
    }
    // the lowest lane of each peer group advances that expert's slot; only this wave
    // touches column w of cnt, and its LDS accesses complete in program order
    __builtin_amdgcn_wave_barrier();
    if (valid && (peers & ((1ull << lane) - 1ull)) == 0) cnt[id * kSortWaves + w] += __popcll(peers);
    __builtin_amdgcn_wave_barrier();
  }
}

hipError_t launch_moe_sort(const int32_t* ids, int64_t T, int topk, int E, int32_t* perm, int32_t* row_token,
                           int64_t* offsets, hipStream_t st) {
  if (E > kSortMaxE) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_moe_sort, dim3(1), dim3(1024), 0, st, ids, (int)(T * topk), topk, E, perm, row_token,
                     offsets);
  return hipGetLastError();
}

}  // namespace wq
