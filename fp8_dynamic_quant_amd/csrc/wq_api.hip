// Host side of libwq: argument validation, launch-shape selection and the C ABI.
//
// Launch-shape rules (the MI355X counterpart of the host tiling the W8A8 article reads in
// sections 二 and 三: the launch follows the real shape, not a bucket table):
//  * quant: one wave per (row, K slice).  Rows alone give M waves; when that leaves most
//    of the CUs idle (M < CUs / 2, the condition under which the article's arch35 tiling
//    also splits a row along its tail axis) the row is split into S slices with
//    M * S <= CUs, each slice at least 512 elements.
//  * INT8 GEMM, M < 256 with K % 512 == 0 and K <= 4096: the 8-wave decode kernel
//    (k_fused.hip), workgroups of R rows x nt columns, each streaming its columns' whole K,
//    the shape from a cost model (fused_shape); no workgroup talks to another.  Other K at
//    M <= 64: the dot4 GEMV (M <= 4) or the 4-wave decode kernel (k_decode.hip).
//  * INT8 GEMM, M and N >= 256: persistent 256 x 256 tiles (k_gemm_big.hip); other shapes
//    128 x 128 tiles.
//  * FP8: the 16- or 32-column weight-streaming kernels at T <= 64, 128 x 128 tiles above.
#include <algorithm>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/wq.h"
#include "wq_kernels.h"

struct wq_ctx {
  int device;
  int num_cu;
  void* ws;
  size_t ws_bytes;
  int log;
  int force_split;
  int decode_nt;  // 0 = automatic; else 4, 8 or 16 (WQ_DECODE_NT)
  int decode_mt;  // 0 = automatic; else 1, 2 or 4 16-row tiles per workgroup (WQ_DECODE_MT)
  // The fused call quantises inside the GEMM launch up to fused_max_m rows (default 255, the
  // kernel's limit): every workgroup quantises the rows of its own row tile (no workgroup
  // waits for another); above the limit the call runs the quant kernel and then the GEMM
  // (measured at K = 4096, N = 1024: one launch 11.3 / 12.0 / 21.6 us at M = 96 / 128 / 255
  // against 13.9 / 14.7 / 23.0 us for the two launches).
  int seg_small;         // expert segments: small experts on the streaming kernel (WQ_SEG_SMALL=0 turns off)
  int64_t expected_tokens;  // expert segments: default expected rows per expert (WQ_EXPECTED_TOKENS; 0 = none)
  int fp8_rt;            // FP8 decode: 16-token tiles per workgroup (WQ_FP8_RT, 1..4; 0 = automatic)
  int fp8_cols;          // FP8 decode: output columns per workgroup (WQ_FP8_COLS, 16 or 32; default 32)
  int fused_max_m;       // largest M the one-launch fused kernel takes (WQ_FUSED_MAX_M)
  int fused_gemv_max_m;  // largest M the fused GEMV takes instead (WQ_FUSED_GEMV_MAX_M)
  int fused_r;           // one-launch fused kernel: rows per workgroup (WQ_FUSED_R; 0 = automatic)
  int fused_nt;          // one-launch fused kernel: columns per workgroup (WQ_FUSED_NT; 0 = automatic)
  int gq_ppw;            // FP8 group quant: packs per wave (WQ_GQ_PPW, 1, 2, 4 or 8; 0 = automatic)
};

namespace {

constexpr size_t kWsQBytes = 64u << 20;      // INT8 payload staged between two launches
constexpr size_t kWsScaleBytes = 1u << 20;   // its f32 per-row scales
constexpr size_t kWsBytes = kWsQBytes + kWsScaleBytes;
constexpr int kAbiVersion = 3;

inline bool al16(const void* p) { return p == nullptr || (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct DeviceGuard {
  int prev = -1;
  explicit DeviceGuard(int dev) {
    if (hipGetDevice(&prev) == hipSuccess && prev != dev) (void)hipSetDevice(dev);
    else prev = -1;
  }
  ~DeviceGuard() {
    if (prev >= 0) (void)hipSetDevice(prev);
  }
};

int status_of(hipError_t e) { return e == hipSuccess ? WQ_OK : WQ_ERR_DEVICE; }

int8_t* ws_q(wq_ctx* c) { return reinterpret_cast<int8_t*>(c->ws); }
float* ws_scale(wq_ctx* c) { return reinterpret_cast<float*>(reinterpret_cast<char*>(c->ws) + kWsQBytes); }

// Columns per decode workgroup: the narrowest tile (4, 8 or 16) that still gives at
// most two workgroups per CU, so that every CU streams a distinct slice of W.
int decode_nt(const wq_ctx* c, int64_t N) {
  if (c->decode_nt > 0) return c->decode_nt;
  for (int nt : {4, 8}) {
    if ((N + nt - 1) / nt <= 2 * (int64_t)c->num_cu) return nt;
  }
  return 16;
}

// Decode tile shape for M rows: up to 16 rows, one 16-row tile of decode_nt columns.
// Above 16 rows every workgroup would read all M activation rows from L2 for a handful
// of columns, so the rows are split into 16-row tiles (grid y) and the column tile nt is
// the one that moves the fewest bytes per CU: rounds of workgroups per CU times the bytes
// one workgroup reads (16 K activation bytes per row tile + nt K weight bytes); ties go to
// the shape with more workgroups.
void decode_shape(const wq_ctx* c, int64_t M, int64_t N, int* nt, int* mt) {
  *mt = c->decode_mt > 0 ? c->decode_mt : 1;
  if (M <= 16 && c->decode_mt == 0) {
    *nt = decode_nt(c, N);
    return;
  }
  if (c->decode_nt > 0) {
    *nt = c->decode_nt;
    return;
  }
  const int64_t rt = (M + 16 * *mt - 1) / (16 * *mt);
  int64_t best = -1;
  for (int w : {16, 8, 4}) {
    const int64_t wgs = (N + w - 1) / w * rt;
    const int64_t rounds = (wgs + c->num_cu - 1) / c->num_cu;
    const int64_t cost = rounds * (16 * *mt + w);
    if (best < 0 || cost <= best) {
      best = cost;
      *nt = w;
    }
  }
}

int quant_split(const wq_ctx* c, int64_t M, int64_t K) {
  if (c->force_split > 0) return c->force_split;
  if (M <= 0 || M >= c->num_cu / 2) return 1;
  int S = 1;
  while (M * (S * 2) <= c->num_cu && K / (S * 2) >= 512) S *= 2;
  return S;
}

// Shape of the one-launch fused kernel: nt columns and r rows per workgroup.  Every
// workgroup quantises its r rows (VALU time ~ r) and streams nt K weight bytes (the row
// tiles of one column slice share them through their XCD's L2).  The cost of a shape is
// the rounds of workgroups per CU times the per-workgroup time row_cost r + max(nt,
// col_floor).  With the quantisation (col_floor 16) a slice narrower than 16 columns costs
// as much as 16: the kernel's MFMA tile is 16 columns wide, and a narrower slice runs a
// partly used one.  Measured at K = 4096, N = 1024 on 256 CUs over every shape of r in
// 1..16 and nt in 4..32, the pick is the fastest shape or within 0.1 us of it at M = 2, 4,
// 7, 8, 16, 32, 64 for both weight layouts (row_cost 3 on plain weights, 6 on fragment-order
// weights, which stream faster; with the one-fma quantisation, row_cost 4 on plain weights
// picked 4 x 32 at M = 32, 7.23 us against 6.19 for 8 x 16); a linear column cost had picked
// 2 x 8 at M = 4 (4.70 against 4.34 us for 1 x 16) and, on fragment-order weights, 2 x 32 at
// M = 16 (5.29 against 4.85 us for 4 x 16).
// Ties go to the smaller r (a smaller kernel instance: less code, fewer registers); r is
// at most the power of two at or above M.
// row_cost: a row's cost in columns (3 with the quantisation; 6 with fragment-order
// weights; the decode GEMM on given codes passes 1 above M = 16 and 4 below); col_floor: 16
// with the quantisation, 0 (a linear column cost) for the decode GEMM on given codes
void fused_shape(const wq_ctx* c, int64_t M, int64_t N, int* nt, int* r, int row_cost = 3, int col_floor = 16) {
  int64_t best = -1;
  for (int rr : {1, 2, 4, 8, 16}) {
    if (c->fused_r > 0 ? rr != c->fused_r : rr >= 2 * M) continue;
    for (int w : {4, 8, 16, 32}) {
      if (c->fused_nt > 0 && w != c->fused_nt) continue;
      const int64_t wgs = (N + w - 1) / w * ((M + rr - 1) / rr);
      const int64_t rounds = (wgs + c->num_cu - 1) / c->num_cu;
      const int64_t cost = rounds * (row_cost * std::min<int64_t>(rr, M) + std::max(w, col_floor));
      if (best < 0 || cost < best) {
        best = cost;
        *nt = w;
        *r = rr;
      }
    }
  }
}

// The knobs a context reads from the environment once, at creation (include/wq.h).
void read_env_knobs(wq_ctx* c) {
  const char* lg = std::getenv("WQ_LOG");
  c->log = lg && lg[0] == '1';
  const char* fs = std::getenv("WQ_FORCE_SPLIT");
  c->force_split = fs ? std::atoi(fs) : 0;
  const char* dn = std::getenv("WQ_DECODE_NT");
  c->decode_nt = dn ? std::atoi(dn) : 0;
  if (c->decode_nt != 0 && c->decode_nt != 4 && c->decode_nt != 8 && c->decode_nt != 16) c->decode_nt = 0;
  const char* dm = std::getenv("WQ_DECODE_MT");
  c->decode_mt = dm ? std::atoi(dm) : 0;
  if (c->decode_mt != 0 && c->decode_mt != 1 && c->decode_mt != 2 && c->decode_mt != 4) c->decode_mt = 0;
  const char* fm = std::getenv("WQ_FUSED_MAX_M");
  c->fused_max_m = fm ? std::atoi(fm) : 255;
  if (c->fused_max_m < 0 || c->fused_max_m > 255) c->fused_max_m = 255;
  const char* fr = std::getenv("WQ_FP8_RT");
  c->fp8_rt = fr ? std::atoi(fr) : 0;
  const char* fc = std::getenv("WQ_FP8_COLS");
  c->fp8_cols = fc ? std::atoi(fc) : 32;
  if (c->fp8_cols != 16) c->fp8_cols = 32;
  if (c->fp8_rt < 0 || c->fp8_rt > 4) c->fp8_rt = 0;
  const char* ss = std::getenv("WQ_SEG_SMALL");
  c->seg_small = ss ? std::atoi(ss) != 0 : 1;
  const char* et = std::getenv("WQ_EXPECTED_TOKENS");
  c->expected_tokens = et ? std::atoll(et) : 0;
  if (c->expected_tokens < 0) c->expected_tokens = 0;
  const char* gm = std::getenv("WQ_FUSED_GEMV_MAX_M");
  c->fused_gemv_max_m = gm ? std::atoi(gm) : 0;
  if (c->fused_gemv_max_m < 0 || c->fused_gemv_max_m > 4) c->fused_gemv_max_m = 0;
  const char* fr2 = std::getenv("WQ_FUSED_R");
  c->fused_r = fr2 ? std::atoi(fr2) : 0;
  if (c->fused_r != 0 && c->fused_r != 1 && c->fused_r != 2 && c->fused_r != 4 && c->fused_r != 8 && c->fused_r != 16)
    c->fused_r = 0;
  const char* gp = std::getenv("WQ_GQ_PPW");
  c->gq_ppw = gp ? std::atoi(gp) : 0;
  if (c->gq_ppw != 1 && c->gq_ppw != 2 && c->gq_ppw != 4 && c->gq_ppw != 8) c->gq_ppw = 0;
  const char* fn = std::getenv("WQ_FUSED_NT");
  c->fused_nt = fn ? std::atoi(fn) : 0;
  if (c->fused_nt != 0 && c->fused_nt != 4 && c->fused_nt != 8 && c->fused_nt != 16 && c->fused_nt != 32)
    c->fused_nt = 0;
}

}  // namespace

namespace wq {
// (kernel, device) pairs whose limit is raised, in a fixed table (no heap allocation, so the
// allocation-free entry point may use it); once the table is full the attribute is set on
// every launch, which is correct, only slower
hipError_t set_lds_limit(const void* kernel, int bytes) {
  struct Done {
    const void* kernel;
    int device;
  };
  constexpr int kMaxDone = 2048;
  static std::mutex mu;
  static Done done[kMaxDone];
  static int n_done = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  for (int i = 0; i < n_done; ++i)
    if (done[i].kernel == kernel && done[i].device == dev) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && n_done < kMaxDone) done[n_done++] = Done{kernel, dev};
  return e;
}
}  // namespace wq

extern "C" {

const char* wq_status_str(int s) {
  switch (s) {
    case WQ_OK: return "ok";
    case WQ_ERR_NULL: return "a required pointer is NULL";
    case WQ_ERR_SHAPE: return "invalid or unsupported shape";
    case WQ_ERR_ALIGN: return "pointer or leading dimension not 16-byte aligned";
    case WQ_ERR_WORKSPACE: return "workspace missing or too small";
    case WQ_ERR_DEVICE: return "device is not gfx950 or a launch failed";
    case WQ_ERR_UNSUPPORTED: return "unsupported option combination";
    default: return "unknown status";
  }
}

int wq_abi_version(void) { return kAbiVersion; }

size_t wq_workspace_bytes(void) { return kWsBytes; }

int wq_ctx_create(int device, void* workspace, size_t workspace_bytes, wq_ctx** out) {
  if (!out) return WQ_ERR_NULL;
  *out = nullptr;
  if (!workspace) return WQ_ERR_NULL;
  if (workspace_bytes < kWsBytes) return WQ_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return WQ_ERR_ALIGN;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, device) != hipSuccess) return WQ_ERR_DEVICE;
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return WQ_ERR_DEVICE;
  wq_ctx* c = new wq_ctx;
  c->device = device;
  c->num_cu = prop.multiProcessorCount;
  c->ws = workspace;
  c->ws_bytes = workspace_bytes;
  read_env_knobs(c);
  *out = c;
  return WQ_OK;
}

void wq_ctx_destroy(wq_ctx* c) { delete c; }

int wq_ctx_set_split(wq_ctx* c, int n) {
  if (!c) return WQ_ERR_NULL;
  if (n < 0) return WQ_ERR_SHAPE;
  c->force_split = n;
  return WQ_OK;
}

int wq_ctx_set_fused_shape(wq_ctx* c, int rows_per_wg, int cols_per_wg) {
  if (!c) return WQ_ERR_NULL;
  const bool r_ok = rows_per_wg == 0 || rows_per_wg == 1 || rows_per_wg == 2 || rows_per_wg == 4 ||
                    rows_per_wg == 8 || rows_per_wg == 16;
  const bool n_ok = cols_per_wg == 0 || cols_per_wg == 4 || cols_per_wg == 8 || cols_per_wg == 16 || cols_per_wg == 32;
  if (!r_ok || !n_ok) return WQ_ERR_SHAPE;
  c->fused_r = rows_per_wg;
  c->fused_nt = cols_per_wg;
  return WQ_OK;
}

int wq_dynamic_quant(wq_ctx* c, const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                     const void* rms_gamma, float rms_eps, const int32_t* row_index, int8_t* x_q,
                     float* x_scale, void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (x_dtype != WQ_IN_BF16 && x_dtype != WQ_IN_F32) return WQ_ERR_SHAPE;
  if (M < 0 || K < 0 || K % 16 != 0 || K > 131072 || ldx < K) return WQ_ERR_SHAPE;
  if (M == 0 || K == 0) {
    if (M > 0 && K == 0) return WQ_ERR_SHAPE;
    return WQ_OK;
  }
  if (!x || !x_q || !x_scale) return WQ_ERR_NULL;
  const int esz = x_dtype == WQ_IN_F32 ? 4 : 2;
  if (!al16(x) || !al16(x_q) || !al16(rms_gamma) || (ldx * esz) % 16 != 0) return WQ_ERR_ALIGN;
  int S = quant_split(c, M, K);
  const int chunk = 16 / esz;
  if (S < 1 || S > K / chunk) return WQ_ERR_SHAPE;
  DeviceGuard g(c->device);
  int ch = 0;
  hipError_t e = wq::launch_dynamic_quant(x, x_dtype == WQ_IN_F32, M, (int)K, ldx,
                                          static_cast<const uint16_t*>(rms_gamma), rms_eps, row_index, x_q,
                                          x_scale, S, static_cast<hipStream_t>(stream), &ch);
  if (c->log)
    std::fprintf(stderr, "[wq] dynamic_quant M=%lld K=%lld in=%s rms=%d gather=%d split=%d waves=%lld cache=%d\n",
                 (long long)M, (long long)K, esz == 4 ? "f32" : "bf16", rms_gamma != nullptr,
                 row_index != nullptr, S, (long long)(M * S), ch);
  return status_of(e);
}

int wq_group_quant_fp8_ue8m0(wq_ctx* c, const void* x, int64_t T, int64_t G, int64_t D, uint8_t* x_q,
                             int32_t* x_s, void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (T < 0 || G <= 0 || D <= 0 || D % 128 != 0 || G > 65535 || D > (1 << 20)) return WQ_ERR_SHAPE;
  // the kernel indexes waves and packed words in 32 bits
  if ((T + 3) / 4 * 4 * G * ((D / 128 + 3) / 4) >= ((int64_t)1 << 31)) return WQ_ERR_SHAPE;
  if (T == 0) return WQ_OK;
  if (!x || !x_q || !x_s) return WQ_ERR_NULL;
  if (!al16(x) || !al16(x_q) || !al16(x_s)) return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  hipError_t e = wq::launch_group_quant_fp8(static_cast<const uint16_t*>(x), T, (int)G, (int)D, x_q, x_s,
                                            static_cast<hipStream_t>(stream), c->gq_ppw);
  if (c->log)
    std::fprintf(stderr, "[wq] group_quant_fp8 T=%lld G=%lld D=%lld waves=%lld\n", (long long)T, (long long)G,
                 (long long)D, (long long)(((T + 3) / 4 * 4) * G * ((D / 128 + 3) / 4)));
  return status_of(e);
}

int wq_group_quant_mxfp8(wq_ctx* c, const void* x, int64_t T, int64_t G, int64_t D, uint8_t* x_q, int32_t* x_s,
                         void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (T < 0 || G <= 0 || D <= 0 || D % 32 != 0 || G > 65535 || D > (1 << 20)) return WQ_ERR_SHAPE;
  if (T == 0) return WQ_OK;
  if (!x || !x_q || !x_s) return WQ_ERR_NULL;
  if (!al16(x) || !al16(x_q) || !al16(x_s)) return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  hipError_t e = wq::launch_group_quant_mx(static_cast<const uint16_t*>(x), T, (int)G, (int)D, x_q, x_s,
                                           static_cast<hipStream_t>(stream));
  if (c->log)
    std::fprintf(stderr, "[wq] group_quant_mxfp8 T=%lld G=%lld D=%lld\n", (long long)T, (long long)G, (long long)D);
  return status_of(e);
}

static int int8_matmul(wq_ctx* c, const wq_matmul_desc* d, hipStream_t st) {
  const int64_t M = d->M, N = d->N, K = d->K;
  if (N % 16 != 0 || K % 16 != 0 || K > 131072 || d->lda < K || d->ldy < (d->epilogue == WQ_EPI_SWIGLU_F32 ? N / 2 : N))
    return WQ_ERR_SHAPE;
  if (!d->a || !d->a_scale || !d->b || !d->b_scale || !d->y) return WQ_ERR_NULL;
  const int ysz = d->epilogue == WQ_EPI_SWIGLU_F32 ? 4 : 2;
  if (!al16(d->a) || !al16(d->b) || !al16(d->y) || !al16(d->acc_out) || d->lda % 16 != 0 || (d->ldy * ysz) % 16 != 0)
    return WQ_ERR_ALIGN;
  if (d->seg_offsets == nullptr && d->batch != 1) return WQ_ERR_UNSUPPORTED;
  // fragment-order weights: expert segments, or the decode kernel on given codes (dense
  // M <= 64, K % 512 == 0, K <= 4096)
  if (d->b_layout == WQ_LAYOUT_FRAGMENT) {
    if (K % 64 != 0) return WQ_ERR_UNSUPPORTED;
    if (d->seg_offsets == nullptr && (M >= 256 || !wq::given_decode_fits((int)std::max<int64_t>(M, 1), (int)K) ||
                                      d->epilogue != WQ_EPI_BF16))
      return WQ_ERR_UNSUPPORTED;
  }
  if (d->seg_offsets != nullptr) {
    // expert segments: persistent 128x128 tiles over the non-empty (expert, row tile) pairs
    if (!wq::tile_fits((int)K, d->lda) || d->acc_out) return WQ_ERR_UNSUPPORTED;
    if (d->epilogue == WQ_EPI_SWIGLU_F32 && N % 256 != 0) return WQ_ERR_SHAPE;
    if (d->b_batch_stride < N * K) return WQ_ERR_SHAPE;
    if (d->batch > 4096) return WQ_ERR_SHAPE;
    // every expert adds at most one partial row tile: E + ceil(M/128) bounds the
    // (expert, row tile) pairs the persistent kernel lists in LDS
    if (d->batch + (M + 127) / 128 > wq::kSegMaxPairs) return WQ_ERR_UNSUPPORTED;
    wq::TileArgs t{};
    t.a = static_cast<const int8_t*>(d->a);
    t.lda = d->lda;
    t.a_scale = static_cast<const float*>(d->a_scale);
    t.w = static_cast<const int8_t*>(d->b);
    t.w_batch_stride = d->b_batch_stride;
    t.w_scale = d->b_scale;
    t.M = (int)M; t.N = (int)N; t.K = (int)K;
    t.epilogue = d->epilogue;
    t.y = d->y;
    t.ldy = d->ldy;
    t.seg_offsets = d->seg_offsets;
    t.batch = (int)d->batch;
    t.b_frag = d->b_layout == WQ_LAYOUT_FRAGMENT ? 1 : 0;
    // experts with few rows stream their weights through the 16-column kernel; the tiled
    // kernel takes the rest (both read the offsets on the device and skip the other set).
    // The expected-rows hint only chooses which launches run: expecting more than 64 rows
    // per expert, every expert goes to the tiled kernel (no streaming launch); expecting at
    // most 128, the tiled kernel takes 128-row tiles only (no 256-row launch).  Either way
    // every expert's rows are computed, with the same bytes.
    const int64_t hint = d->expected_rows > 0 ? d->expected_rows : c->expected_tokens;
    const bool small = c->seg_small && wq::seg_decode_fits((int)N, (int)K, d->epilogue, d->batch) &&
                       !(hint > 4 * wq::kSegSmallRows);
    t.seg_min_rows = small ? wq::kSegSmallRows + 1 : 0;
    t.seg_tall = hint > 0 && hint <= 128 ? 0 : 1;
    if (small) {
      hipError_t e = wq::launch_seg_decode(t, c->num_cu, st);
      if (e != hipSuccess) return status_of(e);
    }
    hipError_t e = wq::launch_gemm_tile(t, false, st);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul int8 segments E=%lld rows=%lld N=%lld K=%lld epilogue=%s persistent grid=%d "
                   "small-expert kernel=%s 256-row tiles=%s expected rows=%lld\n", (long long)d->batch, (long long)M,
                   (long long)N, (long long)K, d->epilogue == WQ_EPI_SWIGLU_F32 ? "swiglu-f32" : "bf16", 2 * c->num_cu,
                   small ? "yes" : "no", t.seg_tall ? "yes" : "no", (long long)hint);
    return status_of(e);
  }
  if (d->epilogue != WQ_EPI_BF16) return WQ_ERR_UNSUPPORTED;
  // fragment-order weights reach only the decode kernel below (the checks above admit them at
  // M < 256 with given_decode_fits), whatever the decode knobs say: the other kernels read [N, K]
  const bool frag = d->b_layout == WQ_LAYOUT_FRAGMENT;
  wq::DecodeArgs a{};
  a.a = static_cast<const int8_t*>(d->a);
  a.lda = d->lda;
  a.a_scale = static_cast<const float*>(d->a_scale);
  a.w = static_cast<const int8_t*>(d->b);
  a.w_scale = d->b_scale;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.y = static_cast<uint16_t*>(d->y);
  a.ldy = d->ldy;
  a.acc_out = d->acc_out;
  if (M > 64 && M < 256 && wq::given_decode_fits((int)M, (int)K) && ((c->decode_nt == 0 && c->decode_mt == 0) || frag)) {
    // between the decode sizes and the 256-row prefill tiles: the decode kernel on the given
    // codes with row tiles of up to 16 rows (at M = 128, N = 1024 the 128 x 128 tiles gave
    // only 8 workgroups: 41.6 us with the quant)
    int nt = 16, rr = 16;
    fused_shape(c, M, N, &nt, &rr, 1, 0);
    hipError_t e = wq::launch_fused_decode(a, nt, rr, st, frag);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul int8 mid-M (decode kernel, given codes) M=%lld N=%lld K=%lld cols/wg=%d "
                   "rows/wg=%d\n", (long long)M, (long long)N, (long long)K, nt, rr);
    return status_of(e);
  }
  if (M <= 64) {
    // M > 2: the fused decode kernel without its quantisation, the given codes and scales
    // going straight to its tiles (row tiles x column slices; at M <= 2 the dot4 GEMV below
    // measured faster)
    if ((M > 2 || frag) && wq::fused_decode_fits((int)M, (int)K) && ((c->decode_nt == 0 && c->decode_mt == 0) || frag)) {
      // shape: the fused call's model up to M = 16; above, a row without quantisation
      // costs about a column (both measured fastest at K = 4096, N = 1024).  Fragment-order
      // weights (any M <= 64) always take this kernel: it is the decode kernel that reads them
      int nt = 16, rr = 16;
      fused_shape(c, M, N, &nt, &rr, M > 16 ? 1 : 4, 0);
      hipError_t e = wq::launch_fused_decode(a, nt, rr, st, frag);
      if (c->log)
        std::fprintf(stderr, "[wq] quant_matmul int8 decode (fused kernel, given codes) M=%lld N=%lld K=%lld cols/wg=%d "
                     "rows/wg=%d\n", (long long)M, (long long)N, (long long)K, nt, rr);
      return status_of(e);
    }
    // other K.  M <= 4: dense dot4 rows beat the MFMA layout (measured on MI355X; at M = 8
    // the MFMA decode kernel is already faster)
    if (M <= 4 && wq::gemv_fits((int)M, (int)K, false) && c->decode_nt == 0) {
      hipError_t e = wq::launch_gemv(a, st);
      if (c->log)
        std::fprintf(stderr, "[wq] quant_matmul int8 gemv M=%lld N=%lld K=%lld rows/wg=4 grid=%lld\n", (long long)M,
                     (long long)N, (long long)K, (long long)((N + 3) / 4));
      return status_of(e);
    }
    int nt, mt;
    decode_shape(c, M, N, &nt, &mt);
    hipError_t e = wq::launch_decode(a, nt, mt, st);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul int8 decode M=%lld N=%lld K=%lld cols/wg=%d rows/wg=%d grid=%lldx%lld cus=%d\n",
                   (long long)M, (long long)N, (long long)K, nt, 16 * mt, (long long)((N + nt - 1) / nt),
                   (long long)((M + 16 * mt - 1) / (16 * mt)), c->num_cu);
    return status_of(e);
  }
  if (frag) return WQ_ERR_UNSUPPORTED;  // not reached: the branches above take every fragment-order call
  wq::TileArgs t{};
  t.a = static_cast<const int8_t*>(d->a);
  t.lda = d->lda;
  t.a_scale = static_cast<const float*>(d->a_scale);
  t.w = static_cast<const int8_t*>(d->b);
  t.w_batch_stride = d->b_batch_stride;
  t.w_scale = d->b_scale;
  t.M = (int)M; t.N = (int)N; t.K = (int)K;
  t.epilogue = d->epilogue;
  t.y = d->y;
  t.ldy = d->ldy;
  t.acc_out = d->acc_out;
  t.seg_offsets = d->seg_offsets;
  t.batch = (int)d->batch;
  if (wq::big_fits((int)M, (int)N, (int)K, d->lda, d->ldy, d->y, d->acc_out) && c->num_cu % 8 == 0) {
    hipError_t e = wq::launch_gemm_i8_big(t, c->num_cu, st);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul int8 persistent-256 M=%lld N=%lld K=%lld tiles=%lld grid=%d\n",
                   (long long)M, (long long)N, (long long)K, (long long)(((M + 255) / 256) * ((N + 255) / 256)),
                   c->num_cu);
    return status_of(e);
  }
  const bool dma_tiles = wq::tile_fits((int)K, d->lda);
  hipError_t e = dma_tiles ? wq::launch_gemm_tile(t, false, st) : wq::launch_gemm_i8_tile(t, st);
  if (c->log)
    std::fprintf(stderr, "[wq] quant_matmul int8 %s M=%lld N=%lld K=%lld grid=%lld\n",
                 dma_tiles ? "tile128-lds-dma" : "tile128", (long long)M, (long long)N, (long long)K,
                 (long long)(((M + 127) / 128) * ((N + 127) / 128)));
  return status_of(e);
}

static int fp8_matmul(wq_ctx* c, const wq_matmul_desc* d, hipStream_t st) {
  const int64_t M = d->M, N = d->N, K = d->K, G = d->batch;
  if (N % 128 != 0 || K % 128 != 0 || K > 131072 || d->seg_offsets != nullptr || d->epilogue != WQ_EPI_BF16)
    return WQ_ERR_SHAPE;
  if (d->lda < K || d->ldy < N || d->a_batch_stride < 0 || d->y_batch_stride < 0) return WQ_ERR_SHAPE;
  const int64_t TA = (M + 3) / 4 * 4;
  if (d->a_scale_tokens < TA) return WQ_ERR_SHAPE;
  const bool mx = d->payload == WQ_PAYLOAD_MXFP8;
  if (!d->a || !d->a_scale || !d->b || !d->b_scale || !d->y) return WQ_ERR_NULL;
  if (!al16(d->a) || !al16(d->b) || !al16(d->y) || !al16(d->a_scale) || d->lda % 16 != 0 ||
      d->a_batch_stride % 16 != 0 || (d->ldy * 2) % 16 != 0 || (d->y_batch_stride * 2) % 16 != 0 ||
      d->b_batch_stride % 16 != 0)
    return WQ_ERR_ALIGN;
  wq::TileArgs t{};
  t.a = static_cast<const int8_t*>(d->a);
  t.lda = d->lda;
  t.a_batch_stride = d->a_batch_stride;
  t.a_scale_packed = static_cast<const int32_t*>(d->a_scale);
  t.a_scale_tokens = d->a_scale_tokens;
  t.w = static_cast<const int8_t*>(d->b);
  t.w_batch_stride = d->b_batch_stride;
  t.w_scale = d->b_scale;
  t.M = (int)M; t.N = (int)N; t.K = (int)K;
  t.epilogue = WQ_EPI_BF16;
  t.y = d->y;
  t.ldy = d->ldy;
  t.y_batch_stride = d->y_batch_stride;
  t.batch = (int)G;
  t.mx = mx ? 1 : 0;
  if (mx && c->fp8_cols == 32 && wq::fp8_decode32_fits((int)M, (int)N, (int)K)) {
    // MX-like 32-element blocks at 17..64 tokens: the 32-column decode kernel
    hipError_t e = wq::launch_fp8_decode32(t, st, true);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul mxfp8 decode32 M=%lld N=%lld K=%lld groups=%lld\n", (long long)M,
                   (long long)N, (long long)K, (long long)G);
    return status_of(e);
  }
  if (mx && wq::fp8_decode_fits((int)M, (int)N, (int)K)) {
    // MX-like 32-element blocks at decode-sized T: the 16-column decode kernel (larger T:
    // the tiled kernel below)
    hipError_t e = wq::launch_fp8_decode(t, c->fp8_rt > 0 ? c->fp8_rt : 4, st, true);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul mxfp8 decode M=%lld N=%lld K=%lld groups=%lld\n", (long long)M,
                   (long long)N, (long long)K, (long long)G);
    return status_of(e);
  }
  if (!mx && c->fp8_cols == 32 && wq::fp8_decode32_fits((int)M, (int)N, (int)K)) {
    // 17..64 tokens: weight streaming, 32 columns x whole K per workgroup of 8 waves, every
    // token tile in flight at once (T = 64: 22.4 us with 16 columns, 17.3 us with 32)
    hipError_t e = wq::launch_fp8_decode32(t, st);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul fp8 decode32 M=%lld N=%lld K=%lld groups=%lld grid=%lldx%lld\n",
                   (long long)M, (long long)N, (long long)K, (long long)G, (long long)(N / 32), (long long)G);
    return status_of(e);
  }
  if (!mx && wq::fp8_decode_fits((int)M, (int)N, (int)K)) {
    // up to 16 tokens (or K not a multiple of 1024): weight streaming, 16 columns x whole K
    // per workgroup (T = 1: 9.1 us, against 10.1 us with 32 columns)
    // all token tiles in one workgroup: splitting them over more workgroups re-reads the
    // weights (measured at T = 64: 29.5 us whole, 34.4 us in halves, 43.3 us in quarters)
    hipError_t e = wq::launch_fp8_decode(t, c->fp8_rt > 0 ? c->fp8_rt : 4, st);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul fp8 decode M=%lld N=%lld K=%lld groups=%lld grid=%lldx%lld\n",
                   (long long)M, (long long)N, (long long)K, (long long)G, (long long)(N / 16), (long long)G);
    return status_of(e);
  }
  hipError_t e = wq::launch_gemm_tile(t, true, st);
  if (c->log)
    std::fprintf(stderr, "[wq] quant_matmul fp8 tile128-lds-dma M=%lld N=%lld K=%lld groups=%lld grid=%lld\n",
                 (long long)M, (long long)N, (long long)K, (long long)G,
                 (long long)(((M + 127) / 128) * (N / 128) * G));
  return status_of(e);
}

int wq_quant_matmul(wq_ctx* c, const wq_matmul_desc* d, void* stream) {
  if (!c || !d) return WQ_ERR_NULL;
  if (d->M < 0 || d->N <= 0 || d->K <= 0 || d->batch < 1) return WQ_ERR_SHAPE;
  if (d->M > (int64_t)1 << 30 || d->N > (int64_t)1 << 30) return WQ_ERR_SHAPE;
  if (d->epilogue != WQ_EPI_BF16 && d->epilogue != WQ_EPI_SWIGLU_F32) return WQ_ERR_SHAPE;
  if (d->b_layout != WQ_LAYOUT_PLAIN && d->b_layout != WQ_LAYOUT_FRAGMENT) return WQ_ERR_SHAPE;
  if (d->b_layout == WQ_LAYOUT_FRAGMENT && d->payload != WQ_PAYLOAD_INT8) return WQ_ERR_UNSUPPORTED;
  if (d->M == 0) return WQ_OK;
  DeviceGuard g(c->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d->payload == WQ_PAYLOAD_INT8) return int8_matmul(c, d, st);
  if (d->payload == WQ_PAYLOAD_FP8_E4M3 || d->payload == WQ_PAYLOAD_MXFP8) return fp8_matmul(c, d, st);
  return WQ_ERR_SHAPE;
}

namespace {
// the launch sequence of the fused call (valid sizes, M >= 1): see wq_fused_path
int fused_path(const wq_ctx* c, int64_t M, int64_t K) {
  if (M <= c->fused_gemv_max_m && wq::gemv_fits((int)M, (int)K, true)) return 1;
  if (M <= c->fused_max_m && wq::fused_decode_fits((int)M, (int)K)) return 2;
  if (M <= c->fused_max_m && wq::gemv_fits((int)M, (int)K, true)) return 1;  // K the MFMA kernel does not take
  return 0;
}
}  // namespace

int wq_fused_path(const wq_ctx* c, int64_t M, int64_t K, int64_t N) {
  if (!c) return -WQ_ERR_NULL;
  if (M < 1 || K <= 0 || N <= 0 || K % 16 != 0 || N % 16 != 0 || K > 131072) return -WQ_ERR_SHAPE;
  return fused_path(c, M, K);
}

}  // extern "C"

namespace {
// The fused call; when M is above the one-launch limit and the caller exported no payload,
// the payload and its scales are staged in stage_q / stage_s (the context workspace, or the
// static scratch of wq_fused_quant_matmul_static), of the given capacities.
int fused_impl(wq_ctx* c, const void* x, int64_t M, int64_t K, int64_t ldx, const int8_t* w, const float* w_scale,
               int64_t N, void* y, int64_t ldy, int8_t* x_q_out, float* x_scale_out, int32_t* acc_out, void* stream,
               int8_t* stage_q, size_t stage_q_bytes, float* stage_s, size_t stage_s_bytes) {
  if (M < 0 || K <= 0 || N <= 0 || K % 16 != 0 || N % 16 != 0 || K > 131072 || ldx < K || ldy < N)
    return WQ_ERR_SHAPE;
  if (M == 0) return WQ_OK;
  if (!x || !w || !w_scale || !y) return WQ_ERR_NULL;
  if (!al16(x) || !al16(w) || !al16(y) || !al16(x_q_out) || !al16(acc_out) || (ldx * 2) % 16 != 0 ||
      (ldy * 2) % 16 != 0)
    return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int path = fused_path(c, M, K);
  const bool one_launch_gemv = path == 1;
  const bool one_launch_mfma = path == 2;
  if (!one_launch_gemv && !one_launch_mfma) {
    // quantise, then the GEMM (two launches); the INT8 payload goes through the
    // caller's buffers when given, else through the staging buffers
    if (!x_q_out && (size_t)M * K > stage_q_bytes) return WQ_ERR_WORKSPACE;
    if (!x_scale_out && (size_t)M * 4 > stage_s_bytes) return WQ_ERR_WORKSPACE;
    if (!x_q_out) x_q_out = stage_q;
    if (!x_scale_out) x_scale_out = stage_s;
    int r = wq_dynamic_quant(c, x, WQ_IN_BF16, M, K, ldx, nullptr, 0.0f, nullptr, x_q_out, x_scale_out, stream);
    if (r != WQ_OK) return r;
    wq_matmul_desc d{};
    d.payload = WQ_PAYLOAD_INT8; d.epilogue = WQ_EPI_BF16;
    d.M = M; d.N = N; d.K = K; d.batch = 1;
    d.a = x_q_out; d.lda = K; d.a_scale = x_scale_out; d.b = w; d.b_scale = w_scale;
    d.y = y; d.ldy = ldy; d.acc_out = acc_out;
    return wq_quant_matmul(c, &d, stream);
  }
  wq::DecodeArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = ldx;
  a.w = w;
  a.w_scale = w_scale;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.y = static_cast<uint16_t*>(y);
  a.ldy = ldy;
  a.acc_out = acc_out;
  a.xq_out = x_q_out;
  a.xs_out = x_scale_out;
  if (one_launch_gemv) {
    hipError_t e = wq::launch_gemv(a, st);
    if (c->log)
      std::fprintf(stderr, "[wq] fused_quant_matmul gemv M=%lld N=%lld K=%lld rows/wg=4 grid=%lld\n", (long long)M,
                   (long long)N, (long long)K, (long long)((N + 3) / 4));
    return status_of(e);
  }
  int nt = 16, rr = 16;  // fused_shape always sets both: the loops hold every knob value
  fused_shape(c, M, N, &nt, &rr);
  hipError_t e = wq::launch_fused_decode(a, nt, rr, st);
  if (c->log)
    std::fprintf(stderr,
                 "[wq] fused_quant_matmul one launch M=%lld N=%lld K=%lld cols/wg=%d rows/wg=%d grid=%lldx%lld cus=%d\n",
                 (long long)M, (long long)N, (long long)K, nt, rr, (long long)((N + nt - 1) / nt),
                 (long long)((M + rr - 1) / rr), c->num_cu);
  return status_of(e);
}

// The allocation-free variant's staging buffer: the INT8 payload [M, K] (at most
// kScratchQBytes), then its f32 scales [M] (at most kScratchScaleBytes).  One copy per device,
// held until the process ends; host code reaches it only through the address that
// hipGetSymbolAddress returns for the device (static_device).
constexpr size_t kScratchQBytes = 16u << 20;
constexpr size_t kScratchScaleBytes = 64u << 10;
static __device__ __align__(256) int8_t scratch[kScratchQBytes + kScratchScaleBytes];

struct StaticDevice {
  bool ready;
  int num_cu;
  int8_t* scratch;  // this device's address of `scratch`
};
constexpr int kMaxDevices = 64;
StaticDevice g_static[kMaxDevices];
std::mutex g_static_mu;

// First call on a device: with the device current, check it is gfx950, read its CU count and
// the device address of `scratch`; later calls reuse them.
int static_device(int device, StaticDevice* out) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDevice& d = g_static[device];
  if (!d.ready) {
    DeviceGuard g(device);
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, device) != hipSuccess) return WQ_ERR_DEVICE;
    if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) return WQ_ERR_DEVICE;
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return WQ_ERR_DEVICE;
    d.num_cu = prop.multiProcessorCount;
    d.scratch = static_cast<int8_t*>(p);
    d.ready = true;
  }
  *out = d;
  return WQ_OK;
}
}  // namespace

extern "C" {

int wq_fused_quant_matmul(wq_ctx* c, const void* x, int64_t M, int64_t K, int64_t ldx, const int8_t* w,
                          const float* w_scale, int64_t N, void* y, int64_t ldy, int8_t* x_q_out,
                          float* x_scale_out, int32_t* acc_out, void* stream) {
  if (!c) return WQ_ERR_NULL;
  return fused_impl(c, x, M, K, ldx, w, w_scale, N, y, ldy, x_q_out, x_scale_out, acc_out, stream, ws_q(c), kWsQBytes,
                    ws_scale(c), kWsScaleBytes);
}

int wq_fused_quant_matmul_static(int device, const void* x, int64_t M, int64_t K, int64_t ldx, const int8_t* w,
                                 const float* w_scale, int64_t N, void* y, int64_t ldy, int8_t* x_q_out,
                                 float* x_scale_out, int32_t* acc_out, void* stream) {
  int count = 0;
  if (hipGetDeviceCount(&count) != hipSuccess || device < 0 || device >= count || device >= kMaxDevices)
    return WQ_ERR_DEVICE;
  StaticDevice sd;
  const int r = static_device(device, &sd);
  if (r != WQ_OK) return r;
  wq_ctx c{};
  c.device = device;
  c.num_cu = sd.num_cu;
  c.ws = nullptr;
  c.ws_bytes = 0;
  read_env_knobs(&c);
  return fused_impl(&c, x, M, K, ldx, w, w_scale, N, y, ldy, x_q_out, x_scale_out, acc_out, stream, sd.scratch,
                    kScratchQBytes, reinterpret_cast<float*>(sd.scratch + kScratchQBytes), kScratchScaleBytes);
}

int wq_pack_weight_i8(wq_ctx* c, const int8_t* w, int64_t N, int64_t K, int64_t ldw, int8_t* wp, void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (N <= 0 || K <= 0 || N % 16 != 0 || K % 64 != 0 || K > 131072 || N > ((int64_t)1 << 30) || ldw < K)
    return WQ_ERR_SHAPE;
  if (!w || !wp) return WQ_ERR_NULL;
  if (!al16(w) || !al16(wp) || ldw % 16 != 0) return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  return status_of(wq::launch_pack_weight_i8(w, ldw, (int)N, (int)K, wp, static_cast<hipStream_t>(stream)));
}

int wq_fused_quant_matmul_packed(wq_ctx* c, const void* x, int64_t M, int64_t K, int64_t ldx, const int8_t* wp,
                                 const float* w_scale, int64_t N, void* y, int64_t ldy, int8_t* x_q_out,
                                 float* x_scale_out, int32_t* acc_out, void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (M < 0 || K <= 0 || N <= 0 || K % 16 != 0 || N % 16 != 0 || ldx < K || ldy < N) return WQ_ERR_SHAPE;
  if (M == 0) return WQ_OK;
  if (M > c->fused_max_m || !wq::fused_decode_fits((int)M, (int)K)) return WQ_ERR_SHAPE;
  if (!x || !wp || !w_scale || !y) return WQ_ERR_NULL;
  if (!al16(x) || !al16(wp) || !al16(y) || !al16(x_q_out) || !al16(acc_out) || (ldx * 2) % 16 != 0 ||
      (ldy * 2) % 16 != 0)
    return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  wq::DecodeArgs a{};
  a.x = static_cast<const uint16_t*>(x);
  a.ldx = ldx;
  a.w = wp;
  a.w_scale = w_scale;
  a.M = (int)M; a.N = (int)N; a.K = (int)K;
  a.y = static_cast<uint16_t*>(y);
  a.ldy = ldy;
  a.acc_out = acc_out;
  a.xq_out = x_q_out;
  a.xs_out = x_scale_out;
  // fragment-order weights stream faster, so a row of quantisation weighs more against a
  // column: about 6 columns (the shape model above)
  int nt = 16, rr = 16;
  fused_shape(c, M, N, &nt, &rr, 6);
  hipError_t e = wq::launch_fused_decode(a, nt, rr, static_cast<hipStream_t>(stream), true);
  if (c->log)
    std::fprintf(stderr, "[wq] fused_quant_matmul_packed M=%lld N=%lld K=%lld cols/wg=%d rows/wg=%d\n",
                 (long long)M, (long long)N, (long long)K, nt, rr);
  return status_of(e);
}

int wq_moe_sort(wq_ctx* c, const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E, int32_t* perm,
                int32_t* row_token, int64_t* offsets, void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (T < 0 || topk <= 0 || E <= 0 || E > 1024 || T * topk > (int64_t)1 << 28) return WQ_ERR_SHAPE;
  if (!offsets) return WQ_ERR_NULL;
  if (T > 0 && (!topk_ids || !perm || !row_token)) return WQ_ERR_NULL;
  DeviceGuard g(c->device);
  hipError_t e = wq::launch_moe_sort(topk_ids, T, (int)topk, (int)E, perm, row_token, offsets,
                                     static_cast<hipStream_t>(stream));
  if (c->log) std::fprintf(stderr, "[wq] moe_sort T=%lld topk=%lld E=%lld\n", (long long)T, (long long)topk, (long long)E);
  return status_of(e);
}

}  // extern "C"
