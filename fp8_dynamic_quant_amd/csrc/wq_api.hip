// Host side of libwq: argument validation, launch-shape selection and the C ABI.
//
// Launch-shape rules (the MI355X analogue of the host tiling the W8A8 article reads in
// sections 二 and 三: launch width derived continuously from the real shape, not from a
// bucket table):
//  * quant: one wave per (row, K slice).  Rows alone give M waves; when that leaves most
//    of the CUs idle (M < CUs / 2, the condition under which the article's arch35 tiling
//    also splits a row along its tail axis) the row is split into S slices with
//    M * S <= CUs, each slice at least 512 elements.
//  * INT8 GEMM, M <= 64: split-K.  A workgroup owns 64 columns and a K slice of
//    64 * ksteps; the slice shrinks (down to 256) until the grid covers every CU with a
//    distinct piece of W.
//  * INT8 GEMM, M > 64: 128x128 tiles.
#include <cstdio>
#include <cstdlib>
#include <cstring>
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
};

namespace {

constexpr size_t kWsAccBytes = 16u << 20;  // int32 split-K accumulators
constexpr size_t kWsCntBytes = 64u << 10;  // per-column-block arrival counters
constexpr size_t kWsBytes = kWsAccBytes + kWsCntBytes;
constexpr int kAbiVersion = 1;

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

int32_t* ws_acc(wq_ctx* c) { return reinterpret_cast<int32_t*>(c->ws); }
uint32_t* ws_cnt(wq_ctx* c) { return reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(c->ws) + kWsAccBytes); }

int quant_split(const wq_ctx* c, int64_t M, int64_t K) {
  if (c->force_split > 0) return c->force_split;
  if (M <= 0 || M >= c->num_cu / 2) return 1;
  int S = 1;
  while (M * (S * 2) <= c->num_cu && K / (S * 2) >= 512) S *= 2;
  return S;
}

}  // namespace

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
  const char* lg = std::getenv("WQ_LOG");
  c->log = lg && lg[0] == '1';
  const char* fs = std::getenv("WQ_FORCE_SPLIT");
  c->force_split = fs ? std::atoi(fs) : 0;
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
  if (T == 0) return WQ_OK;
  if (!x || !x_q || !x_s) return WQ_ERR_NULL;
  if (!al16(x) || !al16(x_q) || !al16(x_s)) return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  hipError_t e = wq::launch_group_quant_fp8(static_cast<const uint16_t*>(x), T, (int)G, (int)D, x_q, x_s,
                                            static_cast<hipStream_t>(stream));
  if (c->log)
    std::fprintf(stderr, "[wq] group_quant_fp8 T=%lld G=%lld D=%lld waves=%lld\n", (long long)T, (long long)G,
                 (long long)D, (long long)(((T + 3) / 4 * 4) * G * ((D / 128 + 3) / 4)));
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
  if (d->seg_offsets != nullptr || d->epilogue != WQ_EPI_BF16) return WQ_ERR_UNSUPPORTED;  // see below
  if (M <= 64) {
    wq::SplitKArgs a{};
    a.a = static_cast<const int8_t*>(d->a);
    a.lda = d->lda;
    a.a_scale = static_cast<const float*>(d->a_scale);
    a.w = static_cast<const int8_t*>(d->b);
    a.w_scale = d->b_scale;
    a.M = (int)M; a.N = (int)N; a.K = (int)K;
    a.y = static_cast<uint16_t*>(d->y);
    a.ldy = d->ldy;
    a.acc_out = d->acc_out;
    a.ws_acc = ws_acc(c);
    a.ws_cnt = ws_cnt(c);
    const int64_t nblk = (N + 63) / 64;
    int ksteps = 16;
    if (c->force_split > 0) {
      const int64_t per = (K + c->force_split - 1) / c->force_split;
      ksteps = 1;
      while (ksteps * 64 < per && ksteps < 16) ksteps *= 2;
    } else {
      while (ksteps > 4 && nblk * ((K + 64 * ksteps - 1) / (64 * ksteps)) < c->num_cu) ksteps /= 2;
    }
    a.ksteps = ksteps;
    a.S = (int)((K + 64 * ksteps - 1) / (64 * ksteps));
    if ((size_t)M * N * 4 > kWsAccBytes && a.S > 1) return WQ_ERR_WORKSPACE;
    if (nblk > (int64_t)(kWsCntBytes / 4)) return WQ_ERR_SHAPE;
    hipError_t e = wq::launch_gemm_i8_splitk(a, st);
    if (c->log)
      std::fprintf(stderr, "[wq] quant_matmul int8 splitk M=%lld N=%lld K=%lld kslice=%d S=%d grid=%lld cus=%d\n",
                   (long long)M, (long long)N, (long long)K, 64 * ksteps, a.S, (long long)(nblk * a.S), c->num_cu);
    return status_of(e);
  }
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
  hipError_t e = wq::launch_gemm_i8_tile(t, st);
  if (c->log)
    std::fprintf(stderr, "[wq] quant_matmul int8 tile128 M=%lld N=%lld K=%lld grid=%lld\n", (long long)M,
                 (long long)N, (long long)K, (long long)(((M + 127) / 128) * ((N + 127) / 128)));
  return status_of(e);
}

int wq_quant_matmul(wq_ctx* c, const wq_matmul_desc* d, void* stream) {
  if (!c || !d) return WQ_ERR_NULL;
  if (d->M < 0 || d->N <= 0 || d->K <= 0 || d->batch < 1) return WQ_ERR_SHAPE;
  if (d->M > (int64_t)1 << 30 || d->N > (int64_t)1 << 30) return WQ_ERR_SHAPE;
  if (d->epilogue != WQ_EPI_BF16 && d->epilogue != WQ_EPI_SWIGLU_F32) return WQ_ERR_SHAPE;
  if (d->M == 0) return WQ_OK;
  DeviceGuard g(c->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (d->payload == WQ_PAYLOAD_INT8) return int8_matmul(c, d, st);
  if (d->payload == WQ_PAYLOAD_FP8_E4M3) return WQ_ERR_UNSUPPORTED;
  return WQ_ERR_SHAPE;
}

int wq_fused_quant_matmul(wq_ctx* c, const void* x, int64_t M, int64_t K, int64_t ldx, const int8_t* w,
                          const float* w_scale, int64_t N, void* y, int64_t ldy, int8_t* x_q_out,
                          float* x_scale_out, int32_t* acc_out, void* stream) {
  if (!c) return WQ_ERR_NULL;
  if (M < 0 || K <= 0 || N <= 0 || K % 16 != 0 || N % 16 != 0 || K > 131072 || ldx < K || ldy < N)
    return WQ_ERR_SHAPE;
  if (M == 0) return WQ_OK;
  if (!x || !w || !w_scale || !y) return WQ_ERR_NULL;
  if (!al16(x) || !al16(w) || !al16(y) || !al16(x_q_out) || !al16(acc_out) || (ldx * 2) % 16 != 0 ||
      (ldy * 2) % 16 != 0)
    return WQ_ERR_ALIGN;
  DeviceGuard g(c->device);
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (M > 64) {
    // prefill sizes: the GEMM dominates; run quant then the tiled GEMM (two launches)
    if (!x_q_out || !x_scale_out) return WQ_ERR_UNSUPPORTED;
    int r = wq_dynamic_quant(c, x, WQ_IN_BF16, M, K, ldx, nullptr, 0.0f, nullptr, x_q_out, x_scale_out, stream);
    if (r != WQ_OK) return r;
    wq_matmul_desc d{};
    d.payload = WQ_PAYLOAD_INT8; d.epilogue = WQ_EPI_BF16;
    d.M = M; d.N = N; d.K = K; d.batch = 1;
    d.a = x_q_out; d.lda = K; d.a_scale = x_scale_out; d.b = w; d.b_scale = w_scale;
    d.y = y; d.ldy = ldy; d.acc_out = acc_out;
    return wq_quant_matmul(c, &d, stream);
  }
  wq::SplitKArgs a{};
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
  a.ws_acc = ws_acc(c);
  a.ws_cnt = ws_cnt(c);
  const int64_t nblk = (N + 63) / 64;
  int ksteps = 16;
  if (c->force_split > 0) {
    const int64_t per = (K + c->force_split - 1) / c->force_split;
    ksteps = 1;
    while (ksteps * 64 < per && ksteps < 16) ksteps *= 2;
  } else {
    while (ksteps > 4 && nblk * ((K + 64 * ksteps - 1) / (64 * ksteps)) < c->num_cu) ksteps /= 2;
  }
  a.ksteps = ksteps;
  a.S = (int)((K + 64 * ksteps - 1) / (64 * ksteps));
  if ((size_t)M * N * 4 > kWsAccBytes && a.S > 1) return WQ_ERR_WORKSPACE;
  if (nblk > (int64_t)(kWsCntBytes / 4)) return WQ_ERR_SHAPE;
  hipError_t e = wq::launch_gemm_i8_splitk(a, st);
  if (c->log)
    std::fprintf(stderr, "[wq] fused_quant_matmul M=%lld N=%lld K=%lld kslice=%d S=%d grid=%lld cus=%d\n",
                 (long long)M, (long long)N, (long long)K, 64 * ksteps, a.S, (long long)(nblk * a.S), c->num_cu);
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
