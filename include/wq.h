/*
 * wq.h - W8A8 dynamic-quant linear and FP8 per-token-group quant for MI355X (gfx950).
 *
 * The operation (from "DeepSeek-V4 W8A8 性能分析：小 M、NZ 布局与测量方法", section 一):
 * a dense linear Y = X W with X [M, K], W [K, N], Y [M, N], run as BF16 X -> per-token
 * dynamic quant -> INT8 X + per-token f32 scale -> INT8 x INT8 -> INT32 GEMM against
 * per-output-channel-scaled INT8 weights -> BF16 Y.  The FP8 variant (SGLang PR #34277
 * summary, 功能与动机 / 实现拆解) quantises each 128-wide hidden group of each token to
 * E4M3FN with a power-of-two UE8M0 scale, and writes the scales packed 4 per int32 in the
 * [G, ceil((D/128)/4), align4(T)] layout the grouped FP8 contraction reads directly.
 *
 * Conventions for every call:
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library never
 *    allocates, frees or synchronises in these calls: it validates the arguments on the
 *    host, enqueues kernels on `stream` (a hipStream_t passed as void*; NULL = the null
 *    stream) and returns.  Device faults surface at the caller's next synchronisation.
 *  - Weights are stored [N, K] with K contiguous (output-channel rows), the logical
 *    W[K, N] transposed once at load time.
 *  - Every base pointer and every leading dimension times the element size must be a
 *    multiple of 16 bytes (the 16-byte scale-base rule of PR #34277, 实现拆解 item 1);
 *    INT8 GEMMs need K % 16 == 0 and N % 16 == 0; FP8 needs D, K and N multiples of 128.
 *  - On any failed check nothing is written and nothing is launched.
 *  - An empty problem (M == 0 or T == 0) returns WQ_OK with no launch (the wrapper in
 *    PR #34277 launches only when x has elements).
 *  - Outputs are deterministic: the same inputs give the same bytes on every call.
 *  - A context and its workspace serve one stream at a time: calls that overlap on two
 *    streams must use two contexts.
 */
#ifndef WQ_H
#define WQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------------------ */
enum {
  WQ_OK = 0,
  WQ_ERR_NULL = 1,        /* a required pointer is NULL                                  */
  WQ_ERR_SHAPE = 2,       /* negative or inconsistent sizes, unsupported divisibility   */
  WQ_ERR_ALIGN = 3,       /* a base pointer or leading dimension not 16-byte aligned    */
  WQ_ERR_WORKSPACE = 4,   /* workspace missing or smaller than wq_workspace_bytes()     */
  WQ_ERR_DEVICE = 5,      /* not a gfx950 device, or the launch failed                  */
  WQ_ERR_UNSUPPORTED = 6  /* a valid but unimplemented combination of options           */
};

/* input element types */
enum { WQ_IN_BF16 = 1, WQ_IN_F32 = 2 };
/* GEMM payload types */
enum { WQ_PAYLOAD_INT8 = 1, WQ_PAYLOAD_FP8_E4M3 = 2, WQ_PAYLOAD_MXFP8 = 3 };
/* GEMM epilogues */
enum { WQ_EPI_BF16 = 1, WQ_EPI_SWIGLU_F32 = 2 };
/* weight layout of wq_matmul_desc.b: plain [batch][N][K], or the fragment order of
 * wq_pack_weight_i8 applied to each batch (INT8: segments, or dense M < 256) */
enum { WQ_LAYOUT_PLAIN = 0, WQ_LAYOUT_FRAGMENT = 1 };

/* Human-readable text for a status code (static storage). */
const char* wq_status_str(int status);

/* ABI revision of this header (3: wq_matmul_desc.expected_rows). */
int wq_abi_version(void);

/* ---- context ----------------------------------------------------------------------- */
typedef struct wq_ctx wq_ctx;

/* Bytes of device workspace a context needs (a fixed bound, independent of shapes). */
size_t wq_workspace_bytes(void);

/* Create a context for `device`.  `workspace` is caller-owned device memory of at least
 * wq_workspace_bytes() bytes, 256-byte aligned; its contents need no initialisation.  The
 * library uses it only to stage the INT8 payload and scales between the two launches of
 * wq_fused_quant_matmul when M is above the one-launch limit and the caller passed no
 * x_q_out / x_scale_out.  Fails with WQ_ERR_DEVICE if the device is not gfx950.
 * Reads the environment once:
 *   WQ_LOG=1          one line per call describing the chosen launch;
 *   WQ_FORCE_SPLIT=n  the K-split factor of the quant kernel (tests use it to show every
 *                     split gives the same bytes);
 *   WQ_DECODE_NT=n    columns per workgroup of the decode GEMM of wq_quant_matmul (4, 8
 *                     or 16; 0 = auto);
 *   WQ_DECODE_MT=t    16-row tiles per workgroup of the decode GEMM (1, 2 or 4; 0 = auto);
 *   WQ_FUSED_MAX_M=m  the largest M wq_fused_quant_matmul runs as one launch (0..255,
 *                     default 255; 0 = always two launches);
 *   WQ_FUSED_GEMV_MAX_M=m  up to this M (0..4, default 0) that one launch is the dot4
 *                     GEMV kernel rather than the 8-wave MFMA kernel;
 *   WQ_FUSED_R=r, WQ_FUSED_NT=n  rows (1, 2, 4, 8, 16) and columns (4, 8, 16, 32) per
 *                     workgroup of that MFMA kernel (0 = auto; see wq_ctx_set_fused_shape);
 *   WQ_SEG_SMALL=0    expert segments: run every expert on the tiled kernel instead of
 *                     sending the experts with at most 16 rows to the streaming kernel;
 *   WQ_FP8_RT=r       grouped FP8 contraction at T <= 16: 16-token tiles per workgroup
 *                     (1..4; 0 = auto, all of them);
 *   WQ_FP8_COLS=16    grouped FP8 contraction at 16 < T <= 64: keep the 16-column kernel
 *                     instead of the 32-column one (default 32);
 *   WQ_GQ_PPW=p       FP8 group quant: packs of four hidden groups per wave (1, 2, 4 or
 *                     8; 0 = auto by grid size);
 *   WQ_EXPECTED_TOKENS=n  expert segments: the expected rows per expert when a call's
 *                     descriptor gives none (wq_matmul_desc.expected_rows; 0 = no hint).
 * Values out of range fall back to the default.  Every setting gives bit-identical
 * results except WQ_FP8_COLS, which changes the order of the FP8 contraction's f32 sums
 * (4 or 8 partial sums per output; both within the contraction's stated tolerance).  The
 * knobs exist for tests and measurement. */
int wq_ctx_create(int device, void* workspace, size_t workspace_bytes, wq_ctx** out);
void wq_ctx_destroy(wq_ctx* ctx);

/* Force the K-split factor of later quant calls on this context (the same knob as
 * WQ_FORCE_SPLIT); n = 0 restores the automatic choice.  Results are bit-identical for
 * every split; tests use this to show it.  Returns WQ_ERR_SHAPE for n < 0; a split larger
 * than K / 8 (bf16 input) or K / 4 (f32 input), one 16-byte piece of the row per slice,
 * makes later quant calls return WQ_ERR_SHAPE. */
int wq_ctx_set_split(wq_ctx* ctx, int n);

/* Force the shape of the one-launch fused kernel of wq_fused_quant_matmul on this context
 * (the same knobs as WQ_FUSED_R / WQ_FUSED_NT): rows_per_wg rows (1, 2, 4, 8 or 16) and
 * cols_per_wg output columns (4, 8, 16 or 32) per workgroup; 0 restores the automatic
 * choice of that dimension.  Results are bit-identical for every shape; tests use this to
 * show it.  Returns WQ_ERR_SHAPE for other values and changes nothing then. */
int wq_ctx_set_fused_shape(wq_ctx* ctx, int rows_per_wg, int cols_per_wg);

/* ---- per-token dynamic INT8 quantisation --------------------------------------------
 * Follows section 一 of the W8A8 article (npu_dynamic_quant: BF16 X -> INT8 X plus a
 * per-token scale) and section 二 (row-parallel work whose parallelism is capped by the
 * row count; long rows may additionally be split along K over several workgroups).
 * Optionally fuses an RMSNorm in front and a row gather, following "DeepSeek V4 950 低精度
 * 优化全复盘" section 2.3 (RMSNorm fused with quantisation in registers) and section 3.2
 * (rows gathered in expert-sorted order).
 *
 * For output row r (0 <= r < M), with src = row_index ? row_index[r] : r:
 *   v[k]  = x[src, k]                                  (no RMSNorm)
 *   v[k]  = (x[src, k] * inv) * gamma[k],  inv = 1 / sqrt(f32(sum_k x^2 / K) + rms_eps)
 *                                                      (rms_gamma != NULL; sum in f64)
 *   a     = max_k |v[k]|,   x_scale[r] = RN_f32(a / 127)
 *   x_q[r, k] = clamp(rint(RN_f32(v[k] / x_scale[r])), -127, 127)   (0 when a == 0)
 * x: x_dtype WQ_IN_BF16 or WQ_IN_F32, row stride ldx elements (ldx >= K).
 * rms_gamma: NULL or bf16 [K].  row_index: NULL or int32 [M] (values are not checked).
 * x_q: int8 [M, K] contiguous.  x_scale: f32 [M].  K % 16 == 0, K <= 131072. */
int wq_dynamic_quant(wq_ctx* ctx, const void* x, int x_dtype, int64_t M, int64_t K, int64_t ldx,
                     const void* rms_gamma, float rms_eps, const int32_t* row_index,
                     int8_t* x_q, float* x_scale, void* stream);

/* ---- per-token-group FP8 quantisation with packed UE8M0 scales -----------------------
 * Follows the SGLang PR #34277 summary (实现拆解 items 1-2 and the kernel write-logic and
 * wrapper snippets).  x: bf16 [T, G, D] contiguous, D % 128 == 0.  HG = D / 128,
 * PH = ceil(HG / 4), TA = 4 * ceil(T / 4).  For each (t, g, h):
 *   a = max |x[t, g, 128h .. 128h+127]|,  e = max(-127, smallest e with 2^e >= a / 448)
 *   x_q[t, g, 128h + i] = E4M3FN(x * 2^-e), nearest-even       (uint8 [T, G, D])
 *   byte e + 127 goes to byte (h % 4) of int32 word (g * PH + h / 4) * TA + t of x_s
 * x_s: int32 storage [G, PH, TA] (16-byte aligned).  Every byte of x_s not written this
 * way - the tail of the last pack and the token-padding words t in [T, TA) - is written
 * as zero.  The logical [T, G, PH] view has element strides (1, PH * TA, TA).
 * TA * G * PH < 2^31 (WQ_ERR_SHAPE otherwise). */
int wq_group_quant_fp8_ue8m0(wq_ctx* ctx, const void* x, int64_t T, int64_t G, int64_t D,
                             uint8_t* x_q, int32_t* x_s, void* stream);

/* The MX-like variant of "DeepSeek V4 950 低精度优化全复盘", section 2.1: every 32
 * elements share one 8-bit scale, E4M3 values.  Same contract as wq_group_quant_fp8_ue8m0
 * with 32-element groups: D % 32 == 0, HG = D / 32 (so PH = ceil(D / 128)),
 *   a = max |x[t, g, 32h .. 32h+31]|, e = max(-127, smallest e with 2^e >= a / 448),
 *   x_q = E4M3FN(x * 2^-e), byte e + 127 at byte (h % 4) of word (g * PH + h / 4) * TA + t,
 * every other byte of x_s [G, PH, TA] zero.  One pack word holds the four 32-element
 * scales of one 128-deep K block. */
int wq_group_quant_mxfp8(wq_ctx* ctx, const void* x, int64_t T, int64_t G, int64_t D,
                         uint8_t* x_q, int32_t* x_s, void* stream);

/* ---- quantised matmul ---------------------------------------------------------------
 * INT8 (section 一 of the W8A8 article; npu_quant_matmul, and the tuple-reuse path where
 * an upstream producer already gave (x_q, x_scale)):
 *   acc[m, n] = sum_k a[m, k] * b[n, k]                    (exact int32)
 *   y[m, n]   = bf16_RN((f32(acc) * a_scale[m]) * b_scale[n])            (WQ_EPI_BF16)
 * WQ_EPI_SWIGLU_F32 (MoE gate/up, "DeepSeek V4 950" section 2.3): with N = 2I,
 *   g = (f32(acc[m, n]) * a_scale[m]) * b_scale[n],  u likewise for column n + I,
 *   y[m, n] = f32( g / (1 + exp(-g)) * u )  for n < I   (f32 [M, I]; exp is the fixed
 *   f32 sequence: n = rint(x*log2e), Cody-Waite r, degree-7 Taylor Horner, ldexp).
 * Segments (MoE, section 五 of the W8A8 article: group_list = tokens per expert):
 *   batch = E experts and seg_offsets = device int64 [E + 1], non-decreasing, with
 *   seg_offsets[E] == M; rows [seg_offsets[e], seg_offsets[e+1]) use b + e*b_batch_stride
 *   and b_scale + e*N.  Segments need K % 128 == 0, E + ceil(M / 128) <= 4096 and no
 *   acc_out (else WQ_ERR_UNSUPPORTED); WQ_EPI_SWIGLU_F32 is available with segments only
 *   and needs N % 256 == 0 (WQ_ERR_SHAPE otherwise).
 * FP8 (SGLang PR #34277: the grouped contraction that reads the packed scales):
 *   payload WQ_PAYLOAD_FP8_E4M3, batch = G groups, a = E4M3 codes with row stride lda
 *   bytes and group stride a_batch_stride bytes; a_scale = the int32 packed storage
 *   [G, PH, TA] written by wq_group_quant_fp8_ue8m0 with TA = a_scale_tokens; b = E4M3
 *   [G][N][K]; b_scale = f32 powers of two [G][N/128][K/128] (the kernels pass each scale's
 *   exponent field to the matrix unit as its E8M0 scale, so a value that is not a normal
 *   power of two acts as 2^(its biased exponent - 127): its mantissa is ignored, and zero
 *   or a subnormal acts as 2^-127); K <= 131072 (else WQ_ERR_SHAPE);
 *   y[m, g, n] = bf16_RN( sum_kb 2^(e_a(m,g,kb)) * b_scale[g, n/128, kb]
 *                         * sum_{k in block kb} a[m, g, k] * b[g, n, k] )   (f32 accumulate)
 * MX-like 32-element blocks ("DeepSeek V4 950 低精度优化全复盘", section 2.1): payload
 *   WQ_PAYLOAD_MXFP8, as the FP8 payload but a_scale = the storage of wq_group_quant_mxfp8
 *   ([G, K/128, TA]) and b_scale pointing at UE8M0 bytes [G][N][K/32] (not floats);
 *   y[m, g, n] = bf16_RN( sum over 32-deep blocks kb of 2^(e_a(m,g,kb))
 *                         * 2^(b_scale[g, n, kb] - 127) * sum_{k in kb} a[m,g,k] * b[g,n,k] );
 *   any M (decode-sized M on the weight-streaming kernel, larger M on the tiled one).
 * acc_out (INT8 dense only, may be NULL): the raw int32 accumulators [M, N], row stride N. */
typedef struct {
  int32_t payload;         /* WQ_PAYLOAD_INT8, WQ_PAYLOAD_FP8_E4M3 or WQ_PAYLOAD_MXFP8    */
  int32_t epilogue;        /* WQ_EPI_BF16 or WQ_EPI_SWIGLU_F32                            */
  int64_t M, N, K;         /* rows (per batch for strided batches), columns, depth        */
  int64_t batch;           /* 1 = dense; G for FP8 groups; E for segments                 */
  const int64_t* seg_offsets; /* device int64 [batch + 1] for segments, else NULL         */
  const void* a;           /* payload rows                                                */
  int64_t lda;             /* row stride of a in elements (bytes: 1-byte payloads)        */
  int64_t a_batch_stride;  /* elements between batches of a (strided batches)             */
  const void* a_scale;     /* INT8: f32 [M]; FP8: int32 packed storage [batch, PH, TA]    */
  int64_t a_scale_tokens;  /* FP8: TA, the token stride of the packed storage             */
  const void* b;           /* weights [batch][N][K]                                       */
  int64_t b_batch_stride;  /* elements between batches of b                               */
  const float* b_scale;    /* INT8: [batch][N]; FP8: [batch][N/128][K/128]                */
  void* y;                 /* output                                                      */
  int64_t ldy;             /* row stride of y in elements                                 */
  int64_t y_batch_stride;  /* elements between batches of y (strided batches)             */
  int32_t* acc_out;        /* optional raw INT8 accumulators [M, N]                       */
  int32_t b_layout;        /* WQ_LAYOUT_PLAIN, or WQ_LAYOUT_FRAGMENT: the [N][K] weights (of
                              every expert) cast by wq_pack_weight_i8, same b_batch_stride.
                              INT8 only, with seg_offsets, or dense with M < 256,
                              K % 512 == 0, K <= 4096 and WQ_EPI_BF16; other combinations
                              give WQ_ERR_UNSUPPORTED.  Outputs are the same bytes as with
                              the plain layout.                                             */
  int64_t expected_rows;   /* segments: the rows per expert the caller expects (the
                              expected-tokens hint of section 五 of the W8A8 article, which
                              picks the grouped GEMM's tiling from it); 0 = no hint, and the
                              context's WQ_EXPECTED_TOKENS applies.  It selects kernels only:
                              above 64 no expert goes to the 16-row streaming kernel; at
                              most 128, no 256-row tiles (one launch fewer).  Every value
                              gives the same bytes; row counts may differ from it freely.   */
} wq_matmul_desc;

int wq_quant_matmul(wq_ctx* ctx, const wq_matmul_desc* desc, void* stream);

/* ---- fused quant + INT8 GEMM -------------------------------------------------------
 * The whole chain of section 一 of the W8A8 article: per-token quant of the bf16 x [M, K]
 * (row stride ldx), the INT8 GEMM against w [N, K] and the bf16 epilogue.  Outputs are
 * bit-identical to wq_dynamic_quant followed by wq_quant_matmul.  y: bf16 [M, N] row
 * stride ldy.  For M up to the one-launch limit (WQ_FUSED_MAX_M, default 255) one kernel
 * quantises in registers and never writes the INT8 payload to HBM; above it the call runs
 * the quant and the GEMM as two launches, staging the payload in x_q_out / x_scale_out
 * when given, else in the context workspace (WQ_ERR_WORKSPACE if M*K bytes exceed it).
 * The optional outputs export the (x_q, x_scale) tuple and the int32 accumulators so a
 * downstream Linear can reuse them (the tuple-reuse path of section 一). */
int wq_fused_quant_matmul(wq_ctx* ctx, const void* x, int64_t M, int64_t K, int64_t ldx,
                          const int8_t* w, const float* w_scale, int64_t N, void* y, int64_t ldy,
                          int8_t* x_q_out, float* x_scale_out, int32_t* acc_out, void* stream);

/* For callers that cannot allocate device memory: code under HIP graph capture, serving
 * loops that must not allocate, harnesses that forbid it.  wq_fused_quant_matmul with no
 * context and no workspace: `device` is the HIP device index, every other argument and the
 * outputs are those of wq_fused_quant_matmul, bit for bit (the knobs come from the same
 * environment variables, read on every call).  When M is above the one-launch limit and
 * x_q_out / x_scale_out are NULL, the INT8 payload and its scales are staged in a static
 * device buffer of the library instead of a context workspace: at most 16 MiB of payload
 * (M * K bytes) and 16384 scales (M <= 16384); larger calls return WQ_ERR_WORKSPACE and launch
 * nothing.  Each device the library runs on holds that buffer (16 MiB + 64 KiB) until the
 * process ends; the first call on a device looks up its address there, later calls only
 * launch.  The call allocates nothing (no hipMalloc, no hipFree, no host heap).  Calls on one
 * device share the buffer: two such calls that may overlap in time (on different streams, or
 * from different host threads) race and must be serialised by the caller.  WQ_ERR_DEVICE for
 * an invalid or non-gfx950 device. */
int wq_fused_quant_matmul_static(int device, const void* x, int64_t M, int64_t K, int64_t ldx,
                                 const int8_t* w, const float* w_scale, int64_t N, void* y, int64_t ldy,
                                 int8_t* x_q_out, float* x_scale_out, int32_t* acc_out, void* stream);

/* Which launch sequence wq_fused_quant_matmul takes for these sizes on this context:
 * 0 = the quant kernel, then the GEMM (two launches); 1 = one launch of the dot4 GEMV
 * kernel (M <= WQ_FUSED_GEMV_MAX_M, or M <= 4 with a K the MFMA kernel does not take:
 * K % 512 != 0 or 4096 < K <= 8192); 2 = one launch of the 8-wave MFMA kernel
 * (K % 512 == 0, K <= 4096), its rows and columns per workgroup chosen from M and N.
 * A negative value is -status for invalid sizes (M < 1, or K, N as wq_fused_quant_matmul
 * requires).  Host only: no device work. */
int wq_fused_path(const wq_ctx* ctx, int64_t M, int64_t K, int64_t N);

/* ---- weight pre-pack (fragment order) ------------------------------------------------
 * Section 四 of the W8A8 article: the weights are cast once at load time into the layout
 * the matrix unit reads (FRACTAL_NZ there).  The gfx950 form here is fragment order: for
 * the int8 weight w [N, K] (row stride ldw bytes), byte (n, k) goes to
 *   wp[((k/64 * N/4 + n/4) * 4 + (k%64)/16) * 64 + (n%4) * 16 + k%16],
 * so for each 64-deep K step the 4-column blocks follow one another, each 256 bytes as
 * [K quarter 0..3][column 0..3][16 bytes], and the 16 columns x 64 K bytes of one
 * v_mfma_i32_16x16x64_i8 B operand are 1 KiB contiguous in lane order.  wp: int8, N*K
 * bytes, caller-allocated, 16-byte aligned; w 16-byte aligned, ldw % 16 == 0, ldw >= K.
 * N % 16 == 0, K % 64 == 0 (else WQ_ERR_SHAPE).  One device-side permutation on `stream`;
 * w and wp must not overlap. */
int wq_pack_weight_i8(wq_ctx* ctx, const int8_t* w, int64_t N, int64_t K, int64_t ldw, int8_t* wp,
                      void* stream);

/* wq_fused_quant_matmul with the weights in fragment order (wp from wq_pack_weight_i8),
 * same arguments otherwise and bit-identical outputs.  Only the one-launch MFMA path:
 * 1 <= M <= 255 (and M <= WQ_FUSED_MAX_M), K % 512 == 0, K <= 4096, N % 16 == 0; other
 * sizes give WQ_ERR_SHAPE (M = 0 returns WQ_OK with nothing launched). */
int wq_fused_quant_matmul_packed(wq_ctx* ctx, const void* x, int64_t M, int64_t K, int64_t ldx,
                                 const int8_t* wp, const float* w_scale, int64_t N, void* y, int64_t ldy,
                                 int8_t* x_q_out, float* x_scale_out, int32_t* acc_out, void* stream);

/* ---- expert sort (MoE) ---------------------------------------------------------------
 * "DeepSeek V4 950" section 3.2: sort the (token, slot) pairs by expert id before the
 * gather so each expert's rows are contiguous.  topk_ids: int32 [T, topk], values in
 * [0, E).  Outputs: perm int32 [T*topk] (flattened pair index t*topk + slot of each sorted
 * row; stable: ties keep pair order), row_token int32 [T*topk] (= perm / topk),
 * offsets int64 [E + 1] (exclusive prefix sum of rows per expert; the group_list of
 * section 五 of the W8A8 article).  An id outside [0, E) drops its pair: the kept pairs are
 * sorted as above, offsets[E] is their count, and the slots from offsets[E] to T*topk get
 * perm = -1 and row_token = 0, so a gather over all T*topk rows stays in bounds. */
int wq_moe_sort(wq_ctx* ctx, const int32_t* topk_ids, int64_t T, int64_t topk, int64_t E,
                int32_t* perm, int32_t* row_token, int64_t* offsets, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* WQ_H */
