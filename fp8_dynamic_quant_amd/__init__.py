"""Python binding for libwq: the W8A8 dynamic-quant linear and the FP8 per-token-group
quant with packed UE8M0 scales, hand-written for MI355X (gfx950).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI in
``include/wq.h``; PyTorch supplies device memory and the current stream.  There is no
fallback: if libwq.so is missing or the device is not gfx950, calls raise.

The functions carry the C names:
  wq_dynamic_quant(x, ...)                -> (x_q int8 [M,K], x_scale f32 [M])
  wq_group_quant_fp8_ue8m0(x)             -> (x_q uint8 [T,G,D], x_s int32 view [T,G,PH], storage [G,PH,TA])
  wq_quant_matmul(a, a_scale, b, b_scale) -> y bf16 [M,N]   (INT8 dense / segments, FP8 groups)
  wq_fused_quant_matmul(x, w, w_scale)    -> y bf16 [M,N]
  wq_moe_sort(ids, E)                     -> (perm, row_token, offsets)
"""

from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwq.so")

WQ_OK = 0
WQ_IN_BF16, WQ_IN_F32 = 1, 2
WQ_PAYLOAD_INT8, WQ_PAYLOAD_FP8_E4M3, WQ_PAYLOAD_MXFP8 = 1, 2, 3
WQ_EPI_BF16, WQ_EPI_SWIGLU_F32 = 1, 2
WQ_LAYOUT_PLAIN, WQ_LAYOUT_FRAGMENT = 0, 1

_c_void_p = ctypes.c_void_p
_i64 = ctypes.c_int64


class WqError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: status {status} ({lib().wq_status_str(status).decode()})")
        self.status = status


class MatmulDesc(ctypes.Structure):
    _fields_ = [
        ("payload", ctypes.c_int32), ("epilogue", ctypes.c_int32),
        ("M", _i64), ("N", _i64), ("K", _i64), ("batch", _i64),
        ("seg_offsets", _c_void_p),
        ("a", _c_void_p), ("lda", _i64), ("a_batch_stride", _i64),
        ("a_scale", _c_void_p), ("a_scale_tokens", _i64),
        ("b", _c_void_p), ("b_batch_stride", _i64),
        ("b_scale", _c_void_p),
        ("y", _c_void_p), ("ldy", _i64), ("y_batch_stride", _i64),
        ("acc_out", _c_void_p),
        ("b_layout", ctypes.c_int32),
        ("expected_rows", _i64),
    ]


EXPORTS = {
    "wq_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "wq_abi_version": (ctypes.c_int, []),
    "wq_workspace_bytes": (ctypes.c_size_t, []),
    "wq_ctx_create": (ctypes.c_int, [ctypes.c_int, _c_void_p, ctypes.c_size_t, ctypes.POINTER(_c_void_p)]),
    "wq_ctx_destroy": (None, [_c_void_p]),
    "wq_ctx_set_split": (ctypes.c_int, [_c_void_p, ctypes.c_int]),
    "wq_ctx_set_fused_shape": (ctypes.c_int, [_c_void_p, ctypes.c_int, ctypes.c_int]),
    "wq_dynamic_quant": (ctypes.c_int, [_c_void_p, _c_void_p, ctypes.c_int, _i64, _i64, _i64, _c_void_p,
                                        ctypes.c_float, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "wq_group_quant_fp8_ue8m0": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                                _c_void_p]),
    "wq_quant_matmul": (ctypes.c_int, [_c_void_p, ctypes.POINTER(MatmulDesc), _c_void_p]),
    "wq_fused_quant_matmul": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _i64,
                                             _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p, _c_void_p]),
    "wq_moe_sort": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p, _c_void_p,
                                   _c_void_p]),
    "wq_fused_path": (ctypes.c_int, [_c_void_p, _i64, _i64, _i64]),
    "wq_group_quant_mxfp8": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                            _c_void_p]),
    "wq_pack_weight_i8": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p]),
    "wq_fused_quant_matmul_packed": (ctypes.c_int, [_c_void_p, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                                    _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p,
                                                    _c_void_p]),
    "wq_fused_quant_matmul_static": (ctypes.c_int, [ctypes.c_int, _c_void_p, _i64, _i64, _i64, _c_void_p, _c_void_p,
                                                    _i64, _c_void_p, _i64, _c_void_p, _c_void_p, _c_void_p,
                                                    _c_void_p]),
}

_LIB = None


def lib() -> ctypes.CDLL:
    """Load libwq.so (built by fp8_dynamic_quant_amd.build); raise if it is missing."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m fp8_dynamic_quant_amd.build` first")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in EXPORTS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _LIB = L
    return _LIB


class Context:
    """One libwq context per device; owns its zero-initialised workspace tensor."""

    def __init__(self, device: torch.device):
        L = lib()
        self.device = device
        self.workspace = torch.zeros(int(L.wq_workspace_bytes()), dtype=torch.uint8, device=device)
        h = _c_void_p()
        st = L.wq_ctx_create(device.index, self.workspace.data_ptr(), self.workspace.numel(), ctypes.byref(h))
        if st != WQ_OK:
            raise WqError("wq_ctx_create", st)
        self.handle = h

    def __del__(self):
        try:
            if self.handle:
                lib().wq_ctx_destroy(self.handle)
        except Exception:
            pass


_CTX: dict[int, Context] = {}


def set_split(device, n: int) -> None:
    """Force the K-split factor of later calls on `device` (0 = automatic)."""
    _check("wq_ctx_set_split", lib().wq_ctx_set_split(context(device).handle, int(n)))


def set_fused_shape(device, rows_per_wg: int, cols_per_wg: int) -> None:
    """Force the one-launch fused kernel's rows and columns per workgroup on `device` (0 = automatic)."""
    _check("wq_ctx_set_fused_shape",
           lib().wq_ctx_set_fused_shape(context(device).handle, int(rows_per_wg), int(cols_per_wg)))


def context(device) -> Context:
    device = torch.device(device)
    if device.type != "cuda":
        raise RuntimeError("libwq runs on the GPU only; got a tensor on " + str(device))
    idx = device.index if device.index is not None else torch.cuda.current_device()
    if idx not in _CTX:
        _CTX[idx] = Context(torch.device("cuda", idx))
    return _CTX[idx]


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t):
    return None if t is None else t.data_ptr()


def _check(fn, st):
    if st != WQ_OK:
        raise WqError(fn, st)


# ------------------------------------------------------------------------------------


def wq_dynamic_quant(x: torch.Tensor, rms_gamma: torch.Tensor | None = None, rms_eps: float = 1e-6,
                     row_index: torch.Tensor | None = None, x_q: torch.Tensor | None = None,
                     x_scale: torch.Tensor | None = None):
    """Per-token INT8 quant of x [*, K] (bf16 or f32, unit stride along K).  With
    row_index, output row r reads input row row_index[r]; with rms_gamma an RMSNorm runs
    first.  Returns (x_q int8 [M, K], x_scale f32 [M])."""
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be 2-D with unit stride along K")
    if x.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("x must be bf16 or f32")
    M = row_index.numel() if row_index is not None else x.shape[0]
    K = x.shape[1]
    ctx = context(x.device)
    if x_q is None:
        x_q = torch.empty((M, K), dtype=torch.int8, device=x.device)
    if x_scale is None:
        x_scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    st = lib().wq_dynamic_quant(ctx.handle, _ptr(x), WQ_IN_F32 if x.dtype == torch.float32 else WQ_IN_BF16, M, K,
                                x.stride(0), _ptr(rms_gamma), float(rms_eps), _ptr(row_index), _ptr(x_q),
                                _ptr(x_scale), _stream(x.device))
    _check("wq_dynamic_quant", st)
    return x_q, x_scale


def packed_scale_dims(T: int, D: int, group: int = 128):
    HG = D // group
    return HG, (HG + 3) // 4, (T + 3) // 4 * 4


def wq_group_quant_fp8_ue8m0(x: torch.Tensor, x_q: torch.Tensor | None = None, storage: torch.Tensor | None = None,
                             group: int = 128):
    """x bf16 [T, G, D] contiguous -> (x_q uint8 [T, G, D] E4M3FN codes,
    x_s int32 logical view [T, G, PH] with strides (1, PH*TA, TA), storage [G, PH, TA]).
    x_q / storage may be passed in (contiguous, those shapes) instead of allocated.
    group=32: the MX-like 32-element blocks (wq_group_quant_mxfp8)."""
    if x.dim() != 3 or not x.is_contiguous() or x.dtype != torch.bfloat16:
        raise ValueError("x must be a contiguous bf16 [T, G, D] tensor")
    if group not in (128, 32):
        raise ValueError("group must be 128 or 32")
    T, G, D = x.shape
    _, PH, TA = packed_scale_dims(T, D, group)
    ctx = context(x.device)
    if x_q is None:
        x_q = torch.empty((T, G, D), dtype=torch.uint8, device=x.device)
    if storage is None:
        storage = torch.empty((G, PH, TA), dtype=torch.int32, device=x.device)
    if tuple(x_q.shape) != (T, G, D) or not x_q.is_contiguous() or tuple(storage.shape) != (G, PH, TA) \
            or not storage.is_contiguous() or storage.dtype != torch.int32:
        raise ValueError("x_q must be uint8 [T, G, D] and storage int32 [G, PH, TA], both contiguous")
    if x.numel() > 0:
        fn = "wq_group_quant_fp8_ue8m0" if group == 128 else "wq_group_quant_mxfp8"
        st = getattr(lib(), fn)(ctx.handle, _ptr(x), T, G, D, _ptr(x_q), _ptr(storage), _stream(x.device))
        _check(fn, st)
    x_s = storage.transpose(-1, -2)[:, :T, :].transpose(0, 1)
    return x_q, x_s, storage


def wq_quant_matmul(a, a_scale, b, b_scale, *, y=None, acc_out=None, seg_offsets=None,
                    epilogue=WQ_EPI_BF16, fp8_groups=None, a_scale_tokens=0, b_fragment=False, n=None,
                    mx=False, expected_rows=0):
    """INT8: a int8 [M, K] (row stride a.stride(0)), a_scale f32 [M], b int8 [N, K] (or
    [E, N, K] with seg_offsets int64 [E+1]), b_scale f32 [N] (or [E, N]) -> y.
    FP8 (fp8_groups=G): a uint8 [M, G, K], a_scale = packed storage [G, PH, TA],
    b uint8 [G, N, K], b_scale f32 [G, N/128, K/128] -> y bf16 [M, G, N].
    mx (with fp8_groups): the MX-like 32-element blocks: a_scale = storage of
    wq_group_quant_mxfp8 [G, K/128, TA], b_scale = UE8M0 bytes uint8 [G, N, K/32].
    b_fragment: INT8 weights cast by wq_pack_weight_i8: expert weights [E, N, K] (same shape
    and strides) with seg_offsets, or a dense [N, K] cast (flat N*K bytes; give n = N) at
    M < 256 (K % 512 == 0, K <= 4096).
    expected_rows: with seg_offsets, the rows per expert the caller expects (a kernel-choice
    hint; the same bytes for every value)."""
    d = MatmulDesc()
    d.b_layout = WQ_LAYOUT_FRAGMENT if b_fragment else WQ_LAYOUT_PLAIN
    d.expected_rows = expected_rows
    dev = a.device
    if fp8_groups is not None:
        G = fp8_groups
        M, Ga, K = a.shape
        N = b.shape[1]
        if y is None:
            y = torch.empty((M, G, N), dtype=torch.bfloat16, device=dev)
        d.payload, d.epilogue = (WQ_PAYLOAD_MXFP8 if mx else WQ_PAYLOAD_FP8_E4M3), WQ_EPI_BF16
        d.M, d.N, d.K, d.batch = M, N, K, G
        d.a, d.lda, d.a_batch_stride = _ptr(a), a.stride(0), a.stride(1)
        d.a_scale, d.a_scale_tokens = _ptr(a_scale), a_scale.shape[2]
        d.b, d.b_batch_stride, d.b_scale = _ptr(b), b.stride(0), _ptr(b_scale)
        d.y, d.ldy, d.y_batch_stride = _ptr(y), y.stride(0), y.stride(1)
    else:
        M, K = a.shape
        if b.dim() == 1:
            if not b_fragment or n is None:
                raise ValueError("a flat b is a fragment-order cast: pass b_fragment=True and n")
            N = n
        else:
            N = b.shape[-2]
        batch = b.shape[0] if b.dim() == 3 else 1
        ncols = N // 2 if epilogue == WQ_EPI_SWIGLU_F32 else N
        if y is None:
            y = torch.empty((M, ncols), dtype=torch.float32 if epilogue == WQ_EPI_SWIGLU_F32 else torch.bfloat16,
                            device=dev)
        d.payload, d.epilogue = WQ_PAYLOAD_INT8, epilogue
        d.M, d.N, d.K, d.batch = M, N, K, batch
        d.seg_offsets = _ptr(seg_offsets)
        d.a, d.lda, d.a_scale = _ptr(a), a.stride(0), _ptr(a_scale)
        d.b, d.b_batch_stride, d.b_scale = _ptr(b), (b.stride(0) if b.dim() == 3 else 0), _ptr(b_scale)
        d.y, d.ldy = _ptr(y), y.stride(0)
        d.acc_out = _ptr(acc_out)
    ctx = context(dev)
    _check("wq_quant_matmul", lib().wq_quant_matmul(ctx.handle, ctypes.byref(d), _stream(dev)))
    return y


def wq_fused_quant_matmul(x, w, w_scale, *, y=None, x_q_out=None, x_scale_out=None, acc_out=None):
    """x bf16 [M, K], w int8 [N, K], w_scale f32 [N] -> y bf16 [M, N] in one launch."""
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16 [M, K] with unit stride along K")
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ctx = context(x.device)
    st = lib().wq_fused_quant_matmul(ctx.handle, _ptr(x), M, K, x.stride(0), _ptr(w), _ptr(w_scale), N, _ptr(y),
                                     y.stride(0), _ptr(x_q_out), _ptr(x_scale_out), _ptr(acc_out),
                                     _stream(x.device))
    _check("wq_fused_quant_matmul", st)
    return y


def wq_fused_quant_matmul_static(x, w, w_scale, *, y=None, x_q_out=None, x_scale_out=None, acc_out=None):
    """wq_fused_quant_matmul through the allocation-free entry point (no context, the library's
    static staging buffer); y is allocated here unless given."""
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16 [M, K] with unit stride along K")
    M, K = x.shape
    N = w.shape[0]
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    idx = x.device.index if x.device.index is not None else torch.cuda.current_device()
    st = lib().wq_fused_quant_matmul_static(idx, _ptr(x), M, K, x.stride(0), _ptr(w), _ptr(w_scale), N, _ptr(y),
                                            y.stride(0), _ptr(x_q_out), _ptr(x_scale_out), _ptr(acc_out),
                                            _stream(x.device))
    _check("wq_fused_quant_matmul_static", st)
    return y


def wq_pack_weight_i8(w, wp=None):
    """int8 w [N, K] (unit stride along K) -> the same bytes in fragment order (wq.h), as a
    flat int8 tensor of N*K bytes for wq_fused_quant_matmul_packed.  For expert weights
    [E, N, K] (contiguous) each expert is cast in place of its own [N, K] block: the result
    has w's shape, for wq_quant_matmul(..., seg_offsets=..., b_fragment=True)."""
    if w.dim() == 3:
        if not w.is_contiguous() or w.dtype != torch.int8:
            raise ValueError("expert weights must be contiguous int8 [E, N, K]")
        out = torch.empty_like(w) if wp is None else wp
        for e in range(w.shape[0]):
            wq_pack_weight_i8(w[e], out[e].view(-1))
        return out
    if w.dim() != 2 or w.stride(1) != 1 or w.dtype != torch.int8:
        raise ValueError("w must be int8 [N, K] with unit stride along K")
    N, K = w.shape
    if wp is None:
        wp = torch.empty((N * K,), dtype=torch.int8, device=w.device)
    ctx = context(w.device)
    _check("wq_pack_weight_i8", lib().wq_pack_weight_i8(ctx.handle, _ptr(w), N, K, w.stride(0), _ptr(wp),
                                                         _stream(w.device)))
    return wp


def wq_fused_quant_matmul_packed(x, wp, w_scale, N, *, y=None, x_q_out=None, x_scale_out=None, acc_out=None):
    """x bf16 [M, K], wp from wq_pack_weight_i8 (N*K bytes), w_scale f32 [N] -> y bf16 [M, N]."""
    if x.dim() != 2 or x.stride(1) != 1 or x.dtype != torch.bfloat16:
        raise ValueError("x must be bf16 [M, K] with unit stride along K")
    M, K = x.shape
    if wp.numel() != N * K:
        raise ValueError("wp must hold N*K bytes")
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    ctx = context(x.device)
    st = lib().wq_fused_quant_matmul_packed(ctx.handle, _ptr(x), M, K, x.stride(0), _ptr(wp), _ptr(w_scale), N,
                                            _ptr(y), y.stride(0), _ptr(x_q_out), _ptr(x_scale_out), _ptr(acc_out),
                                            _stream(x.device))
    _check("wq_fused_quant_matmul_packed", st)
    return y


FUSED_PATHS = {0: "quant kernel + GEMM (two launches)", 1: "one launch: dot4 GEMV", 2: "one launch: 8-wave MFMA"}


def wq_fused_path(M: int, K: int, N: int, device=None) -> int:
    """Launch sequence wq_fused_quant_matmul takes for these sizes (see FUSED_PATHS)."""
    ctx = context(device or torch.device("cuda", torch.cuda.current_device()))
    r = lib().wq_fused_path(ctx.handle, M, K, N)
    if r < 0:
        _check("wq_fused_path", -r)
    return r


def wq_moe_sort(ids: torch.Tensor, num_experts: int):
    """ids int32 [T, topk] -> (perm int32 [T*topk], row_token int32 [T*topk], offsets int64 [E+1])."""
    T, topk = ids.shape
    dev = ids.device
    perm = torch.empty(T * topk, dtype=torch.int32, device=dev)
    row_token = torch.empty(T * topk, dtype=torch.int32, device=dev)
    offsets = torch.empty(num_experts + 1, dtype=torch.int64, device=dev)
    ctx = context(dev)
    st = lib().wq_moe_sort(ctx.handle, _ptr(ids.contiguous()), T, topk, num_experts, _ptr(perm), _ptr(row_token),
                           _ptr(offsets), _stream(dev))
    _check("wq_moe_sort", st)
    return perm, row_token, offsets
