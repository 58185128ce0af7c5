"""fp8q: FP8 rollout hot path on MI355X (gfx950) — Python binding of libfp8q.

Thin ctypes binding over the C ABI declared in ``include/fp8q.h``.  Each function
has the name of the C entry point it calls and does argument marshalling only:
tensors are turned into device pointers, leading dimensions and the current HIP
stream; every step of the computation runs in libfp8q's HIP kernels.  PyTorch is
used for device memory and streams.

There is no fallback: if ``libfp8q.so`` is missing, or a call fails, an exception
is raised.  Build the library with ``python -m fp8_block_scaled_weight_amd.build``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Iterable, Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8q.so")

FP8Q_OK = 0
FP8Q_ERR_NULL = 1
FP8Q_ERR_SHAPE = 2
FP8Q_ERR_STRIDE = 3
FP8Q_ERR_ALIGN = 4
FP8Q_ERR_LAUNCH = 5
FP8Q_ERR_UNSUPPORTED = 6
FP8Q_ERR_PRECONDITION = 7  # FP8Q_DEBUG=1: a documented precondition is violated
FP8Q_KV_RECALIBRATE = 1
FP8Q_ATTN_RECALIBRATE_Q = 1

EXPORTED = (
    "fp8q_status_string", "fp8q_last_error", "fp8q_abi_version", "fp8q_quant_weight_blk128",
    "fp8q_quant_act_g128", "fp8q_gemm_w8a8_blkscaled", "fp8q_grouped_gemm_w8a8", "fp8q_kv_quant",
    "fp8q_quant_weight_blk128_ue8m0", "fp8q_quant_act_g128_ue8m0", "fp8q_gemm_w8a8_ue8m0",
    "fp8q_grouped_gemm_w8a8_ue8m0", "fp8q_moe_dispatch", "fp8q_swiglu_quant_g128", "fp8q_moe_combine",
    "fp8q_gemm_w8a8_bf16act", "fp8q_paged_decode_attention", "fp8q_grouped_gemm_swiglu_quant",
    "fp8q_moe_route", "fp8q_swiglu_quant_g128_ue8m0", "fp8q_grouped_gemm_swiglu_quant_ue8m0",
    "fp8q_gemm_w8a8_bf16act_ue8m0",
)


class Fp8qError(RuntimeError):
    def __init__(self, status: int, where: str, detail: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}: {detail}")


class WeightDesc(ctypes.Structure):
    """Mirror of ``fp8q_weight_desc``."""
    _fields_ = [("w", ctypes.c_void_p), ("q", ctypes.c_void_p), ("s", ctypes.c_void_p),
                ("n", ctypes.c_int64), ("k", ctypes.c_int64), ("ld_w", ctypes.c_int64),
                ("ld_q", ctypes.c_int64)]


_lib = None


def lib() -> ctypes.CDLL:
    """The loaded libfp8q.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libfp8q.so not found at {LIB_PATH}; build it with "
                              "`python -m fp8_block_scaled_weight_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, i64, i32, u32, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32, ctypes.c_float
        L.fp8q_status_string.argtypes = [ctypes.c_int]
        L.fp8q_status_string.restype = ctypes.c_char_p
        L.fp8q_last_error.argtypes = []
        L.fp8q_last_error.restype = ctypes.c_char_p
        L.fp8q_abi_version.argtypes = []
        L.fp8q_abi_version.restype = ctypes.c_int
        for sfx in ("", "_ue8m0"):
            getattr(L, "fp8q_quant_weight_blk128" + sfx).argtypes = [ctypes.POINTER(WeightDesc), i32, vp]
            getattr(L, "fp8q_quant_act_g128" + sfx).argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp]
            getattr(L, "fp8q_grouped_gemm_w8a8" + sfx).argtypes = [vp, i64, vp, i64, vp, vp, vp, i32, i64, vp, i64,
                                                                   i64, i64, vp]
        L.fp8q_gemm_w8a8_blkscaled.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp]
        L.fp8q_gemm_w8a8_ue8m0.argtypes = L.fp8q_gemm_w8a8_blkscaled.argtypes
        L.fp8q_paged_decode_attention.argtypes = [vp, i64, vp, vp, vp, i64, vp, i32, i32, i32, i32, i32, i64, vp,
                                                  vp, vp, f32, f32, u32, vp, i64, vp]
        L.fp8q_gemm_w8a8_bf16act.argtypes = [vp, i64, vp, i64, vp, vp, i64, i64, i64, i64, vp]
        L.fp8q_gemm_w8a8_bf16act_ue8m0.argtypes = L.fp8q_gemm_w8a8_bf16act.argtypes
        L.fp8q_kv_quant.argtypes = [vp, i64, vp, i64, i64, i32, i32, vp, vp, vp, i32, i64, vp, vp, f32, u32, vp]
        L.fp8q_moe_dispatch.argtypes = [vp, i64, vp, i64, vp, i64, i32, i32, i64, vp, i64, vp, i64, vp, vp, vp]
        L.fp8q_swiglu_quant_g128.argtypes = [vp, i64, i64, i64, vp, i64, vp, i64, vp]
        L.fp8q_grouped_gemm_swiglu_quant.argtypes = [vp, i64, vp, i64, vp, i64, vp, vp, vp, i32, i64, vp, i64,
                                                     vp, i64, i64, i64, vp]
        L.fp8q_swiglu_quant_g128_ue8m0.argtypes = L.fp8q_swiglu_quant_g128.argtypes
        L.fp8q_grouped_gemm_swiglu_quant_ue8m0.argtypes = L.fp8q_grouped_gemm_swiglu_quant.argtypes
        L.fp8q_moe_route.argtypes = [vp, i64, i32, i32, vp, vp, vp, vp]
        L.fp8q_moe_combine.argtypes = [vp, i64, vp, vp, i64, i32, i64, vp, i64, vp]
        for name in EXPORTED[3:]:
            getattr(L, name).restype = ctypes.c_int
        _lib = L
    return _lib


def status_string(status: int) -> str:
    return lib().fp8q_status_string(int(status)).decode()


def last_error() -> str:
    return lib().fp8q_last_error().decode()


def abi_version() -> int:
    return int(lib().fp8q_abi_version())


def _check(status: int, where: str) -> None:
    if status != FP8Q_OK:
        raise Fp8qError(status, where, last_error())


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str, dtypes: Sequence[torch.dtype]) -> int:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor (libfp8q runs on the GPU only)")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {list(dtypes)}")
    return t.data_ptr()


def _rows(t: torch.Tensor, name: str) -> int:
    """Leading dimension (elements) of a 2-D row-major tensor with unit column stride."""
    if t.dim() != 2 or (t.shape[1] > 1 and t.stride(1) != 1):
        raise ValueError(f"{name} must be 2-D with unit column stride")
    return t.stride(0) if t.shape[0] > 1 else max(t.shape[1], t.stride(0))


FP8 = (torch.float8_e4m3fn, torch.uint8)
BF16 = (torch.bfloat16,)
F32 = (torch.float32,)


def fp8q_quant_weight_blk128(weights: Iterable[tuple], stream=None) -> None:
    """Blockwise-quantize many bf16 weights in one call.

    weights: iterable of (w [n,k] bf16, q [n,k] fp8, s [n/128,k/128] fp32) device tensors."""
    _quant_weight("fp8q_quant_weight_blk128", weights, stream)


def fp8q_quant_weight_blk128_ue8m0(weights: Iterable[tuple], stream=None) -> None:
    """As fp8q_quant_weight_blk128, with power-of-two (UE8M0) scales."""
    _quant_weight("fp8q_quant_weight_blk128_ue8m0", weights, stream)


def _quant_weight(fn: str, weights: Iterable[tuple], stream) -> None:
    items = list(weights)
    arr = (WeightDesc * max(len(items), 1))()
    for i, (w, q, s) in enumerate(items):
        n, k = w.shape
        if tuple(q.shape) != (n, k) or tuple(s.shape) != (n // 128, k // 128) or not s.is_contiguous():
            raise ValueError(f"weight {i}: q must be [n,k] and s contiguous [n/128,k/128]")
        arr[i] = WeightDesc(_dev(w, "w", BF16), _dev(q, "q", FP8), _dev(s, "s", F32), n, k,
                            _rows(w, "w"), _rows(q, "q"))
    _check(getattr(lib(), fn)(arr, len(items), _stream(stream)), fn)


def fp8q_quant_act_g128(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """Per-token 1x128 group quantization: x [m,k] bf16 -> q [m,k] fp8, s [k/128, ld_s] fp32."""
    _quant_act("fp8q_quant_act_g128", x, q, s, stream)


def fp8q_quant_act_g128_ue8m0(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """As fp8q_quant_act_g128, with power-of-two (UE8M0) scales."""
    _quant_act("fp8q_quant_act_g128_ue8m0", x, q, s, stream)


def _quant_act(fn: str, x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream) -> None:
    m, k = x.shape
    if tuple(q.shape) != (m, k) or s.dim() != 2 or s.shape[0] != k // 128 or s.stride(1) != 1:
        raise ValueError("q must be [m,k] and s [k/128, ld_s] with unit column stride")
    _check(getattr(lib(), fn)(_dev(x, "x", BF16), m, k, _rows(x, "x"), _dev(q, "q", FP8), _rows(q, "q"),
                              _dev(s, "s", F32), s.stride(0), _stream(stream)), fn)


def fp8q_gemm_w8a8_blkscaled(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                             y: torch.Tensor, stream=None) -> None:
    """y [m,n] bf16 = block-scaled a [m,k] fp8 (scales a_s [k/128, ld_as]) x b [n,k] fp8 (b_s [n/128,k/128])^T."""
    _gemm("fp8q_gemm_w8a8_blkscaled", a, a_s, b, b_s, y, stream)


def fp8q_gemm_w8a8_ue8m0(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                         y: torch.Tensor, stream=None) -> None:
    """As fp8q_gemm_w8a8_blkscaled for power-of-two scales, applied by the matrix core."""
    _gemm("fp8q_gemm_w8a8_ue8m0", a, a_s, b, b_s, y, stream)


def _gemm(fn, a, a_s, b, b_s, y, stream) -> None:
    m, k = a.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(y.shape) != (m, n) or not b_s.is_contiguous() or a_s.stride(1) != 1:
        raise ValueError("shape mismatch between a, b and y")
    _check(getattr(lib(), fn)(_dev(a, "a", FP8), _rows(a, "a"), _dev(a_s, "a_s", F32), a_s.stride(0),
                              _dev(b, "b", FP8), _rows(b, "b"), _dev(b_s, "b_s", F32),
                              _dev(y, "y", BF16), _rows(y, "y"), m, n, k, _stream(stream)), fn)


def fp8q_gemm_w8a8_bf16act(x: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor, y: torch.Tensor,
                           stream=None) -> None:
    """y [m,n] bf16 = the block-scaled GEMM of x [m,k] bf16 (m <= 64), quantized per 1x128 group
    inside the kernel, with b [n,k] fp8 (b_s [n/128,k/128])."""
    _bf16act("fp8q_gemm_w8a8_bf16act", x, b, b_s, y, stream)


def fp8q_gemm_w8a8_bf16act_ue8m0(x: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor, y: torch.Tensor,
                                 stream=None) -> None:
    """As fp8q_gemm_w8a8_bf16act with power-of-two (UE8M0) scales."""
    _bf16act("fp8q_gemm_w8a8_bf16act_ue8m0", x, b, b_s, y, stream)


def _bf16act(fn, x, b, b_s, y, stream) -> None:
    m, k = x.shape
    n = b.shape[0]
    if b.shape[1] != k or tuple(y.shape) != (m, n) or not b_s.is_contiguous():
        raise ValueError("shape mismatch between x, b and y")
    _check(getattr(lib(), fn)(_dev(x, "x", BF16), _rows(x, "x"), _dev(b, "b", FP8), _rows(b, "b"),
                              _dev(b_s, "b_s", F32), _dev(y, "y", BF16), _rows(y, "y"), m, n, k, _stream(stream)),
           fn)


def fp8q_grouped_gemm_w8a8(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                           group_offsets: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """Grouped GEMM: rows [off[g], off[g+1]) of a [M,k] times b[g] ([G,n,k]) with scales b_s [G,n/128,k/128]."""
    _grouped("fp8q_grouped_gemm_w8a8", a, a_s, b, b_s, group_offsets, y, stream)


def fp8q_grouped_gemm_w8a8_ue8m0(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                                 group_offsets: torch.Tensor, y: torch.Tensor, stream=None) -> None:
    """As fp8q_grouped_gemm_w8a8 for power-of-two scales, applied by the matrix core."""
    _grouped("fp8q_grouped_gemm_w8a8_ue8m0", a, a_s, b, b_s, group_offsets, y, stream)


def _grouped(fn, a, a_s, b, b_s, group_offsets, y, stream) -> None:
    total_m, k = a.shape
    g, n, kb = b.shape
    if kb != k or tuple(y.shape) != (total_m, n) or not b.is_contiguous() or not b_s.is_contiguous():
        raise ValueError("shape mismatch between a, b and y")
    if group_offsets.numel() != g + 1:
        raise ValueError("group_offsets must have G+1 entries")
    _check(getattr(lib(), fn)(_dev(a, "a", FP8), _rows(a, "a"), _dev(a_s, "a_s", F32), a_s.stride(0),
                              _dev(b, "b", FP8), _dev(b_s, "b_s", F32),
                              _dev(group_offsets, "group_offsets", (torch.int32,)), g, total_m,
                              _dev(y, "y", BF16), _rows(y, "y"), n, k, _stream(stream)), fn)


def fp8q_kv_quant(k: torch.Tensor, v: torch.Tensor, slot_mapping: torch.Tensor, k_cache: torch.Tensor,
                  v_cache: torch.Tensor, k_scale: torch.Tensor, v_scale: torch.Tensor,
                  fp8_range: float = 448.0, recalibrate: bool = False, stream=None) -> None:
    """Quantize-on-write of k, v [T, H, 128] bf16 into paged caches [P, page, H, 128] fp8."""
    t = k.shape[0]
    heads, hd = k.shape[1], k.shape[2]
    pages, page_size = k_cache.shape[0], k_cache.shape[1]
    if tuple(v.shape) != tuple(k.shape) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k/v and k_cache/v_cache shapes must match")
    if k_cache.shape[2:] != (heads, hd) or not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("caches must be contiguous [pages, page_size, heads, head_dim]")
    if k.stride(2) != 1 or k.stride(1) != hd or v.stride(2) != 1 or v.stride(1) != hd:
        raise ValueError("k/v rows must be contiguous over (heads, head_dim)")
    _check(lib().fp8q_kv_quant(_dev(k, "k", BF16), k.stride(0), _dev(v, "v", BF16), v.stride(0), t, heads, hd,
                               _dev(slot_mapping, "slot_mapping", (torch.int64,)), _dev(k_cache, "k_cache", FP8),
                               _dev(v_cache, "v_cache", FP8), page_size, pages, _dev(k_scale, "k_scale", F32),
                               _dev(v_scale, "v_scale", F32), float(fp8_range),
                               FP8Q_KV_RECALIBRATE if recalibrate else 0, _stream(stream)),
           "fp8q_kv_quant")


def fp8q_moe_dispatch(xq: torch.Tensor, xs: torch.Tensor, topk_ids: torch.Tensor, num_experts: int,
                      aq: torch.Tensor, a_s: torch.Tensor, offsets: torch.Tensor, row_of: torch.Tensor,
                      stream=None) -> None:
    """Dispatch quantized tokens xq [T,k] fp8 (scales xs [k/128, ld_xs]) to the experts recorded in
    topk_ids [T,topk] int16: aq [>=T*topk, k] fp8, a_s [k/128, >=T*topk], offsets [E+1] int32 and
    row_of [T,topk] int32 (row of each entry, -1 if dropped)."""
    t, k = xq.shape
    topk = topk_ids.shape[1] if topk_ids.dim() == 2 else 1
    if topk_ids.shape[0] != t or not topk_ids.is_contiguous() or not row_of.is_contiguous():
        raise ValueError("topk_ids and row_of must be contiguous [T, topk]")
    if row_of.numel() != t * topk or offsets.numel() != num_experts + 1:
        raise ValueError("row_of must have T*topk entries and offsets E+1")
    if aq.shape[1] != k or aq.shape[0] < t * topk or a_s.shape[0] != k // 128 or a_s.stride(1) != 1 \
            or xs.stride(1) != 1:
        raise ValueError("aq must be [>=T*topk, k] and a_s [k/128, >=T*topk] with unit column stride")
    _check(lib().fp8q_moe_dispatch(_dev(xq, "xq", FP8), _rows(xq, "xq"), _dev(xs, "xs", F32), xs.stride(0),
                                   _dev(topk_ids, "topk_ids", (torch.int16,)), t, topk, int(num_experts), k,
                                   _dev(aq, "aq", FP8), _rows(aq, "aq"), _dev(a_s, "a_s", F32), a_s.stride(0),
                                   _dev(offsets, "offsets", (torch.int32,)), _dev(row_of, "row_of", (torch.int32,)),
                                   _stream(stream)), "fp8q_moe_dispatch")


def fp8q_moe_route(topk_ids: torch.Tensor, num_experts: int, offsets: torch.Tensor, row_of: torch.Tensor,
                   row_token: torch.Tensor, stream=None) -> None:
    """The routing of fp8q_moe_dispatch without its copies: offsets [E+1], row_of [T, topk], and
    row_token [T*topk] (row -> token) for a fc1 that reads the token rows directly."""
    t, topk = topk_ids.shape
    if offsets.numel() != num_experts + 1 or row_of.numel() != t * topk or row_token.numel() < t * topk:
        raise ValueError("offsets must have E+1 entries, row_of and row_token T*topk")
    _check(lib().fp8q_moe_route(_dev(topk_ids, "topk_ids", (torch.int16,)), t, topk, int(num_experts),
                                _dev(offsets, "offsets", (torch.int32,)), _dev(row_of, "row_of", (torch.int32,)),
                                _dev(row_token, "row_token", (torch.int32,)), _stream(stream)), "fp8q_moe_route")


def fp8q_swiglu_quant_g128(h: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """silu(gate) * up of h = [gate | up] ([m, 2n] bf16), quantized per 1x128 group:
    q [m, n] fp8, s [n/128, ld_s] fp32."""
    _swiglu("fp8q_swiglu_quant_g128", h, q, s, stream)


def fp8q_swiglu_quant_g128_ue8m0(h: torch.Tensor, q: torch.Tensor, s: torch.Tensor, stream=None) -> None:
    """As fp8q_swiglu_quant_g128 with power-of-two (UE8M0) scales."""
    _swiglu("fp8q_swiglu_quant_g128_ue8m0", h, q, s, stream)


def _swiglu(fn, h, q, s, stream) -> None:
    m, n2 = h.shape
    n = n2 // 2
    if tuple(q.shape) != (m, n) or s.dim() != 2 or s.shape[0] != n // 128 or s.stride(1) != 1:
        raise ValueError("q must be [m, n] and s [n/128, ld_s] with unit column stride")
    _check(getattr(lib(), fn)(_dev(h, "h", BF16), m, n, _rows(h, "h"), _dev(q, "q", FP8), _rows(q, "q"),
                              _dev(s, "s", F32), s.stride(0), _stream(stream)), fn)


def fp8q_grouped_gemm_swiglu_quant(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                                   group_offsets: torch.Tensor, q: torch.Tensor, s: torch.Tensor,
                                   row_token: Optional[torch.Tensor] = None, stream=None) -> None:
    """MoE fc1 with SwiGLU and fc2's 1x128 input quantization fused: b [G, 2*n_half, k] holds each
    expert's gate rows, then its up rows.  Equal, bit for bit, to fp8q_grouped_gemm_w8a8 into a
    bf16 [total_m, 2*n_half] buffer followed by fp8q_swiglu_quant_g128 on it: q [total_m, n_half]
    fp8, s [n_half/128, ld_s] fp32.  With row_token (fp8q_moe_route's), a [T, k] and a_s are the
    token rows and dispatched row r reads token row_token[r]."""
    _grouped_swiglu("fp8q_grouped_gemm_swiglu_quant", a, a_s, b, b_s, group_offsets, q, s, row_token, stream)


def fp8q_grouped_gemm_swiglu_quant_ue8m0(a: torch.Tensor, a_s: torch.Tensor, b: torch.Tensor, b_s: torch.Tensor,
                                         group_offsets: torch.Tensor, q: torch.Tensor, s: torch.Tensor,
                                         row_token: Optional[torch.Tensor] = None, stream=None) -> None:
    """As fp8q_grouped_gemm_swiglu_quant for power-of-two (UE8M0) scales: equal, bit for bit, to
    fp8q_grouped_gemm_w8a8_ue8m0 followed by fp8q_swiglu_quant_g128_ue8m0."""
    _grouped_swiglu("fp8q_grouped_gemm_swiglu_quant_ue8m0", a, a_s, b, b_s, group_offsets, q, s, row_token,
                    stream)


def _grouped_swiglu(fn, a, a_s, b, b_s, group_offsets, q, s, row_token, stream) -> None:
    a_rows, k = a.shape
    total_m = q.shape[0]
    g, n2, kb = b.shape
    n_half = n2 // 2
    if row_token is None and a_rows != total_m:
        raise ValueError("without row_token, a holds the total_m dispatched rows")
    if kb != k or n2 % 2 or q.shape[1] != n_half or not b.is_contiguous() or not b_s.is_contiguous():
        raise ValueError("shape mismatch between a, b and q")
    if s.dim() != 2 or s.shape[0] != n_half // 128 or s.stride(1) != 1:
        raise ValueError("s must be [n_half/128, ld_s] with unit column stride")
    if group_offsets.numel() != g + 1:
        raise ValueError("group_offsets must have G+1 entries")
    tok = 0 if row_token is None else _dev(row_token, "row_token", (torch.int32,))
    _check(getattr(lib(), fn)(
        _dev(a, "a", FP8), _rows(a, "a"), _dev(a_s, "a_s", F32), a_s.stride(0), tok, a_rows, _dev(b, "b", FP8),
        _dev(b_s, "b_s", F32), _dev(group_offsets, "group_offsets", (torch.int32,)), g, total_m,
        _dev(q, "q", FP8), _rows(q, "q"), _dev(s, "s", F32), s.stride(0), n_half, k, _stream(stream)), fn)


def fp8q_moe_combine(y: torch.Tensor, row_of: torch.Tensor, weights: torch.Tensor, out: torch.Tensor,
                     stream=None) -> None:
    """out [T, hidden] bf16 = sum_j weights[t, j] * y[row_of[t, j]] (rows -1 skipped), fp32 sum, one rounding."""
    t, topk = row_of.shape
    hidden = out.shape[1]
    if out.shape[0] != t or y.shape[1] != hidden or tuple(weights.shape) != (t, topk):
        raise ValueError("shape mismatch between y, row_of, weights and out")
    if not row_of.is_contiguous() or not weights.is_contiguous():
        raise ValueError("row_of and weights must be contiguous [T, topk]")
    _check(lib().fp8q_moe_combine(_dev(y, "y", BF16), _rows(y, "y"), _dev(row_of, "row_of", (torch.int32,)),
                                  _dev(weights, "weights", F32), t, topk, hidden, _dev(out, "out", BF16),
                                  _rows(out, "out"), _stream(stream)), "fp8q_moe_combine")


def fp8q_paged_decode_attention(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                block_table: torch.Tensor, seq_lens: torch.Tensor, q_scale: torch.Tensor,
                                k_scale: torch.Tensor, v_scale: torch.Tensor, sm_scale: float, out: torch.Tensor,
                                recalibrate_q: bool = False, fp8_range: float = 448.0, stream=None) -> None:
    """FP8 decode attention: q [S, H, 128] bf16 over caches [P, page, Hkv, 128] fp8 with block_table
    [S, ld_bt] int32 and seq_lens [S] int32 -> out [S, H, 128] bf16.  recalibrate_q first sets
    q_scale from the queries."""
    seqs, hq, hd = q.shape
    pages, page_size, hkv = k_cache.shape[0], k_cache.shape[1], k_cache.shape[2]
    if tuple(v_cache.shape) != tuple(k_cache.shape) or not k_cache.is_contiguous() or not v_cache.is_contiguous():
        raise ValueError("caches must be contiguous [pages, page_size, heads, head_dim] of one shape")
    if q.stride(2) != 1 or q.stride(1) != hd or out.stride(2) != 1 or out.stride(1) != hd:
        raise ValueError("q/out rows must be contiguous over (heads, head_dim)")
    if tuple(out.shape) != (seqs, hq, hd) or block_table.dim() != 2 or block_table.shape[0] != seqs:
        raise ValueError("out must be [S, H, 128] and block_table [S, ld_bt]")
    if block_table.stride(1) != 1 or not seq_lens.is_contiguous():
        raise ValueError("block_table rows and seq_lens must be contiguous")
    _check(lib().fp8q_paged_decode_attention(
        _dev(q, "q", BF16), q.stride(0), _dev(k_cache, "k_cache", FP8), _dev(v_cache, "v_cache", FP8),
        _dev(block_table, "block_table", (torch.int32,)), block_table.stride(0),
        _dev(seq_lens, "seq_lens", (torch.int32,)), seqs, hq, hkv, hd, page_size, pages,
        _dev(q_scale, "q_scale", F32), _dev(k_scale, "k_scale", F32), _dev(v_scale, "v_scale", F32),
        float(sm_scale), float(fp8_range), FP8Q_ATTN_RECALIBRATE_Q if recalibrate_q else 0,
        _dev(out, "out", BF16), out.stride(0), _stream(stream)), "fp8q_paged_decode_attention")
