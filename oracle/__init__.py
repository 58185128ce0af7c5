"""CPU oracle for the FP8 rollout hot path (test infrastructure only).

This package wraps ``fp8q_oracle.c``: a plain, slow, scalar C implementation of
what the hot path computes, in fp64 where the method leaves precision open.  It
exists to check the HIP library: only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.  It
shares no code with the HIP library and imports nothing from it.

Every function takes numpy arrays (bf16 as ``uint16`` bit patterns, FP8 codes as
``uint8``) and returns numpy arrays.  See ``fp8q_oracle.c`` for the page and
section each computation follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC"]

# FP8Q_ORACLE_SANITIZE=1 builds and loads a separate AddressSanitizer + UndefinedBehavior-
# Sanitizer build of the oracle (host code only; the interpreter must run with gcc's
# libasan preloaded, e.g. LD_PRELOAD=$(gcc -print-file-name=libasan.so)
# ASAN_OPTIONS=detect_leaks=0), so the CPU test suite can run against it.
SANITIZE = os.environ.get("FP8Q_ORACLE_SANITIZE", "0") == "1"
if SANITIZE:
    _LIB_PATH = os.path.join(_HERE, "libfp8q_oracle_asan.so")
    CFLAGS = CFLAGS + ["-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                       "-fno-sanitize-recover=undefined"]
else:
    _LIB_PATH = os.path.join(_HERE, "libfp8q_oracle.so")


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (fp-contract off, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_u8p = np.ctypeslib.ndpointer(dtype=np.uint8, flags="C_CONTIGUOUS")
_u16p = np.ctypeslib.ndpointer(dtype=np.uint16, flags="C_CONTIGUOUS")
_f32p = np.ctypeslib.ndpointer(dtype=np.float32, flags="C_CONTIGUOUS")
_f64p = np.ctypeslib.ndpointer(dtype=np.float64, flags="C_CONTIGUOUS")
_i32p = np.ctypeslib.ndpointer(dtype=np.int32, flags="C_CONTIGUOUS")
_i64p = np.ctypeslib.ndpointer(dtype=np.int64, flags="C_CONTIGUOUS")
_i64 = ctypes.c_int64


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_double]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_scale.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_scale.restype = ctypes.c_float
        L.oracle_quantize_value.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_quantize_value.restype = ctypes.c_uint8
        L.oracle_scale_ue8m0.argtypes = [ctypes.c_float, ctypes.c_float]
        L.oracle_scale_ue8m0.restype = ctypes.c_float
        for f in ("oracle_quant_weight_blk128", "oracle_quant_weight_blk128_ue8m0"):
            getattr(L, f).argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _f32p]
        for f in ("oracle_quant_act_g128", "oracle_quant_act_g128_ue8m0"):
            getattr(L, f).argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _f32p, _i64]
        L.oracle_gemm_w8a8.argtypes = [_u8p, _i64, _f32p, _i64, _u8p, _i64, _f32p, _f64p, _i64,
                                       _i64, _i64, _i64]
        L.oracle_grouped_gemm_w8a8.argtypes = [_u8p, _i64, _f32p, _i64, _u8p, _f32p, _i32p,
                                               ctypes.c_int32, _f64p, _i64, _i64, _i64]
        L.oracle_kv_quant.argtypes = [_u16p, _i64, _u16p, _i64, _i64, ctypes.c_int32,
                                      ctypes.c_int32, _i64p, _u8p, _u8p, ctypes.c_int32, _i64,
                                      _f32p, _f32p, ctypes.c_float, ctypes.c_int]
        L.oracle_kv_scales.argtypes = [_u16p, _i64, _u16p, _i64, _i64, _i64, _i64p, ctypes.c_float, _f32p, _f32p]
        L.oracle_q_scale.argtypes = [_u16p, _i64, ctypes.c_int32, ctypes.c_int32, ctypes.c_float, _f32p]
        L.oracle_paged_decode_attention.argtypes = [_u16p, _i64, _u8p, _u8p, _i32p, _i64, _i32p, ctypes.c_int32,
                                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_float,
                                                    ctypes.c_float, ctypes.c_float, ctypes.c_double, _f64p]
        L.oracle_swiglu_quant_g128.argtypes = [_u16p, _i64, _i64, _i64, _u8p, _i64, _f32p, _i64, _f64p]
        L.oracle_swiglu_quant_g128_ue8m0.argtypes = L.oracle_swiglu_quant_g128.argtypes
        L.oracle_silu_times_up.argtypes = [ctypes.c_double, ctypes.c_double]
        L.oracle_silu_times_up.restype = ctypes.c_double
        for f in ("oracle_kv_scales", "oracle_quant_weight_blk128", "oracle_quant_act_g128", "oracle_gemm_w8a8",
                  "oracle_swiglu_quant_g128", "oracle_swiglu_quant_g128_ue8m0", "oracle_q_scale",
                  "oracle_paged_decode_attention",
                  "oracle_quant_weight_blk128_ue8m0", "oracle_quant_act_g128_ue8m0",
                  "oracle_grouped_gemm_w8a8", "oracle_kv_quant", "oracle_num_threads"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int, what: str) -> None:
    if rc == -1:
        raise ValueError(f"{what}: non-finite input (inputs must be finite)")
    if rc != 0:
        raise ValueError(f"{what}: invalid shape or argument (rc={rc})")


def _u16(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    return a


def num_threads() -> int:
    return lib().oracle_num_threads()


def e4m3_decode(code: int) -> float:
    return lib().oracle_e4m3_decode(int(code))


def e4m3_encode(u: float) -> int:
    """Nearest E4M3FN code to the real number ``u`` (ties to even, saturating)."""
    return int(lib().oracle_e4m3_encode(float(u)))


def scale(amax: float, rng: float = 448.0) -> np.float32:
    return np.float32(lib().oracle_scale(float(amax), float(rng)))


def scale_ue8m0(amax: float, rng: float = 448.0) -> np.float32:
    """Power-of-two scale: the smallest 2^e with rng * 2^e >= amax (e in [-127, 127]); 1 for 0."""
    return np.float32(lib().oracle_scale_ue8m0(float(amax), float(rng)))


def quantize_value(x: float, s: float) -> int:
    """E4M3FN code of the exact quotient x / s (x and s as binary32)."""
    return int(lib().oracle_quantize_value(float(np.float32(x)), float(np.float32(s))))


def quant_weight_blk128(w_bits: np.ndarray, ue8m0: bool = False):
    """128x128 blockwise quantization of a bf16 [n, k] weight -> (codes [n,k], scales [n/128,k/128]).
    ue8m0=True takes power-of-two scales instead of fl32(amax/448)."""
    w = _u16(w_bits)
    n, k = w.shape
    q = np.empty((n, k), dtype=np.uint8)
    s = np.empty((n // 128, k // 128), dtype=np.float32)
    f = lib().oracle_quant_weight_blk128_ue8m0 if ue8m0 else lib().oracle_quant_weight_blk128
    _check(f(w, n, k, k, q, k, s), "quant_weight_blk128")
    return q, s


def quant_act_g128(x_bits: np.ndarray, ld_s: int | None = None, ue8m0: bool = False):
    """1x128 group quantization of bf16 [m, k] -> (codes [m,k], scales [k/128, ld_s]).
    ue8m0=True takes power-of-two scales instead of fl32(amax/448)."""
    x = _u16(x_bits)
    m, k = x.shape
    ld_s = m if ld_s is None else ld_s
    q = np.empty((m, k), dtype=np.uint8)
    s = np.zeros((k // 128, ld_s), dtype=np.float32)
    f = lib().oracle_quant_act_g128_ue8m0 if ue8m0 else lib().oracle_quant_act_g128
    _check(f(x, m, k, k, q, k, s, ld_s), "quant_act_g128")
    return q, s


def gemm_w8a8(a: np.ndarray, a_s: np.ndarray, b: np.ndarray, b_s: np.ndarray) -> np.ndarray:
    """fp64 block-scaled GEMM: a [m,k] codes, a_s [k/128, ld_as], b [n,k] codes, b_s [n/128,k/128]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    b_s = np.ascontiguousarray(b_s, dtype=np.float32)
    m, k = a.shape
    n = b.shape[0]
    y = np.empty((m, n), dtype=np.float64)
    _check(lib().oracle_gemm_w8a8(a, k, a_s, a_s.shape[1], b, k, b_s, y, n, m, n, k), "gemm_w8a8")
    return y


def e4m3_table() -> np.ndarray:
    """The oracle's decoded value of each of the 256 E4M3FN codes (NaN codes as NaN)."""
    return np.array([lib().oracle_e4m3_decode(c) for c in range(256)], dtype=np.float64)


def gemm_w8a8_blockwise(a: np.ndarray, a_s: np.ndarray, b: np.ndarray, b_s: np.ndarray) -> np.ndarray:
    """The same fp64 block-scaled GEMM as ``gemm_w8a8``, for full-size shapes: each K block's
    product sum_{t in kb} dec(a[i,t]) dec(b[j,t]) is one float64 matrix product of the
    decoded codes (a library step; every partial sum is an integer multiple of 2^-18 below
    2^43, so it is exact in any summation order), then y += (sa * sb) * P_kb with kb
    ascending, the definition's outer sum in the C oracle's order and operations."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_s = np.asarray(a_s, dtype=np.float32)
    b_s = np.asarray(b_s, dtype=np.float32)
    m, k = a.shape
    n = b.shape[0]
    dec = e4m3_table()
    y = np.zeros((m, n), dtype=np.float64)
    for kb in range(k // 128):
        da = dec[a[:, kb * 128:(kb + 1) * 128]]
        db = dec[b[:, kb * 128:(kb + 1) * 128]]
        p = da @ db.T
        s = a_s[kb, :m].astype(np.float64)[:, None] * np.repeat(b_s[:, kb].astype(np.float64), 128)[None, :]
        y += s * p
    return y


def grouped_gemm_w8a8(a, a_s, b, b_s, offsets) -> np.ndarray:
    """fp64 grouped GEMM: rows [off[g], off[g+1]) of a use b[g] ([G, n, k]) and b_s[g]."""
    a = np.ascontiguousarray(a, dtype=np.uint8)
    b = np.ascontiguousarray(b, dtype=np.uint8)
    a_s = np.ascontiguousarray(a_s, dtype=np.float32)
    b_s = np.ascontiguousarray(b_s, dtype=np.float32)
    off = np.ascontiguousarray(offsets, dtype=np.int32)
    m, k = a.shape
    g, n, _ = b.shape
    y = np.zeros((m, n), dtype=np.float64)
    _check(lib().oracle_grouped_gemm_w8a8(a, k, a_s, a_s.shape[1], b, b_s, off, g, y, n, n, k),
           "grouped_gemm_w8a8")
    return y


def kv_scales(k_bits, v_bits, slot_mapping, rng: float = 448.0):
    """Recalibrated (k_scale, v_scale) of a KV write call: fl32(amax / rng) over the
    tokens with slot >= 0 (1 when amax is 0).  k_bits, v_bits: bf16 [T, heads*head_dim]."""
    kx = _u16(k_bits)
    vx = _u16(v_bits)
    t = kx.shape[0]
    row = int(np.prod(kx.shape[1:])) if kx.ndim > 1 else 1
    ks = np.zeros(1, np.float32)
    vs = np.zeros(1, np.float32)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    _check(lib().oracle_kv_scales(kx.reshape(t, row), row, vx.reshape(t, row), row, t, row, slots, float(rng), ks, vs),
           "kv_scales")
    return ks[0], vs[0]


def kv_quant(k_bits, v_bits, slot_mapping, k_cache, v_cache, page_size: int,
             k_scale: float = 1.0, v_scale: float = 1.0, rng: float = 448.0,
             recalibrate: bool = True):
    """Quantize-on-write into copies of the paged caches.

    k_bits, v_bits: bf16 [T, heads, head_dim]; caches: uint8 [pages, page_size, heads, head_dim].
    Returns (k_cache', v_cache', k_scale', v_scale')."""
    kx = _u16(k_bits)
    vx = _u16(v_bits)
    t, heads, hd = kx.shape
    kc = np.array(k_cache, dtype=np.uint8, copy=True, order="C")
    vc = np.array(v_cache, dtype=np.uint8, copy=True, order="C")
    ks = np.array([k_scale], dtype=np.float32)
    vs = np.array([v_scale], dtype=np.float32)
    slots = np.ascontiguousarray(slot_mapping, dtype=np.int64)
    num_pages = kc.shape[0]
    _check(lib().oracle_kv_quant(kx.reshape(t, heads * hd), heads * hd, vx.reshape(t, heads * hd), heads * hd, t,
                                 heads, hd, slots, kc, vc, page_size, num_pages, ks, vs,
                                 float(rng), 1 if recalibrate else 0), "kv_quant")
    return kc, vc, ks[0], vs[0]


# ---------------------------------------------------------------- MoE layer around the grouped GEMM
# MoE routing-replay page, "Rollout Routing Replay" (section 4) and its cost analysis
# (section 5): the rollout keeps each token's top-k expert indices (int16) and tokens are
# dispatched to exactly those experts; [FP8-RL] step 1 quantizes fc1/fc2's inputs.

def moe_dispatch(xq: np.ndarray, xs: np.ndarray, topk_ids: np.ndarray, num_experts: int):
    """Dispatch quantized tokens to their recorded experts.

    xq: FP8 codes [T, K]; xs: fp32 scales [K/128, ld_s >= T]; topk_ids: int16 [T, topk].
    Entry f = t*topk + j (token t's j-th expert) is valid when 0 <= id < num_experts;
    invalid entries are dropped.  Valid entries are ordered by expert, and within an
    expert by f (a stable sort).  Returns (aq [R, K], as [K/128, R], offsets int32
    [E+1], row_of int32 [T, topk] = the sorted row of entry (t, j), -1 if dropped),
    R = number of valid entries."""
    ids = np.asarray(topk_ids).astype(np.int64)
    t, topk = ids.shape
    flat = ids.reshape(-1)
    valid = np.nonzero((flat >= 0) & (flat < num_experts))[0]
    order = valid[np.argsort(flat[valid], kind="stable")]
    counts = np.bincount(flat[valid], minlength=num_experts)
    offsets = np.zeros(num_experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    row_of = np.full(t * topk, -1, dtype=np.int32)
    row_of[order] = np.arange(order.size, dtype=np.int32)
    tok = order // topk
    aq = np.ascontiguousarray(np.asarray(xq)[tok])
    as_ = np.ascontiguousarray(np.asarray(xs)[:, tok])
    return aq, as_, offsets, row_of.reshape(t, topk)


def swiglu_quant_g128(h_bits: np.ndarray, ld_s: int | None = None, with_amax: bool = False,
                      ue8m0: bool = False):
    """silu(gate) * up of a bf16 fc1 output [m, 2n] (gate = first n columns), quantized
    in 1x128 groups -> (codes [m, n], scales [n/128, ld_s]) and, with_amax, the fp64
    group maxima [n/128, m].  ue8m0=True takes the power-of-two scale of each group's fp64
    maximum instead of fl32(amax/448)."""
    h = _u16(h_bits)
    m, n2 = h.shape
    n = n2 // 2
    ld_s = m if ld_s is None else ld_s
    q = np.empty((m, n), dtype=np.uint8)
    s = np.zeros((n // 128, ld_s), dtype=np.float32)
    amax = np.zeros((n // 128, m), dtype=np.float64)
    f = lib().oracle_swiglu_quant_g128_ue8m0 if ue8m0 else lib().oracle_swiglu_quant_g128
    _check(f(h, m, n, n2, q, n, s, ld_s, amax), "swiglu_quant_g128")
    return (q, s, amax) if with_amax else (q, s)


def silu_times_up(g: float, u: float) -> float:
    """The fp64 value silu(g) * u that swiglu_quant_g128 quantizes."""
    return float(lib().oracle_silu_times_up(float(g), float(u)))


def moe_combine(y_bits: np.ndarray, row_of: np.ndarray, weights: np.ndarray) -> np.ndarray:
    """out[t] = sum_j weights[t, j] * y[row_of[t, j]] in fp64, skipping row_of = -1.
    y: bf16 [R, H] (fc2 output rows in dispatch order); weights: fp32 [T, topk]."""
    y = np.asarray(y_bits)
    if y.dtype != np.uint16:
        raise TypeError("bf16 inputs are passed as uint16 bit patterns")
    yf = (y.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    rows = np.asarray(row_of).astype(np.int64)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    t, topk = rows.shape
    out = np.zeros((t, yf.shape[1]), dtype=np.float64)
    for j in range(topk):
        live = rows[:, j] >= 0
        out[live] += w[live, j][:, None] * yf[rows[live, j]]
    return out


# ---------------------------------------------------------------- FP8 paged decode attention
# FP8-RL summary page, "Method step details" step 3 (Q/K/V scales recalibrated every RL
# step) and "Experimental results" (full FP8: linear, KV cache and attention).

def q_scale(q_bits: np.ndarray, rng: float = 448.0) -> np.float32:
    """Recalibrated query scale fl32(amax / rng) over q bf16 [seqs, hq, 128] (1 if amax is 0)."""
    q = _u16(q_bits)
    seqs = q.shape[0]
    row = int(np.prod(q.shape[1:]))
    out = np.zeros(1, np.float32)
    _check(lib().oracle_q_scale(q.reshape(seqs, row), row, seqs, row // 128, float(rng), out), "q_scale")
    return out[0]


def paged_decode_attention(q_bits, k_cache, v_cache, block_table, seq_lens, q_scale_: float, k_scale: float,
                           v_scale: float, sm_scale: float) -> np.ndarray:
    """fp64 decode attention of q bf16 [seqs, hq, 128] over FP8 paged caches
    [pages, page_size, hkv, 128]; block_table int32 [seqs, ld_bt]; seq_lens int32 [seqs].
    Returns fp64 [seqs, hq, 128]."""
    q = _u16(q_bits)
    seqs, hq, d = q.shape
    kc = np.ascontiguousarray(k_cache, dtype=np.uint8)
    vc = np.ascontiguousarray(v_cache, dtype=np.uint8)
    pages, page_size, hkv, _ = kc.shape
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    sl = np.ascontiguousarray(seq_lens, dtype=np.int32)
    out = np.zeros((seqs, hq, d), np.float64)
    _check(lib().oracle_paged_decode_attention(q.reshape(seqs, hq * d), hq * d, kc.reshape(-1), vc.reshape(-1), bt,
                                               bt.shape[1], sl, seqs, hq, hkv, page_size, float(q_scale_),
                                               float(k_scale), float(v_scale), float(sm_scale), out),
           "paged_decode_attention")
    return out
