"""Shared helpers for the GPU parity tests: host<->device byte transfers and the GEMM
acceptance gate.  No arithmetic of the method lives here."""
import os

import numpy as np
import torch

# (test id, element count, worst err/bound, normwise error) of every gate evaluation,
# listed at the end of the run by conftest's terminal summary
GATE_MARGINS = []


def to_dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def u8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def f32(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v|: 2^(floor(log2|v|) - 7), 2^-133 below 2^-126."""
    a = np.abs(v)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -126.0)
    return np.exp2(e - 7.0)


def gemm_gate(y_gpu_bits: np.ndarray, y_ref: np.ndarray, rel: float = 2e-3):
    """Acceptance gate for bf16 GEMM outputs against the fp64 oracle: every element
    within half a bf16 ulp of the exact value plus rel * max|y_ref|.
    Returns (ok, worst ratio err/bound, normwise relative error)."""
    y = bf16_to_f64(y_gpu_bits)
    err = np.abs(y - y_ref)
    bound = 0.5 * ulp_bf16(y_ref) + rel * np.max(np.abs(y_ref))
    ratio = float(np.max(err / bound)) if err.size else 0.0
    nrm = float(np.linalg.norm(y - y_ref) / max(np.linalg.norm(y_ref), 1e-300)) if err.size else 0.0
    test = os.environ.get("PYTEST_CURRENT_TEST", "?").split(" ")[0]
    GATE_MARGINS.append((test, int(err.size), ratio, nrm))
    return bool(np.all(err <= bound)), ratio, nrm


def _e4m3_midpoints() -> np.ndarray:
    """Midpoints between adjacent non-negative finite E4M3FN values (from torch's decode)."""
    v = torch.arange(0, 0x7F, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    return (v[1:] + v[:-1]) / 2


def swiglu_near_decisions(h_bits: np.ndarray, scales: np.ndarray, rel: float = 2.0 ** -44):
    """How many SwiGLU-quantization decisions of bf16 [m, 2n] = [gate | up] input lie within
    ``rel`` (relative) of a boundary, with silu(g)*u formed here by numpy's fp64 exp: group
    amax/448 against fp32 rounding boundaries, and quotients a/scale against E4M3 midpoints.
    The GPU and the oracle each form the fp64 value with their own exp; when this returns
    (0, 0), exp results a few ulps apart cannot change a scale or a code.
    scales: fp32 [n/128, >= m] (the call's scale layout)."""
    h = bf16_to_f64(h_bits)
    m, n2 = h.shape
    n = n2 // 2
    g, u = h[:, :n], h[:, n:]
    with np.errstate(over="ignore", invalid="ignore"):
        a = g / (1.0 + np.exp(-g)) * u
    amax = np.abs(a).reshape(m, n // 128, 128).max(axis=2)
    v = amax / 448.0
    with np.errstate(over="ignore"):  # a power-of-two call's group maximum may exceed 448 * FLT_MAX
        f32 = v.astype(np.float32)
    up = np.nextafter(f32, np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(f32, np.float32(0)).astype(np.float64)
    f = f32.astype(np.float64)
    near_scale = (v > 0) & ((np.abs((f + up) / 2 - v) <= v * rel) | (np.abs((f + dn) / 2 - v) <= v * rel))
    s = np.repeat(np.asarray(scales, np.float32)[:, :m].T.astype(np.float64), 128, axis=1)
    qv = np.abs(a) / s
    mids = _e4m3_midpoints()
    i = np.clip(np.searchsorted(mids, qv), 1, len(mids) - 1)
    d = np.minimum(np.abs(mids[i] - qv), np.abs(mids[i - 1] - qv))
    near_code = (qv > 0) & (qv < 464) & (d <= qv * rel)
    return int(near_scale.sum()), int(near_code.sum())
