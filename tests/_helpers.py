"""Shared helpers for the GPU parity tests: host<->device byte transfers and the GEMM
acceptance gate.  No arithmetic of the method lives here."""
import numpy as np
import torch


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
    return bool(np.all(err <= bound)), ratio, nrm
