"""GPU parity of the few-token GEMM with the activation quantization fused into its operand
load (FP8-RL summary page, "Method step details" step 1: activations quantized on every
forward).

The fused call must be bit-identical to the activation quantizer followed by the GEMM (same
codes, scales and accumulation order), and within the GEMM gate of the oracle (half a bf16
ulp of the exact value plus 2e-3 of max|y|) applied to the oracle's own quantization.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import bf16_bits, gemm_gate, to_dev_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _weight(n, k, tensor):
    wq, ws = oracle.quant_weight_blk128(synth.weight(2, 0, tensor, n, k))
    return torch.from_numpy(wq).to(DEV), torch.from_numpy(ws).to(DEV), wq, ws


@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (5, 1024, 4096), (16, 4096, 4096), (17, 1024, 512),
                                   (33, 4096, 4096), (64, 1024, 4096), (64, 12288, 4096), (16, 256, 256),
                                   (12, 6144, 1024), (40, 12288, 1024)])  # last two: 32 weight rows per workgroup
def test_fused_equals_quantize_then_gemm(m, n, k):
    x_bits = synth.activation(2, 0, 200 + m, m, k)
    b, bs, wq, ws = _weight(n, k, n // 128 + m)
    x = to_dev_bf16(x_bits)
    y_fused = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_bf16act(x, b, bs, y_fused)
    xq = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    xs = torch.empty((k // 128, m), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128(x, xq, xs)
    y_two = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_blkscaled(xq, xs, b, bs, y_two)
    torch.cuda.synchronize()
    got = bf16_bits(y_fused)
    assert np.array_equal(got, bf16_bits(y_two)), "fused result differs from quantize + GEMM"
    rq, rs = oracle.quant_act_g128(x_bits)
    ok, ratio, _ = gemm_gate(got, oracle.gemm_w8a8(rq, rs, wq, ws))
    assert ok, f"worst err/bound {ratio:.3f}"


def test_fused_padded_rows_and_zero_rows():
    m, n, k = 9, 512, 1024
    x_bits = synth.activation(2, 1, 7, m, k)
    x_bits[3] = 0                      # an all-zero row: scale 1, zero output row
    x_bits[4, 128:256] = 0x8000        # a group of -0
    b, bs, wq, ws = _weight(n, k, 3)
    xp = torch.zeros((m, k + 64), dtype=torch.bfloat16, device=DEV)
    xp[:, :k] = to_dev_bf16(x_bits)
    yp = torch.full((m, n + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_bf16act(xp[:, :k], b, bs, yp[:, :n])
    torch.cuda.synchronize()
    got = bf16_bits(yp[:, :n])
    assert torch.isnan(yp[:, n:].float()).all()
    assert np.all(got[3] & 0x7FFF == 0)
    rq, rs = oracle.quant_act_g128(x_bits)
    ok, ratio, _ = gemm_gate(got, oracle.gemm_w8a8(rq, rs, wq, ws))
    assert ok, f"worst err/bound {ratio:.3f}"


def test_fused_zero_tokens_is_a_no_op():
    b, bs, _, _ = _weight(256, 256, 4)
    fq.fp8q_gemm_w8a8_bf16act(torch.empty((0, 256), dtype=torch.bfloat16, device=DEV), b, bs,
                              torch.empty((0, 256), dtype=torch.bfloat16, device=DEV))
    torch.cuda.synchronize()


@pytest.mark.parametrize("m,n,k", [(1, 4096, 4096), (17, 1024, 512), (33, 4096, 4096), (64, 1024, 4096),
                                   (12, 6144, 1024)])
def test_fused_ue8m0_equals_quantize_then_gemm(m, n, k):
    """Power-of-two scales: the fused call equals fp8q_quant_act_g128_ue8m0 followed by
    fp8q_gemm_w8a8_ue8m0 bit for bit, and passes the GEMM gate of the oracle's UE8M0 path."""
    x_bits = synth.activation(2, 0, 300 + m, m, k)
    wq, ws = oracle.quant_weight_blk128(synth.weight(2, 0, n // 128 + m + 1, n, k), ue8m0=True)
    b, bs = torch.from_numpy(wq).to(DEV), torch.from_numpy(ws).to(DEV)
    x = to_dev_bf16(x_bits)
    y_fused = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_bf16act_ue8m0(x, b, bs, y_fused)
    xq = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    xs = torch.empty((k // 128, m), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128_ue8m0(x, xq, xs)
    y_two = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_ue8m0(xq, xs, b, bs, y_two)
    torch.cuda.synchronize()
    got = bf16_bits(y_fused)
    assert np.array_equal(got, bf16_bits(y_two)), "fused result differs from quantize + GEMM"
    rq, rs = oracle.quant_act_g128(x_bits, ue8m0=True)
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(xs.cpu().numpy(), rs)
    ok, ratio, _ = gemm_gate(got, oracle.gemm_w8a8(rq, rs, wq, ws))
    assert ok, f"worst err/bound {ratio:.3f}"
