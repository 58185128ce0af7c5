"""GPU parity of MoE fc1 with SwiGLU and fc2's 1x128 quantization fused into the GEMM epilogue.

The fused call is defined as fp8q_grouped_gemm_w8a8 (bf16 output) followed by
fp8q_swiglu_quant_g128, so it must reproduce those two calls bit for bit: codes byte for
byte and scales bit for bit.  Rounding-location page, the SwiGLU fusion region (SiLU's
result is multiplied by up before any rounding); FP8-RL summary page, "Method step
details" step 1 (fc2's input is quantized per 1x128 group).  The small cases are also
checked against the oracle's SwiGLU quantization applied to the GEMM's own bf16 output
(the GEMM itself is pinned to the oracle by its own tests, within the GEMM tolerance).
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import swiglu_near_decisions, bf16_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _operands(sizes, n_half, k, seed):
    """Quantized fc1 inputs: tokens ~N(0,1) with outlier channels, expert weights ~N(0,0.02)."""
    g = len(sizes)
    off = np.zeros(g + 1, np.int32)
    off[1:] = np.cumsum(sizes)
    m = int(off[-1])
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    x = torch.randn((max(m, 1), k), device=DEV, generator=gen)
    x[:, 7] *= 40.0
    x = x.to(torch.bfloat16)[:m]
    w = (torch.randn((g * 2 * n_half, k), device=DEV, generator=gen) * 0.02).to(torch.bfloat16)
    aq = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    a_s = torch.empty((k // 128, max(m, 1)), dtype=torch.float32, device=DEV)
    if m:
        fq.fp8q_quant_act_g128(x, aq, a_s)
    bq = torch.empty((g * 2 * n_half, k), dtype=torch.uint8, device=DEV)
    b_s = torch.empty((g * 2 * n_half // 128, k // 128), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_weight_blk128([(w, bq, b_s)])
    return (aq, a_s, bq.view(g, 2 * n_half, k), b_s.view(g, 2 * n_half // 128, k // 128),
            torch.from_numpy(off).to(DEV), m)


def _both(aq, a_s, bq, b_s, off, m, n_half):
    y = torch.empty((m, 2 * n_half), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8(aq, a_s, bq, b_s, off, y)
    q1 = torch.full((m, n_half), 0x5A, dtype=torch.uint8, device=DEV)
    s1 = torch.full((n_half // 128, m + 3), -1.0, device=DEV)
    fq.fp8q_swiglu_quant_g128(y, q1, s1)
    q2 = torch.full((m, n_half), 0xA5, dtype=torch.uint8, device=DEV)
    s2 = torch.full((n_half // 128, m + 3), -2.0, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant(aq, a_s, bq, b_s, off, q2, s2)
    torch.cuda.synchronize()
    return y, q1, s1, q2, s2


@pytest.mark.parametrize("sizes,n_half,k", [
    ([3, 0, 300, 1, 0, 513, 64, 256], 256, 2048),   # empty, sub-tile, ragged multi-tile groups
    ([5, 130, 0, 77], 128, 256),                    # short K, one 128-output tile column
    ([260], 384, 1024),                             # one group, three tile columns
    ([40, 300], 256, 128),                          # one K step: the only step is also the last
    ([200, 128, 129, 0, 384, 255, 1], 256, 2048),   # 256- and 128-row tiles: remainders 200, 128, 129, 127, 1
])
def test_fused_equals_gemm_then_swiglu_and_the_oracle(sizes, n_half, k):
    aq, a_s, bq, b_s, off, m = _operands(sizes, n_half, k, seed=len(sizes) * 7 + k)
    y, q1, s1, q2, s2 = _both(aq, a_s, bq, b_s, off, m, n_half)
    assert torch.equal(q1, q2), f"codes differ at {int((q1 != q2).sum())} places"
    assert torch.equal(s1[:, :m].view(torch.int32), s2[:, :m].view(torch.int32)), "scales differ"
    assert torch.all(s2[:, m:] == -2.0), "scale columns past total_m are not written"
    # the oracle's SwiGLU quantization of the GEMM's own bf16 output
    q_ref, s_ref = oracle.swiglu_quant_g128(bf16_bits(y))
    assert swiglu_near_decisions(bf16_bits(y), s_ref) == (0, 0)
    assert np.array_equal(q2.cpu().numpy(), q_ref)
    assert np.array_equal(s2[:, :m].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_fused_equals_gemm_then_swiglu_at_the_moe_layer_shape():
    """128 experts, 4096 tokens routed top-8 (Zipf-skewed), hidden 2048, expert intermediate
    768: the full fused output against the two calls, every byte."""
    _, off_np, _ = synth.moe_routing(0)
    sizes = list(np.diff(off_np))
    aq, a_s, bq, b_s, off, m = _operands(sizes, 768, 2048, seed=11)
    _, q1, s1, q2, s2 = _both(aq, a_s, bq, b_s, off, m, 768)
    assert torch.equal(q1, q2), f"codes differ at {int((q1 != q2).sum())} places"
    assert torch.equal(s1[:, :m].view(torch.int32), s2[:, :m].view(torch.int32)), "scales differ"


def test_fused_with_no_rows_is_a_no_op():
    aq, a_s, bq, b_s, off, m = _operands([0, 0], 128, 256, seed=3)
    q = torch.empty((0, 128), dtype=torch.uint8, device=DEV)
    s = torch.empty((1, 1), dtype=torch.float32, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant(aq, a_s, bq, b_s, off, q, s)
    torch.cuda.synchronize()


@pytest.mark.parametrize("tokens,experts,topk,invalid", [(4096, 128, 8, 0), (300, 16, 4, 25)])
def test_route_and_token_rows_equal_the_dispatched_rows(tokens, experts, topk, invalid):
    """fp8q_moe_route writes dispatch's offsets and row_of plus row_token; fc1 reading the token
    rows through row_token gives the dispatched-row call's codes and scales, every byte.  The
    second case drops some entries (ids -1 and >= experts)."""
    ids_np, _ = synth.moe_topk(0, tokens=tokens, experts=experts, topk=topk)
    if invalid:
        g = np.random.default_rng(5)
        flat = ids_np.reshape(-1)
        pick = g.choice(flat.size, invalid, replace=False)
        flat[pick[: invalid // 2]] = -1
        flat[pick[invalid // 2:]] = experts + 3
    ids = torch.from_numpy(ids_np).to(DEV)
    n_half, k = 256, 512
    gen = torch.Generator(device=DEV)
    gen.manual_seed(tokens)
    x = torch.randn((tokens, k), device=DEV, generator=gen).to(torch.bfloat16)
    xq = torch.empty((tokens, k), dtype=torch.uint8, device=DEV)
    xs = torch.empty((k // 128, tokens), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128(x, xq, xs)
    n = tokens * topk
    dq = torch.empty((n, k), dtype=torch.uint8, device=DEV)
    ds = torch.empty((k // 128, n), dtype=torch.float32, device=DEV)
    off1 = torch.empty(experts + 1, dtype=torch.int32, device=DEV)
    row1 = torch.empty((tokens, topk), dtype=torch.int32, device=DEV)
    fq.fp8q_moe_dispatch(xq, xs, ids, experts, dq, ds, off1, row1)
    off2 = torch.full((experts + 1,), -7, dtype=torch.int32, device=DEV)
    row2 = torch.full((tokens, topk), -7, dtype=torch.int32, device=DEV)
    tok = torch.full((n,), -7, dtype=torch.int32, device=DEV)
    fq.fp8q_moe_route(ids, experts, off2, row2, tok)
    torch.cuda.synchronize()
    assert torch.equal(off1, off2) and torch.equal(row1, row2)
    rows = int(off2[-1].item())
    r = row2.reshape(-1)
    valid = r >= 0
    f = torch.arange(n, device=DEV)
    assert torch.equal(tok[r[valid].long()], (f[valid] // topk).to(torch.int32))
    w = (torch.randn((experts * 2 * n_half, k), device=DEV, generator=gen) * 0.02).to(torch.bfloat16)
    bq = torch.empty((experts * 2 * n_half, k), dtype=torch.uint8, device=DEV)
    bs = torch.empty((experts * 2 * n_half // 128, k // 128), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_weight_blk128([(w, bq, bs)])
    bq, bs = bq.view(experts, 2 * n_half, k), bs.view(experts, 2 * n_half // 128, k // 128)
    q1 = torch.empty((rows, n_half), dtype=torch.uint8, device=DEV)
    s1 = torch.empty((n_half // 128, rows), dtype=torch.float32, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant(dq[:rows], ds[:, :rows], bq, bs, off1, q1, s1)
    q2 = torch.full((rows, n_half), 0x5A, dtype=torch.uint8, device=DEV)
    s2 = torch.full((n_half // 128, rows), -1.0, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant(xq, xs, bq, bs, off2, q2, s2, row_token=tok)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2), f"codes differ at {int((q1 != q2).sum())} places"
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32))


def test_fused_with_padded_output_strides():
    """q and s with leading dimensions beyond n_half and total_m: the padding is left alone."""
    aq, a_s, bq, b_s, off, m = _operands([70, 0, 190], 256, 512, seed=21)
    y = torch.empty((m, 512), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8(aq, a_s, bq, b_s, off, y)
    q1 = torch.empty((m, 256), dtype=torch.uint8, device=DEV)
    s1 = torch.empty((2, m), dtype=torch.float32, device=DEV)
    fq.fp8q_swiglu_quant_g128(y, q1, s1)
    qbuf = torch.full((m, 256 + 48), 0x33, dtype=torch.uint8, device=DEV)
    sbuf = torch.full((2, m + 40), -5.0, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant(aq, a_s, bq, b_s, off, qbuf[:, :256], sbuf[:, :m])
    torch.cuda.synchronize()
    assert torch.equal(qbuf[:, :256], q1) and torch.all(qbuf[:, 256:] == 0x33)
    assert torch.equal(sbuf[:, :m].view(torch.int32), s1.view(torch.int32)) and torch.all(sbuf[:, m:] == -5.0)
