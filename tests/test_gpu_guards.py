"""Guard bands and launch-geometry determinism of every entry point.

Guard bands: each output buffer is carved out of a larger byte buffer whose 4 KB before and
after it are filled with 0xA5; after the call those bytes must be unchanged (the kernels
write only inside their outputs, for ragged shapes and every tile configuration).

Determinism across launch geometries: results that do not depend on the tile shape must
not depend on it.  Quantization is per block or row group, so quantizing a slice of rows
gives the bytes of the whole call's slice; and every GEMM tile configuration for M >= 1024
(256x256, 128x128 four-stage and two-stage) and the grouped GEMM run each output's K loop as
the same sequence of MFMAs and promotions, so their outputs agree bit for bit.
"""
import numpy as np
import pytest
import torch

import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import to_dev_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
GUARD = 4096


def guarded(shape, dtype, fill=0xA5):
    """(backing byte buffer, view of `shape` and `dtype` starting GUARD bytes in)."""
    n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
    buf = torch.full((2 * GUARD + n,), fill, dtype=torch.uint8, device=DEV)
    return buf, buf[GUARD:GUARD + n].view(dtype).view(shape)


def assert_intact(*bufs):
    torch.cuda.synchronize()
    for buf in bufs:
        assert torch.all(buf[:GUARD] == 0xA5), "guard band before the output was written"
        assert torch.all(buf[-GUARD:] == 0xA5), "guard band after the output was written"


def _codes(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    c = torch.randint(0, 0x7E, shape, dtype=torch.uint8, device=DEV, generator=g)
    return c | (torch.randint(0, 2, shape, dtype=torch.uint8, device=DEV, generator=g) << 7)


def _scales(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    return torch.rand(shape, device=DEV, generator=g) * 1e-2 + 1e-4


def test_quantizer_guards():
    n, k, m = 384, 640, 37
    w = to_dev_bf16(synth.weight(6, 0, 0, n, k))
    bq, q = guarded((n, k), torch.uint8)
    bs, s = guarded((n // 128, k // 128), torch.float32)
    fq.fp8q_quant_weight_blk128([(w, q, s)])
    fq.fp8q_quant_weight_blk128_ue8m0([(w, q, s)])
    assert_intact(bq, bs)
    x = to_dev_bf16(synth.activation(6, 0, 1, m, k))
    bq, q = guarded((m, k), torch.uint8)
    bs, s = guarded((k // 128, m), torch.float32)
    fq.fp8q_quant_act_g128(x, q, s)
    fq.fp8q_quant_act_g128_ue8m0(x, q, s)
    assert_intact(bq, bs)


@pytest.mark.parametrize("m,n,k", [
    (37, 256, 384),      # few tokens
    (40, 12288, 256),    # few tokens, 64 tokens x 48 weight rows per workgroup
    (40, 6272, 256),     # few tokens, 64 x 32
    (20, 12288, 256),    # few tokens, 32 x 48
    (20, 6272, 256),     # few tokens, 32 x 32
    (12, 6144, 256),     # few tokens, 16 x 16 (fused activation quantization: 16 x 32)
    (300, 512, 1152),    # few tiles (24 of 128x64): the few-token kernel
    (500, 1024, 1024),   # few tiles, 64 x 32
    (300, 4096, 1152),   # 128x64 tiles in two K groups
    (700, 1024, 640),    # 128x64 tiles, one K group
    (1100, 256, 384),    # 128x128 tiles
    (4000, 4096, 256),   # 256x256 tiles, ragged
    (4000, 4096, 2048),  # 256x256 tiles, ragged; power-of-two scales: the ping-pong tile
])
def test_gemm_guards(m, n, k):
    a, b = _codes((m, k), 1), _codes((n, k), 2)
    a_s, b_s = _scales((k // 128, m), 3), _scales((n // 128, k // 128), 4)
    by, y = guarded((m, n), torch.bfloat16)
    fq.fp8q_gemm_w8a8_blkscaled(a, a_s, b, b_s, y)
    if m > 64:
        b_s2 = torch.full_like(b_s, 0.25)
        a_s2 = torch.full_like(a_s, 2.0 ** -7)
        fq.fp8q_gemm_w8a8_ue8m0(a, a_s2, b, b_s2, y)
    else:
        x = to_dev_bf16(synth.activation(6, 0, 2, m, k))
        fq.fp8q_gemm_w8a8_bf16act(x, b, b_s, y)
    assert_intact(by)


def test_grouped_and_fused_guards():
    sizes = [200, 0, 129, 1, 300]
    off = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32, device=DEV)
    m, g, k, half = sum(sizes), len(sizes), 2048, 256
    a, a_s = _codes((m, k), 5), _scales((k // 128, m), 6)
    b, b_s = _codes((g, 2 * half, k), 7), _scales((g, 2 * half // 128, k // 128), 8)
    by, y = guarded((m, 2 * half), torch.bfloat16)
    fq.fp8q_grouped_gemm_w8a8(a, a_s, b, b_s, off, y)
    bq, q = guarded((m, half), torch.uint8)
    bs, s = guarded((half // 128, m), torch.float32)
    fq.fp8q_grouped_gemm_swiglu_quant(a, a_s, b, b_s, off, q, s)
    bq2, q2 = guarded((m, half), torch.uint8)
    bs2, s2 = guarded((half // 128, m), torch.float32)
    fq.fp8q_swiglu_quant_g128(y, q2, s2)
    assert_intact(by, bq, bs, bq2, bs2)
    assert torch.equal(q, q2) and torch.equal(s, s2)


def test_moe_helpers_guards():
    t, topk, e, k = 300, 8, 16, 256
    ids_np, w_np = synth.moe_topk(2, tokens=t, experts=e, topk=topk)
    ids = torch.from_numpy(ids_np).to(DEV)
    rw = torch.from_numpy(w_np).to(DEV)
    xq, xs = _codes((t, k), 9), _scales((k // 128, t), 10)
    n = t * topk
    baq, aq = guarded((n, k), torch.uint8)
    bas, a_s = guarded((k // 128, n), torch.float32)
    boff, off = guarded((e + 1,), torch.int32)
    brow, row_of = guarded((t, topk), torch.int32)
    fq.fp8q_moe_dispatch(xq, xs, ids, e, aq, a_s, off, row_of)
    brt, row_token = guarded((n,), torch.int32)
    fq.fp8q_moe_route(ids, e, off, row_of, row_token)
    y = torch.randn((n, 512), device=DEV).to(torch.bfloat16)
    bout, out = guarded((t, 512), torch.bfloat16)
    fq.fp8q_moe_combine(y, row_of, rw, out)
    assert_intact(baq, bas, boff, brow, brt, bout)


def test_kv_and_attention_guards():
    t, h, pages, ps = 100, 8, 12, 16
    k = to_dev_bf16(synth.activation(6, 1, 0, t, h * 128)).view(t, h, 128)
    v = to_dev_bf16(synth.activation(6, 1, 1, t, h * 128)).view(t, h, 128)
    slots = torch.randperm(pages * ps, device=DEV)[:t].to(torch.int64)
    slots[::7] = -1
    bkc, kc = guarded((pages, ps, h, 128), torch.uint8, fill=0x7F)
    bvc, vc = guarded((pages, ps, h, 128), torch.uint8, fill=0x7F)
    bkc[:GUARD] = 0xA5
    bkc[-GUARD:] = 0xA5
    bvc[:GUARD] = 0xA5
    bvc[-GUARD:] = 0xA5
    bks, ks = guarded((1,), torch.float32)
    bvs, vs = guarded((1,), torch.float32)
    fq.fp8q_kv_quant(k, v, slots, kc, vc, ks, vs, 448.0, recalibrate=True)
    assert_intact(bkc, bvc, bks, bvs)
    seqs, hq = 3, 16
    q = to_dev_bf16(synth.activation(6, 1, 2, seqs, hq * 128)).view(seqs, hq, 128)
    bt = torch.tensor([[0, 1, 2, 3], [4, 5, 6, 7], [8, 9, 10, 11]], dtype=torch.int32, device=DEV)
    lens = torch.tensor([64, 17, 1], dtype=torch.int32, device=DEV)
    kc.fill_(0x38)
    vc.fill_(0x30)
    bout, out = guarded((seqs, hq, 128), torch.bfloat16)
    bqs, qs = guarded((1,), torch.float32)
    fq.fp8q_paged_decode_attention(q, kc, vc, bt, lens, qs, ks, vs, 128 ** -0.5, out, recalibrate_q=True)
    assert_intact(bout, bqs)


def test_quantizers_independent_of_launch_geometry():
    """A row slice quantized alone gives the whole call's bytes for those rows; a weight
    quantized alone gives the bytes it gets inside a batched call of several tensors."""
    m, k = 4096, 1024
    x = to_dev_bf16(synth.activation(6, 2, 0, m, k))
    q = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    s = torch.empty((k // 128, m), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128(x, q, s)
    for r0, r1 in ((0, 1), (100, 137), (4000, 4096)):
        qs = torch.empty((r1 - r0, k), dtype=torch.uint8, device=DEV)
        ss = torch.empty((k // 128, r1 - r0), dtype=torch.float32, device=DEV)
        fq.fp8q_quant_act_g128(x[r0:r1], qs, ss)
        assert torch.equal(qs, q[r0:r1]) and torch.equal(ss, s[:, r0:r1])
    ws = [to_dev_bf16(synth.weight(6, 2, i, n, 512)) for i, n in enumerate((256, 1024, 128))]
    outs = [(torch.empty(w.shape, dtype=torch.uint8, device=DEV),
             torch.empty((w.shape[0] // 128, 4), dtype=torch.float32, device=DEV)) for w in ws]
    fq.fp8q_quant_weight_blk128([(w, o[0], o[1]) for w, o in zip(ws, outs)])
    for w, (qb, sb) in zip(ws, outs):
        q1 = torch.empty_like(qb)
        s1 = torch.empty_like(sb)
        fq.fp8q_quant_weight_blk128([(w, q1, s1)])
        assert torch.equal(q1, qb) and torch.equal(s1, sb)


def test_gemm_independent_of_tile_configuration():
    """Rows 0..1099 of a 4096-row GEMM (256x256 tiles) equal a 1100-row GEMM (128x128 tiles,
    four-stage ring) and a 2048-row one (128x128, two-stage ring), bit for bit; and the
    grouped GEMM's rows of one expert equal the dense GEMM of those rows with its weight."""
    n, k = 4096, 1024
    a, b = _codes((4096, k), 11), _codes((n, k), 12)
    a_s, b_s = _scales((k // 128, 4096), 13), _scales((n // 128, k // 128), 14)
    ys = {}
    for m in (4096, 2048, 1100):
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        fq.fp8q_gemm_w8a8_blkscaled(a[:m], a_s[:, :m].contiguous(), b, b_s, y)
        ys[m] = y
    torch.cuda.synchronize()
    assert torch.equal(ys[2048][:1100].view(torch.int16), ys[1100].view(torch.int16))
    assert torch.equal(ys[4096][:2048].view(torch.int16), ys[2048].view(torch.int16))
    # grouped, K >= 2048: 256- and 128-row tiles; rows of expert 1 against the dense GEMM
    k2, n2 = 2048, 512
    sizes = [300, 1100, 90]
    off = torch.tensor(np.concatenate([[0], np.cumsum(sizes)]), dtype=torch.int32, device=DEV)
    m2 = sum(sizes)
    a2, a2_s = _codes((m2, k2), 15), _scales((k2 // 128, m2), 16)
    b2, b2_s = _codes((3, n2, k2), 17), _scales((3, n2 // 128, k2 // 128), 18)
    yg = torch.empty((m2, n2), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8(a2, a2_s, b2, b2_s, off, yg)
    yd = torch.empty((1100, n2), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_blkscaled(a2[300:1400], a2_s[:, 300:1400].contiguous(), b2[1], b2_s[1], yd)
    torch.cuda.synchronize()
    assert torch.equal(yg[300:1400].view(torch.int16), yd.view(torch.int16))


def test_ue8m0_gemm_independent_of_tile_configuration():
    """Power-of-two scales, K = 2048: rows of a 4096-row GEMM (ping-pong 256x256 tiles) equal
    a 4000-row one (the same, ragged), a 2048-row one (128x128 tiles, two-stage ring) and a
    1100-row one (128x128, four-stage ring), bit for bit."""
    n, k = 4096, 2048
    a, b = _codes((4096, k), 21), _codes((n, k), 22)
    a_s = torch.exp2(torch.round(torch.log2(_scales((k // 128, 4096), 23))))
    b_s = torch.exp2(torch.round(torch.log2(_scales((n // 128, k // 128), 24))))
    ys = {}
    for m in (4096, 4000, 2048, 1100):
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        fq.fp8q_gemm_w8a8_ue8m0(a[:m], a_s[:, :m].contiguous(), b, b_s, y)
        ys[m] = y
    torch.cuda.synchronize()
    assert torch.equal(ys[4096][:4000].view(torch.int16), ys[4000].view(torch.int16))
    assert torch.equal(ys[4096][:2048].view(torch.int16), ys[2048].view(torch.int16))
    assert torch.equal(ys[2048][:1100].view(torch.int16), ys[1100].view(torch.int16))
