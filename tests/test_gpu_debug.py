"""Debug mode (FP8Q_DEBUG=1): the documented preconditions are checked before anything is
enqueued, and valid calls give the same results as without it.

Every violating call below is built so that, were it launched anyway, its kernels would
stay inside allocated memory: overlapping outputs alias buffers the call owns, bad group
offsets stay within [0, total_m], out-of-range KV slots and page ids point into pages that
are allocated but not declared, and an over-long sequence reads the next row of an
allocated block table.
"""
import pytest
import torch

import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import to_dev_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture
def debug(monkeypatch):
    monkeypatch.setenv("FP8Q_DEBUG", "1")


def _expect(status, fn, *args, **kw):
    with pytest.raises(fq.Fp8qError) as e:
        fn(*args, **kw)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def _act(m, k, seed=0):
    return to_dev_bf16(synth.activation(4, 9, seed, m, k))


def _codes(shape, seed):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    c = torch.randint(0, 0x7E, shape, dtype=torch.uint8, device=DEV, generator=g)
    return c | (torch.randint(0, 2, shape, dtype=torch.uint8, device=DEV, generator=g) << 7)


def test_valid_calls_match_normal_mode(monkeypatch):
    m, n, k = 40, 256, 384
    x = _act(m, k)
    w = to_dev_bf16(synth.weight(4, 9, 1, n, k))
    outs = {}
    for mode in ("0", "1"):
        monkeypatch.setenv("FP8Q_DEBUG", mode)
        xq = torch.empty((m, k), dtype=torch.uint8, device=DEV)
        xs = torch.empty((k // 128, m), dtype=torch.float32, device=DEV)
        fq.fp8q_quant_act_g128(x, xq, xs)
        wq = torch.empty((n, k), dtype=torch.uint8, device=DEV)
        ws = torch.empty((n // 128, k // 128), dtype=torch.float32, device=DEV)
        fq.fp8q_quant_weight_blk128([(w, wq, ws)])
        y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        fq.fp8q_gemm_w8a8_blkscaled(xq, xs, wq, ws, y)
        off = torch.tensor([0, 15, 15, 40], dtype=torch.int32, device=DEV)
        yg = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
        fq.fp8q_grouped_gemm_w8a8(xq, xs, torch.stack([wq] * 3), torch.stack([ws] * 3), off, yg)
        torch.cuda.synchronize()
        outs[mode] = [t.cpu() for t in (xq, xs, wq, ws, y, yg)]
    for a, b in zip(outs["0"], outs["1"]):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8))


def test_overlapping_output_is_rejected(debug):
    m, k = 8, 256
    x = _act(m, k)
    q = x.view(torch.uint8)[:, :k]  # codes written over the input's own bytes
    s = torch.empty((k // 128, m), dtype=torch.float32, device=DEV)
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_quant_act_g128, x, q, s)
    assert "overlaps" in msg


def test_non_finite_input_is_rejected(debug):
    x = _act(4, 256)
    x[2, 77] = float("nan")
    q = torch.empty((4, 256), dtype=torch.uint8, device=DEV)
    s = torch.empty((2, 4), dtype=torch.float32, device=DEV)
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_quant_act_g128, x, q, s)
    assert "x[2][77]" in msg


def test_gemm_nan_code_and_bad_ue8m0_scale_are_rejected(debug):
    m, n, k = 16, 128, 256
    a, b = _codes((m, k), 1), _codes((n, k), 2)
    a_s = torch.full((k // 128, m), 0.5, device=DEV)
    b_s = torch.full((n // 128, k // 128), 0.25, device=DEV)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_ue8m0(a, a_s, b, b_s, y)  # powers of two: accepted
    a_s[1, 3] = 0.3
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_gemm_w8a8_ue8m0, a, a_s, b, b_s, y)
    assert "power of two" in msg
    # 2^-127 (the smallest E8M0 scale, a binary32 subnormal) is accepted; 2^-130 has no
    # E8M0 code and is rejected
    a_s[1, 3] = 2.0 ** -127
    fq.fp8q_gemm_w8a8_ue8m0(a, a_s, b, b_s, y)
    a_s[1, 3] = 2.0 ** -130
    assert a_s[1, 3].item() == 2.0 ** -130
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_gemm_w8a8_ue8m0, a, a_s, b, b_s, y)
    assert "a_s[1][3]" in msg
    a_s[1, 3] = 0.5
    b[5, 9] = 0xFF
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_gemm_w8a8_blkscaled, a, a_s, b, b_s, y)
    assert "NaN code" in msg


@pytest.mark.parametrize("offsets,what", [([0, 200, 100, 300], "decrease"), ([0, 100, 200, 250], "total_m"),
                                          ([5, 100, 200, 300], "not 0")])
def test_bad_group_offsets_are_rejected(debug, offsets, what):
    total, n, k = 300, 128, 256
    a = _codes((total, k), 3)
    a_s = torch.ones((k // 128, total), device=DEV)
    b = _codes((3, n, k), 4)
    b_s = torch.ones((3, n // 128, k // 128), device=DEV)
    y = torch.empty((total, n), dtype=torch.bfloat16, device=DEV)
    off = torch.tensor(offsets, dtype=torch.int32, device=DEV)
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_grouped_gemm_w8a8, a, a_s, b, b_s, off, y)
    assert what in msg


def test_kv_slot_beyond_declared_pages_is_rejected(debug):
    t, heads, ps, declared = 5, 2, 16, 3
    k = torch.randn((t, heads, 128), device=DEV).to(torch.bfloat16)
    v = torch.randn((t, heads, 128), device=DEV).to(torch.bfloat16)
    kc_all = torch.zeros((declared + 2, ps, heads, 128), dtype=torch.uint8, device=DEV)
    vc_all = torch.zeros_like(kc_all)
    ks, vs = torch.zeros(1, device=DEV), torch.zeros(1, device=DEV)
    slots = torch.tensor([0, 5, -1, 47, 3], dtype=torch.int64, device=DEV)
    fq.fp8q_kv_quant(k, v, slots, kc_all[:declared], vc_all[:declared], ks, vs, recalibrate=True)
    slots[3] = declared * ps  # the first slot of an allocated but undeclared page
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_kv_quant, k, v, slots, kc_all[:declared],
                  vc_all[:declared], ks, vs, recalibrate=True)
    assert "slot_mapping[3]" in msg


def test_attention_bad_page_id_and_length_are_rejected(debug):
    seqs, hq, hkv, ps, per, declared = 2, 8, 2, 16, 3, 6
    kc = _codes((declared + 2, ps, hkv, 128), 5)
    vc = _codes((declared + 2, ps, hkv, 128), 6)
    table = torch.tensor([[0, 1, 2], [3, 4, 5], [0, 0, 0]], dtype=torch.int32, device=DEV)
    q = torch.randn((seqs, hq, 128), device=DEV).to(torch.bfloat16)
    out = torch.empty((seqs, hq, 128), dtype=torch.bfloat16, device=DEV)
    qs, ks, vs = torch.tensor([0.01], device=DEV), torch.tensor([0.02], device=DEV), torch.tensor([0.02], device=DEV)
    lens = torch.tensor([40, 33], dtype=torch.int32, device=DEV)
    args = (q, kc[:declared], vc[:declared], table[:seqs], lens, qs, ks, vs, 0.088, out)
    fq.fp8q_paged_decode_attention(*args)
    table[1, 2] = declared  # an allocated but undeclared page
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_paged_decode_attention, *args)
    assert "block_table[1][2]" in msg
    table[1, 2] = 5
    lens[0] = per * ps + 1  # one token past its row of the table
    msg = _expect(fq.FP8Q_ERR_PRECONDITION, fq.fp8q_paged_decode_attention, *args)
    assert "seq_lens[0]" in msg


# the refused call leaves the capture empty, which torch reports with a warning
@pytest.mark.filterwarnings("ignore:The CUDA Graph is empty")
def test_debug_mode_refuses_a_capturing_stream(debug):
    x = _act(4, 256)
    q = torch.empty((4, 256), dtype=torch.uint8, device=DEV)
    s = torch.empty((2, 4), dtype=torch.float32, device=DEV)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    with pytest.raises(fq.Fp8qError) as e:
        with torch.cuda.graph(g, stream=side):
            fq.fp8q_quant_act_g128(x, q, s)
    assert e.value.status == fq.FP8Q_ERR_UNSUPPORTED
    torch.cuda.synchronize()
