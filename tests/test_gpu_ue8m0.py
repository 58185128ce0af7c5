"""GPU parity of the power-of-two (UE8M0) scale variant against the oracle.

FP8-RL summary page, "Experimental results" (scale-format ablation: FP32 versus UE8M0
scales).  Quantizers: codes and scales bit-exact.  GEMMs (the matrix core applies the
E8M0 block scales): every element within half a bf16 ulp of the exact value plus 2e-3
of max|y|, as for the FP32-scale GEMM.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import bf16_bits, f32, gemm_gate, to_dev_bf16, u8

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _gpu_weight(w_bits):
    n, k = w_bits.shape
    w = to_dev_bf16(w_bits)
    q = torch.empty((n, k), dtype=torch.uint8, device=DEV)
    s = torch.empty((n // 128, k // 128), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_weight_blk128_ue8m0([(w, q, s)])
    torch.cuda.synchronize()
    return u8(q), f32(s)


def _gpu_act(x_bits, ld_s=None):
    m, k = x_bits.shape
    ld_s = m if ld_s is None else ld_s
    q = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    s = torch.full((k // 128, ld_s), -7.0, dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128_ue8m0(to_dev_bf16(x_bits), q, s)
    torch.cuda.synchronize()
    return u8(q), f32(s)


def _same(got, ref):
    (gq, gs), (rq, rs) = got, ref
    assert np.array_equal(gs.view(np.uint32), rs.view(np.uint32)), "scales differ"
    assert np.array_equal(gq, rq), f"{int(np.sum(gq != rq))} codes differ"


def test_weight_tiny_and_projection():
    w, _ = synth.tiny()
    _same(_gpu_weight(w), oracle.quant_weight_blk128(w, ue8m0=True))
    w = synth.weight(2, 0, 0, 4096, 4096)
    _same(_gpu_weight(w), oracle.quant_weight_blk128(w, ue8m0=True))


def test_weight_scale_edges():
    """All-zero block (scale 1), amax below the E8M0 range (clamped to 2^-127), the
    largest bf16 (2^120), an exact 448 * 2^k maximum, and blocks of subnormal bf16."""
    w = synth.weight(3, 0, 5, 256, 640)
    w[:128, :128] = 0
    w[:128, 128:256] = synth.to_bf16_bits(np.full((128, 128), 2.0 ** -133, np.float32))
    w[128:, 128:256] = synth.to_bf16_bits(np.linspace(-3e38, 3e38, 128 * 128, dtype=np.float32).reshape(128, 128))
    w[:128, 256:384] = synth.to_bf16_bits((np.arange(128 * 128, dtype=np.float32).reshape(128, 128) % 7) * 2.0 ** -130)
    w[128:, 256] = synth.to_bf16_bits(np.full(128, 448.0 * 2.0 ** -5, np.float32))
    ref = oracle.quant_weight_blk128(w, ue8m0=True)
    assert ref[1][0, 0] == 1.0 and ref[1][0, 1] == np.float32(2.0 ** -127) and ref[1][1, 1] == np.float32(2.0 ** 120)
    _same(_gpu_weight(w), ref)


@pytest.mark.parametrize("m,k", [(16, 256), (1, 4096), (77, 1024), (4096, 4096)])
def test_activation(m, k):
    x = synth.activation(2, 0, 60 + m, m, k)
    got = _gpu_act(x, ld_s=m + 3)
    ref = oracle.quant_act_g128(x, ld_s=m + 3, ue8m0=True)
    assert np.all(got[1][:, m:] == -7.0)  # padding of the scale rows untouched
    _same((got[0], got[1][:, :m]), (ref[0], ref[1][:, :m]))


def _operands(m, n, k, tensor):
    w = synth.weight(2, 0, tensor, n, k)
    x = synth.activation(2, 0, tensor + 50, m, k)
    wq, ws = oracle.quant_weight_blk128(w, ue8m0=True)
    xq, xs = oracle.quant_act_g128(x, ue8m0=True)
    return xq, xs, wq, ws


def _gpu_gemm(fn, xq, xs, wq, ws):
    m, k = xq.shape
    n = wq.shape[0]
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fn(torch.from_numpy(xq).to(DEV), torch.from_numpy(xs).to(DEV), torch.from_numpy(wq).to(DEV),
       torch.from_numpy(ws).to(DEV), y)
    torch.cuda.synchronize()
    return bf16_bits(y)


@pytest.mark.parametrize("m,n,k", [
    (16, 256, 256),      # few tokens: promotion path
    (130, 1024, 512),    # 128x64 tiles, ragged
    (1100, 1024, 1024),  # 128x128 tiles, four-stage ring, ragged
    (2000, 4096, 512),   # 128x128 tiles, two workgroups per CU, ragged
    (65536, 384, 256),   # 128x128 tiles, two workgroups per CU, n not a multiple of 256
    (4000, 4096, 1024),  # 256x256 tiles, ragged
    (4000, 4096, 128),   # 256x256 tiles, one K step
    (4000, 4096, 256),   # 256x256 tiles, two K steps
    (4000, 4096, 2048),  # ping-pong 256x256 tiles, ragged: the last tile's second half 32 rows
    (1030, 16384, 2048),  # ping-pong 256x256 tiles, the last tile's second half empty
    (4096, 2048, 4096),  # ping-pong 256x256 tiles, whole
])
def test_gemm_matches_oracle(m, n, k):
    xq, xs, wq, ws = _operands(m, n, k, tensor=n // 128 + m % 7)
    y = _gpu_gemm(fq.fp8q_gemm_w8a8_ue8m0, xq, xs, wq, ws)
    g = np.random.Generator(np.random.PCG64(m))
    rows = np.unique(np.concatenate([[0, m - 1], g.choice(m, min(m, 48), replace=False)]))
    ref = oracle.gemm_w8a8(xq[rows], xs[:, rows], wq, ws)
    ok, ratio, nrm = gemm_gate(y[rows], ref)
    assert ok, f"worst err/bound {ratio:.3f}"
    assert nrm < 4e-3


def _random_shapes(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    out = []
    for _ in range(count):
        m = int(g.choice([int(g.integers(1, 65)), int(g.integers(65, 1100)), int(g.integers(1100, 5000))]))
        out.append((m, 128 * int(g.integers(1, 33)), 128 * int(g.integers(1, 25))))
    return out


@pytest.mark.parametrize("m,n,k", _random_shapes(12, 88))
def test_gemm_random_shapes(m, n, k):
    """Seeded random shapes over every tile configuration, sampled rows against the oracle."""
    xq, xs, wq, ws = _operands(m, n, k, tensor=(m + n + k) % 11)
    y = _gpu_gemm(fq.fp8q_gemm_w8a8_ue8m0, xq, xs, wq, ws)
    g = np.random.Generator(np.random.PCG64(m + n))
    rows = np.unique(np.concatenate([[0, m - 1], g.choice(m, min(m, 40), replace=False)]))
    ok, ratio, nrm = gemm_gate(y[rows], oracle.gemm_w8a8(xq[rows], xs[:, rows], wq, ws))
    assert ok, f"worst err/bound {ratio:.3f}"
    assert nrm < 4e-3


def test_gemm_agrees_with_fp32_scale_path():
    """Power-of-two scales are valid FP32 scales: both GEMMs pass the same gate."""
    xq, xs, wq, ws = _operands(512, 1024, 2048, tensor=3)
    ref = oracle.gemm_w8a8(xq, xs, wq, ws)
    for fn in (fq.fp8q_gemm_w8a8_ue8m0, fq.fp8q_gemm_w8a8_blkscaled):
        ok, ratio, _ = gemm_gate(_gpu_gemm(fn, xq, xs, wq, ws), ref)
        assert ok, f"{fn.__name__}: worst err/bound {ratio:.3f}"


def test_grouped_with_empty_groups():
    sizes = [3, 0, 130, 1, 0, 257, 64]
    n, k = 256, 384
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m = int(off[-1])
    G = len(sizes)
    bq = np.empty((G, n, k), np.uint8)
    bs = np.empty((G, n // 128, k // 128), np.float32)
    for e in range(G):
        bq[e], bs[e] = oracle.quant_weight_blk128(synth.weight(4, 0, e, n, k, outlier_frac=0.0), ue8m0=True)
    aq, as_ = oracle.quant_act_g128(synth.activation(4, 0, 99, m, k), ue8m0=True)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8_ue8m0(torch.from_numpy(aq).to(DEV), torch.from_numpy(as_).to(DEV),
                                    torch.from_numpy(bq).to(DEV), torch.from_numpy(bs).to(DEV),
                                    torch.from_numpy(off).to(DEV), y)
    torch.cuda.synchronize()
    ref = oracle.grouped_gemm_w8a8(aq, as_, bq, bs, off)
    ok, ratio, _ = gemm_gate(bf16_bits(y), ref)
    assert ok, f"worst err/bound {ratio:.3f}"


def test_pingpong_padded_pitches():
    """The ping-pong 256x256 tile (K >= 2048) with every pitch padded (a, b, y rows; the token
    scale rows) gives the bytes it gives on contiguous buffers and leaves y's padding alone."""
    m, n, k = 1100, 16384, 2048
    g = torch.Generator(device=DEV)
    g.manual_seed(31)
    a_pad = torch.randint(0, 0x77, (m, k + 128), dtype=torch.uint8, device=DEV, generator=g)
    b_pad = torch.randint(0, 0x77, (n, k + 256), dtype=torch.uint8, device=DEV, generator=g)
    as_pad = torch.exp2(torch.randint(-12, -4, (k // 128, m + 5), device=DEV, generator=g).float())
    b_s = torch.exp2(torch.randint(-12, -4, (n // 128, k // 128), device=DEV, generator=g).float())
    a, b, a_s = a_pad[:, :k], b_pad[:, :k], as_pad[:, :m]
    y_pad = torch.full((m, n + 64), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_ue8m0(a, a_s, b, b_s, y_pad[:, :n])
    y = torch.empty((m, n), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_ue8m0(a.contiguous(), a_s.contiguous(), b.contiguous(), b_s, y)
    torch.cuda.synchronize()
    assert torch.equal(y_pad[:, :n].view(torch.int16), y.view(torch.int16))
    assert torch.isnan(y_pad[:, n:].float()).all()


# ------------------------------------------------- SwiGLU + 1x128 quantization, UE8M0
def _near_pow2_boundary(amax, rel=2.0 ** -44):
    """Groups whose fp64 amax lies within rel (relative) of 448 * 2^k for some k: there an
    exp result a few ulps away could move the power-of-two scale."""
    v = np.asarray(amax, np.float64) / 448.0
    with np.errstate(divide="ignore"):
        k = np.round(np.log2(np.where(v > 0, v, 1.0)))
    return (v > 0) & (np.abs(v - np.exp2(k)) <= v * rel)


def _check_swiglu_ue8m0(h, ld_s=None):
    from tests._helpers import swiglu_near_decisions
    m, n2 = h.shape
    n = n2 // 2
    ld_s = m if ld_s is None else ld_s
    q = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    s = torch.full((n // 128, ld_s), -5.0, dtype=torch.float32, device=DEV)
    fq.fp8q_swiglu_quant_g128_ue8m0(to_dev_bf16(h), q, s)
    torch.cuda.synchronize()
    gq, gs = u8(q), f32(s)
    rq, rs, amax = oracle.swiglu_quant_g128(h, ld_s=ld_s, with_amax=True, ue8m0=True)
    assert np.all(gs[:, m:] == -5.0)
    assert not np.any(_near_pow2_boundary(amax)), "a group maximum sits on a power-of-two boundary"
    assert swiglu_near_decisions(h, rs)[1] == 0, "a quotient sits on an E4M3 midpoint"
    assert np.array_equal(gs[:, :m].view(np.uint32), rs[:, :m].view(np.uint32)), "scales differ"
    bad = gq != rq
    assert not np.any(bad), f"{int(bad.sum())} codes differ"
    return rs


def test_swiglu_moe_fc2_input_shape():
    """fc1 output of the MoE layer: 32768 rows of [gate | up], 768 columns each."""
    g = synth.activation(4, 0, 80, 32768, 768, outlier_channels=0)
    u = synth.activation(4, 0, 81, 32768, 768)
    rs = _check_swiglu_ue8m0(np.concatenate([g, u], axis=1))
    e = np.log2(rs)
    assert np.all(e == np.round(e))


def test_swiglu_ragged_and_edges():
    m, n = 13, 384
    g = synth.activation(4, 1, 82, m, n)
    u = synth.activation(4, 1, 83, m, n)
    g[0, :128] = 0                                                            # zero group: scale 1
    g[1, 128:256] = synth.to_bf16_bits(np.full(128, 60.0, np.float32))      # saturated gate: a = g*u
    g[2, :128] = synth.to_bf16_bits(np.full(128, -900.0, np.float32))        # exp overflows: a = -0
    u[3, 256:] = synth.to_bf16_bits(np.full(128, 2.0 ** -130, np.float32))   # tiny group: the 2^-127 clamp
    g[4, 256:] = synth.to_bf16_bits(np.linspace(-3e38, 3e38, 128, dtype=np.float32))
    u[4, 256:] = synth.to_bf16_bits(np.full(128, 2.0 ** 100, np.float32))    # beyond 448 * 2^127: clamp, saturate
    rs = _check_swiglu_ue8m0(np.concatenate([g, u], axis=1), ld_s=m + 3)
    assert rs[0, 0] == 1.0 and rs[2, 3] == np.float32(2.0 ** -127) and rs[2, 4] == np.float32(2.0 ** 127)


def _fused_operands(sizes, n_half, k, seed):
    """fc1 inputs quantized with power-of-two scales: tokens ~N(0,1) with an outlier channel,
    expert weights ~N(0,0.02)."""
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
        fq.fp8q_quant_act_g128_ue8m0(x, aq, a_s)
    bq = torch.empty((g * 2 * n_half, k), dtype=torch.uint8, device=DEV)
    b_s = torch.empty((g * 2 * n_half // 128, k // 128), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_weight_blk128_ue8m0([(w, bq, b_s)])
    return (aq, a_s, bq.view(g, 2 * n_half, k), b_s.view(g, 2 * n_half // 128, k // 128),
            torch.from_numpy(off).to(DEV), m)


@pytest.mark.parametrize("sizes,n_half,k", [
    ([3, 0, 300, 1, 0, 513, 64, 256], 256, 2048),   # empty, sub-tile, ragged multi-tile groups
    ([5, 130, 0, 77], 128, 256),                    # short K, one 128-output tile column
    ([200, 128, 129, 0, 384, 255, 1], 256, 2048),   # 256- and 128-row tiles
])
def test_fused_swiglu_equals_gemm_then_swiglu_and_the_oracle(sizes, n_half, k):
    """fp8q_grouped_gemm_swiglu_quant_ue8m0 = fp8q_grouped_gemm_w8a8_ue8m0 (bf16 output) then
    fp8q_swiglu_quant_g128_ue8m0, bit for bit; the latter against the oracle on that output."""
    from tests._helpers import swiglu_near_decisions
    aq, a_s, bq, b_s, off, m = _fused_operands(sizes, n_half, k, seed=len(sizes) * 5 + k)
    y = torch.empty((m, 2 * n_half), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8_ue8m0(aq, a_s, bq, b_s, off, y)
    q1 = torch.full((m, n_half), 0x5A, dtype=torch.uint8, device=DEV)
    s1 = torch.full((n_half // 128, m + 3), -1.0, device=DEV)
    fq.fp8q_swiglu_quant_g128_ue8m0(y, q1, s1)
    q2 = torch.full((m, n_half), 0xA5, dtype=torch.uint8, device=DEV)
    s2 = torch.full((n_half // 128, m + 3), -2.0, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant_ue8m0(aq, a_s, bq, b_s, off, q2, s2)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2), f"codes differ at {int((q1 != q2).sum())} places"
    assert torch.equal(s1[:, :m].view(torch.int32), s2[:, :m].view(torch.int32)), "scales differ"
    assert torch.all(s2[:, m:] == -2.0), "scale columns past total_m are not written"
    q_ref, s_ref, amax = oracle.swiglu_quant_g128(bf16_bits(y), with_amax=True, ue8m0=True)
    assert not np.any(_near_pow2_boundary(amax))
    assert swiglu_near_decisions(bf16_bits(y), s_ref)[1] == 0
    assert np.array_equal(q2.cpu().numpy(), q_ref)
    assert np.array_equal(s2[:, :m].cpu().numpy().view(np.uint32), s_ref.view(np.uint32))


def test_fused_swiglu_at_the_moe_layer_shape_with_token_rows():
    """128 experts, 4096 tokens routed top-8: the fused call reading the token rows through
    fp8q_moe_route's row_token equals the dispatched-row composition, every byte."""
    _, off_np, _ = synth.moe_routing(0)
    sizes = list(np.diff(off_np))
    aq, a_s, bq, b_s, off, m = _fused_operands(sizes, 768, 2048, seed=13)
    y = torch.empty((m, 1536), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8_ue8m0(aq, a_s, bq, b_s, off, y)
    q1 = torch.empty((m, 768), dtype=torch.uint8, device=DEV)
    s1 = torch.empty((6, m), device=DEV)
    fq.fp8q_swiglu_quant_g128_ue8m0(y, q1, s1)
    # the same rows held once each as "token rows", read through an identity row_token
    q2 = torch.empty_like(q1)
    s2 = torch.empty_like(s1)
    tok = torch.arange(m, dtype=torch.int32, device=DEV)
    fq.fp8q_grouped_gemm_swiglu_quant_ue8m0(aq, a_s, bq, b_s, off, q2, s2, row_token=tok)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2), f"codes differ at {int((q1 != q2).sum())} places"
    assert torch.equal(s1.view(torch.int32), s2.view(torch.int32)), "scales differ"
