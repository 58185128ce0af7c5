"""GPU parity of the MoE layer's data movement (dispatch, SwiGLU + quantization, combine)
against the oracle.

MoE routing-replay page, "Rollout Routing Replay" (section 4): tokens go to their
recorded experts.  Rounding-location page, SwiGLU fusion region: one rounding after
silu(gate) * up.  Dispatch is byte and index work: bit-exact.  SwiGLU-quantization takes
its code decisions in fp64 on both sides: codes and scales bit-exact (a decision is
excused only where the oracle's fp64 value lies within 2^-48 relative of a rounding
boundary, which the test measures and which does not occur on these inputs).  Combine:
every output within half a bf16 ulp of the fp64 sum plus 16 fp32 ulps of the sum of
|terms| (an fp32 sum of at most 10 terms).
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import swiglu_near_decisions, bf16_bits, bf16_to_f64, f32, to_dev_bf16, u8, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _codes(seed, shape):
    g = np.random.default_rng(seed)
    return (g.integers(0, 0x7F, size=shape, dtype=np.uint8) | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7))


def _gpu_dispatch(xq, xs, ids, E, ld_xq=None, ld_as=None):
    T, k = xq.shape
    topk = ids.shape[1]
    n = T * topk
    ld_xq = k if ld_xq is None else ld_xq
    ld_as = max(n, 1) if ld_as is None else ld_as
    xq_d = torch.zeros((T, ld_xq), dtype=torch.uint8, device=DEV)
    xq_d[:, :k] = torch.from_numpy(xq).to(DEV)
    aq = torch.full((max(n, 1), k), 0xAB, dtype=torch.uint8, device=DEV)
    a_s = torch.full((k // 128, ld_as), -3.0, dtype=torch.float32, device=DEV)
    off = torch.full((E + 1,), -7, dtype=torch.int32, device=DEV)
    row_of = torch.full((T, topk), -9, dtype=torch.int32, device=DEV)
    fq.fp8q_moe_dispatch(xq_d[:, :k], torch.from_numpy(xs).to(DEV), torch.from_numpy(ids).to(DEV), E, aq, a_s, off,
                         row_of)
    torch.cuda.synchronize()
    return u8(aq), f32(a_s), off.cpu().numpy(), row_of.cpu().numpy()


def _check_dispatch(xq, xs, ids, E, **kw):
    aq, a_s, off, row_of = _gpu_dispatch(xq, xs, ids, E, **kw)
    r_aq, r_as, r_off, r_row = oracle.moe_dispatch(xq, xs, ids, E)
    R = int(r_off[-1])
    assert np.array_equal(off, r_off), "offsets differ"
    assert np.array_equal(row_of, r_row), "row_of differs"
    assert np.array_equal(aq[:R], r_aq), "dispatched rows differ"
    assert np.array_equal(a_s[:, :R].view(np.uint32), r_as.view(np.uint32)), "dispatched scales differ"
    assert np.all(aq[R:] == 0xAB) and np.all(a_s[:, R:] == -3.0), "rows past the valid ones were written"


def test_dispatch_hand_case():
    ids = np.array([[2, 0], [0, 2], [3, 3]], np.int16)
    xq = _codes(1, (3, 128))
    xs = np.array([[1.0, 2.0, 3.0]], np.float32)
    _check_dispatch(xq, xs, ids, 4)


def test_dispatch_invalid_ids_and_ragged_tail():
    T, topk, E, k = 37, 3, 5, 256
    ids = synth.moe_topk(2, tokens=T, experts=E, topk=topk)[0]
    ids[3, 1] = -1
    ids[10, 0] = E
    ids[36, 2] = -32768
    xs = np.random.default_rng(3).random((k // 128, T + 5), dtype=np.float32)
    _check_dispatch(_codes(2, (T, k)), xs, ids, E, ld_xq=k + 32, ld_as=T * topk + 11)


def test_dispatch_moe_layer_shape():
    """4096 tokens, top-8 of 128 experts (Zipf-skewed), hidden 2048: 32768 rows."""
    T, E, k = 4096, 128, 2048
    ids, _ = synth.moe_topk(0, tokens=T, experts=E, topk=8)
    xs = np.random.default_rng(4).random((k // 128, T), dtype=np.float32)
    _check_dispatch(_codes(4, (T, k)), xs, ids, E)


def test_dispatch_several_chunks_one_expert_and_empty():
    ids = synth.moe_topk(3, tokens=5000, experts=16, topk=8)[0]  # 40000 entries: two scan chunks
    xs = np.random.default_rng(5).random((1, 5000), dtype=np.float32)
    _check_dispatch(_codes(5, (5000, 128)), xs, ids, 16)
    _check_dispatch(_codes(6, (9, 128)), np.ones((1, 9), np.float32), np.zeros((9, 1), np.int16), 1)
    aq, a_s, off, row_of = _gpu_dispatch(np.zeros((0, 128), np.uint8), np.zeros((1, 1), np.float32),
                                         np.zeros((0, 8), np.int16), 6)
    assert off.tolist() == [0] * 7


# ---------------------------------------------------------------- SwiGLU + quantization
def _near_boundary(amax):
    """Groups whose fp64 amax/448 lies within 2^-48 relative of an fp32 rounding boundary."""
    v = np.asarray(amax, np.float64) / 448.0
    f = v.astype(np.float32).astype(np.float64)
    up = np.nextafter(v.astype(np.float32), np.float32(np.inf)).astype(np.float64)
    dn = np.nextafter(v.astype(np.float32), np.float32(0)).astype(np.float64)
    mids = np.stack([(f + up) / 2, (f + dn) / 2])
    return (v > 0) & np.any(np.abs(mids - v) <= np.abs(v) * 2.0 ** -48, axis=0)


def _check_swiglu(h, ld_s=None):
    m, n2 = h.shape
    n = n2 // 2
    ld_s = m if ld_s is None else ld_s
    q = torch.empty((m, n), dtype=torch.uint8, device=DEV)
    s = torch.full((n // 128, ld_s), -5.0, dtype=torch.float32, device=DEV)
    fq.fp8q_swiglu_quant_g128(to_dev_bf16(h), q, s)
    torch.cuda.synchronize()
    gq, gs = u8(q), f32(s)
    rq, rs, amax = oracle.swiglu_quant_g128(h, ld_s=ld_s, with_amax=True)
    assert np.all(gs[:, m:] == -5.0)
    assert not np.any(_near_boundary(amax)), "an input sits on an fp32 rounding boundary"
    # the device's and glibc's fp64 exp are different implementations: no decision may sit
    # close enough to a boundary for a few ulps of exp to move it
    assert swiglu_near_decisions(h, rs) == (0, 0)
    assert np.array_equal(gs[:, :m].view(np.uint32), rs[:, :m].view(np.uint32)), "scales differ"
    bad = gq != rq
    assert not np.any(bad), f"{int(bad.sum())} codes differ"


def test_swiglu_moe_fc2_input_shape():
    """fc1 output of the MoE layer: 32768 rows of [gate | up], 768 columns each."""
    g = synth.activation(4, 0, 70, 32768, 768, outlier_channels=0)
    u = synth.activation(4, 0, 71, 32768, 768)
    _check_swiglu(np.concatenate([g, u], axis=1))


def test_swiglu_ragged_and_edges():
    m, n = 13, 384
    g = synth.activation(4, 1, 72, m, n)
    u = synth.activation(4, 1, 73, m, n)
    g[0, :128] = 0                                                            # zero group: scale 1
    g[1, 128:256] = synth.to_bf16_bits(np.full(128, 60.0, np.float32))      # saturated gate: a = g*u
    g[2, :128] = synth.to_bf16_bits(np.full(128, -900.0, np.float32))        # exp overflows: a = -0
    u[3, 256:] = synth.to_bf16_bits(np.full(128, 2.0 ** -120, np.float32))   # tiny group: subnormal scale
    g[4, 256:] = synth.to_bf16_bits(np.linspace(-3e38, 3e38, 128, dtype=np.float32))
    u[4, 256:] = synth.to_bf16_bits(np.full(128, 2.0 ** -100, np.float32))
    _check_swiglu(np.concatenate([g, u], axis=1), ld_s=m + 3)


# ---------------------------------------------------------------- combine
def _check_combine(y, row_of, w, hidden_pad=0):
    T, topk = row_of.shape
    H = y.shape[1]
    out = torch.full((T, H + hidden_pad), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_moe_combine(to_dev_bf16(y), torch.from_numpy(row_of).to(DEV), torch.from_numpy(w).to(DEV),
                        out[:, :H])
    torch.cuda.synchronize()
    got = bf16_to_f64(bf16_bits(out[:, :H]))
    ref = oracle.moe_combine(y, row_of, w)
    yf = bf16_to_f64(y)
    mag = np.zeros_like(ref)
    for j in range(topk):
        live = row_of[:, j] >= 0
        mag[live] += np.abs(w[live, j].astype(np.float64)[:, None] * yf[row_of[live, j]])
    bound = 0.5 * ulp_bf16(ref) + 16 * 2.0 ** -24 * mag
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"worst err/bound {float(np.max(err / np.maximum(bound, 1e-300))):.3f}"
    if hidden_pad:
        assert torch.isnan(out[:, H:].float()).all()


def test_combine_moe_layer_shape():
    T, E = 4096, 128
    ids, w = synth.moe_topk(0, tokens=T, experts=E, topk=8)
    _, _, _, row_of = oracle.moe_dispatch(np.zeros((T, 128), np.uint8), np.ones((1, T), np.float32), ids, E)
    y = synth.activation(4, 0, 80, T * 8, 2048, outlier_channels=0)
    _check_combine(y, row_of.astype(np.int32), w)


def test_combine_dropped_entries_wide_topk_ragged_hidden():
    T, topk, R, H = 50, 10, 300, 264
    g = np.random.default_rng(7)
    row_of = g.integers(0, R, size=(T, topk)).astype(np.int32)
    row_of[g.random((T, topk)) < 0.2] = -1
    row_of[5] = -1  # a token with no expert: zeros
    w = g.random((T, topk)).astype(np.float32)
    _check_combine(synth.activation(4, 2, 81, R, H), row_of, w, hidden_pad=8)


# ---------------------------------------------------------------- the layer, end to end
def test_moe_layer_composition():
    """dispatch -> fc1 grouped GEMM -> SwiGLU + quantization -> fc2 grouped GEMM -> combine on the
    GPU, against the oracle's chain (its fc1 output rounded to bf16 the same way).  Codes may differ
    where the two bf16 fc1 outputs do, so this is a normwise check; each stage's parity is above."""
    T, E, topk, H, I = 256, 8, 2, 256, 256
    ids, w = synth.moe_topk(5, tokens=T, experts=E, topk=topk)
    x = synth.activation(4, 5, 90, T, H)
    xq, xs = oracle.quant_act_g128(x)
    w1q = np.empty((E, 2 * I, H), np.uint8)
    w1s = np.empty((E, 2 * I // 128, H // 128), np.float32)
    w2q = np.empty((E, H, I), np.uint8)
    w2s = np.empty((E, H // 128, I // 128), np.float32)
    for e in range(E):
        w1q[e], w1s[e] = oracle.quant_weight_blk128(synth.weight(4, 5, e, 2 * I, H, std=0.06))
        w2q[e], w2s[e] = oracle.quant_weight_blk128(synth.weight(4, 5, 100 + e, H, I, std=0.06))
    # oracle chain
    aq, a_s, off, row_of = oracle.moe_dispatch(xq, xs, ids, E)
    h_ref = synth.to_bf16_bits(oracle.grouped_gemm_w8a8(aq, a_s, w1q, w1s, off).astype(np.float32))
    q2, s2 = oracle.swiglu_quant_g128(h_ref)
    y2 = synth.to_bf16_bits(oracle.grouped_gemm_w8a8(q2, s2, w2q, w2s, off).astype(np.float32))
    ref = oracle.moe_combine(y2, row_of, w)
    # GPU chain
    n = T * topk
    d = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(DEV)
    aq_d = torch.empty((n, H), dtype=torch.uint8, device=DEV)
    as_d = torch.empty((H // 128, n), dtype=torch.float32, device=DEV)
    off_d = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    row_d = torch.empty((T, topk), dtype=torch.int32, device=DEV)
    fq.fp8q_moe_dispatch(d(xq), d(xs), d(ids), E, aq_d, as_d, off_d, row_d)
    h_d = torch.empty((n, 2 * I), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8(aq_d, as_d, d(w1q), d(w1s), off_d, h_d)
    q2_d = torch.empty((n, I), dtype=torch.uint8, device=DEV)
    s2_d = torch.empty((I // 128, n), dtype=torch.float32, device=DEV)
    fq.fp8q_swiglu_quant_g128(h_d, q2_d, s2_d)
    y2_d = torch.empty((n, H), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_grouped_gemm_w8a8(q2_d, s2_d, d(w2q), d(w2s), off_d, y2_d)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_moe_combine(y2_d, row_d, d(w), out)
    torch.cuda.synchronize()
    got = bf16_to_f64(bf16_bits(out))
    assert np.array_equal(off_d.cpu().numpy(), off)
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < 2e-2, rel
