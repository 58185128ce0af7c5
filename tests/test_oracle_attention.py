"""Oracle of FP8 paged decode attention, pinned without the oracle itself.

FP8-RL summary page, "Method step details" step 3 (the Q/K/V scales are recalibrated
before every RL step's rollout) and "Experimental results" (full FP8: linear layers, KV
cache and attention); 1T-parameter-RL page, section 3.4 (paged cache in fixed blocks).
Reading: the query is quantized to E4M3 with its own scale, scores are FP8 x FP8 products
times sm_scale * q_scale * k_scale, softmax and the V sum are exact arithmetic on the
decoded codes.

Pins: one token (softmax of one score is 1), identical keys (uniform weights: the mean of
V), one dominant key (the softmax saturates onto its V row), invariance under a permutation
of the pages, the grouped-query head mapping, masking of cache bytes past the sequence
length, query saturation under a stored scale, and the recalibrated query scale.  The
softmax temperature sm_scale * q_scale * k_scale is pinned by closed forms: with two keys
the weights are the logistic function of the score difference, and hand-picked codes make
every dot product a small integer multiple of a power of two, written out by hand below.
"""
import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_weight_amd import synth

PS = 16  # tokens per page


def _dec(codes):
    return torch.from_numpy(np.ascontiguousarray(codes)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _cache(seed, pages, hkv):
    g = np.random.default_rng(seed)
    c = g.integers(0, 0x7F, size=(pages, PS, hkv, 128), dtype=np.uint8)
    return c | (g.integers(0, 2, size=c.shape, dtype=np.uint8) << 7)


def _q(seqs, hq, tensor=0):
    return synth.activation(5, 0, tensor, seqs, hq * 128).reshape(seqs, hq, 128)


def test_one_token_returns_its_value_row():
    q = _q(3, 4)
    kc, vc = _cache(1, 3, 2), _cache(2, 3, 2)
    bt = np.array([[2], [0], [1]], np.int32)
    out = oracle.paged_decode_attention(q, kc, vc, bt, np.ones(3, np.int32), 0.01, 0.5, 0.125, 0.0884)
    for b, page in enumerate((2, 0, 1)):
        for h in range(4):
            assert np.array_equal(out[b, h], 0.125 * _dec(vc[page, 0, h // 2]))


def test_identical_keys_average_the_values():
    L = 37
    q = _q(1, 2)
    kc = np.broadcast_to(_cache(3, 1, 1)[:1, :1], (3, PS, 1, 128)).copy()
    vc = _cache(4, 3, 1)
    bt = np.array([[2, 0, 1]], np.int32)
    out = oracle.paged_decode_attention(q, kc, vc, bt, np.array([L], np.int32), 0.02, 0.3, 0.25, 0.0884)
    rows = np.concatenate([vc[2], vc[0], vc[1]])[:L, 0]
    ref = 0.25 * _dec(rows).mean(axis=0)
    for h in range(2):
        assert np.allclose(out[0, h], ref, rtol=1e-14, atol=1e-300)


def test_dominant_key_takes_all_the_weight():
    L, hot = 50, 33
    q = synth.to_bf16_bits(np.ones((1, 1, 128), np.float32))  # codes 0x7E with q_scale 1/448
    kc = np.zeros((4, PS, 1, 128), np.uint8)
    bt = np.array([[3, 1, 0, 2]], np.int32)
    page, slot = bt[0, hot // PS], hot % PS
    kc[page, slot, 0] = 0x7E               # q.k = 128 * 448 * 448 for the hot token, 0 elsewhere
    vc = _cache(5, 4, 1)
    # hot score 128 * 448 * 448 / 448 = 57344 against 0: exp(-57344) is 0 in fp64
    out = oracle.paged_decode_attention(q, kc, vc, bt, np.array([L], np.int32), 1.0 / 448, 1.0, 0.5, 1.0)
    assert np.array_equal(out[0, 0], 0.5 * _dec(vc[page, slot, 0]))


def test_page_permutation_invariance_and_masking():
    seqs, hq, hkv, L = 2, 8, 2, 70
    q = _q(seqs, hq, 1)
    kc, vc = _cache(6, 12, hkv), _cache(7, 12, hkv)
    bt = np.array([[4, 9, 0, 7, 2], [1, 3, 5, 6, 8]], np.int32)
    sl = np.array([L, 3], np.int32)
    args = (0.015, 0.4, 0.3, 0.0884)
    out = oracle.paged_decode_attention(q, kc, vc, bt, sl, *args)
    # move the pages: same tokens at new page ids
    perm = np.random.default_rng(8).permutation(12)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[perm], vc2[perm] = kc, vc
    out2 = oracle.paged_decode_attention(q, kc2, vc2, perm[bt].astype(np.int32), sl, *args)
    assert np.allclose(out2, out, rtol=1e-13, atol=1e-300)
    # bytes past each sequence's length and pages it does not own do not matter
    kc3, vc3 = kc.copy(), vc.copy()
    kc3[bt[0, 4], L % PS:], vc3[bt[0, 4], L % PS:] = 0x7E, 0xFE
    kc3[bt[1, 0], 3:], vc3[bt[1, 1]] = 0x7E, 0x7E
    kc3[10:], vc3[10:] = 0x55, 0x55
    assert np.array_equal(oracle.paged_decode_attention(q, kc3, vc3, bt, sl, *args), out)


def test_grouped_query_heads_read_their_kv_head():
    seqs, hq, hkv, L = 1, 8, 2, 20
    q = _q(seqs, hq, 2)
    kc, vc = _cache(9, 2, hkv), _cache(10, 2, hkv)
    bt = np.array([[1, 0]], np.int32)
    args = (np.array([L], np.int32), 0.015, 0.4, 0.3, 0.0884)
    out = oracle.paged_decode_attention(q, kc, vc, bt, *args)
    kc2, vc2 = kc.copy(), vc.copy()
    kc2[:, :, 1], vc2[:, :, 1] = _cache(11, 2, 1)[:, :, 0], _cache(12, 2, 1)[:, :, 0]
    out2 = oracle.paged_decode_attention(q, kc2, vc2, bt, *args)
    assert np.array_equal(out2[:, :4], out[:, :4])          # heads 0-3 read KV head 0
    assert not np.array_equal(out2[:, 4:], out[:, 4:])      # heads 4-7 read KV head 1


def test_query_saturates_under_a_stored_scale():
    """Codes of q / q_scale saturate at +-448: a query clipped to +-448 * q_scale gives the
    same attention."""
    L = 24
    qs = 2.0 ** -8
    q = _q(1, 2, 3)
    qf = synth.bf16_bits_to_f32(q)
    clipped = synth.to_bf16_bits(np.clip(qf, -448 * qs, 448 * qs))
    assert np.any(np.abs(qf) > 448 * qs)
    kc, vc = _cache(13, 2, 1), _cache(14, 2, 1)
    bt = np.array([[0, 1]], np.int32)
    a = oracle.paged_decode_attention(q, kc, vc, bt, np.array([L], np.int32), qs, 0.4, 0.3, 0.0884)
    b = oracle.paged_decode_attention(clipped, kc, vc, bt, np.array([L], np.int32), qs, 0.4, 0.3, 0.0884)
    assert np.array_equal(a, b)


def test_recalibrated_query_scale():
    q = np.zeros((2, 4, 128), np.uint16)
    q[1, 2, 5] = synth.to_bf16_bits(np.array([-2.75], np.float32))[0]
    q[0, 0, 0] = synth.to_bf16_bits(np.array([1.5], np.float32))[0]
    assert oracle.q_scale(q) == np.float32(2.75) / np.float32(448)
    assert oracle.q_scale(np.zeros((1, 1, 128), np.uint16)) == 1.0


# Hand-chosen codes for the closed-form pins: E4M3FN 0x7E = 448, 0x76 = 224, 0x38 = 1,
# 0x30 = 0.5, 0x40 = 2, 0xB8 = -1, 0xF6 = -224 (format definition: bias 7, 3 mantissa bits).
# the scales are binary32 at the boundary (sm_scale is fp64), so take binary32 values
SM, QS, KS, VS = 0.08838834764831845, 0.5, float(np.float32(0.05)), 0.375


def _two_key_cache():
    """One KV head, one 16-token page; token 0 keys (1, 0.5), token 1 keys (0.5, -1) in
    dims 0 and 1, zeros elsewhere; value rows seeded."""
    kc = np.zeros((1, PS, 1, 128), np.uint8)
    kc[0, 0, 0, :2] = (0x38, 0x30)
    kc[0, 1, 0, :2] = (0x30, 0xB8)
    return kc, _cache(21, 1, 1)


def test_two_keys_give_logistic_weights():
    """Query head 0 = (224, 0, ...) and head 1 = (0, -112, ...) with q_scale 0.5 encode to
    codes 448 and -224 exactly.  Dots: head 0 -> (448, 224), head 1 -> (-112, 224).  With
    f = sm_scale * q_scale * k_scale the weight of key 0 is 1 / (1 + exp(-f * (d0 - d1)))."""
    q = np.zeros((1, 2, 128), np.float32)
    q[0, 0, 0], q[0, 1, 1] = 224.0, -112.0
    q = synth.to_bf16_bits(q)
    kc, vc = _two_key_cache()
    out = oracle.paged_decode_attention(q, kc, vc, np.array([[0]], np.int32), np.array([2], np.int32),
                                        QS, KS, VS, SM)
    f = SM * QS * KS
    v0, v1 = _dec(vc[0, 0, 0]), _dec(vc[0, 1, 0])
    for h, diff in ((0, 448.0 - 224.0), (1, -112.0 - 224.0)):
        p0 = 1.0 / (1.0 + np.exp(-f * diff))
        ref = VS * (p0 * v0 + (1.0 - p0) * v1)
        assert np.allclose(out[0, h], ref, rtol=1e-13, atol=1e-15), h
    # the weights are far from 0, 1 and 1/2, so each scale factor moves them
    assert 0.55 < 1.0 / (1.0 + np.exp(-f * 224.0)) < 0.65


def test_three_keys_over_two_pages_closed_form():
    """Three tokens over pages of 2 (the second page holds one live token), two query heads
    sharing one KV head, hand dot products; softmax written out with exp."""
    ps = 2
    q = np.zeros((1, 2, 128), np.float32)
    q[0, 0, :3] = (224.0, 112.0, -0.5)     # / 0.5 -> codes 448, 224, -1
    q[0, 1, :3] = (-112.0, 0.5, 1.0)       # / 0.5 -> codes -224, 1, 2
    q = synth.to_bf16_bits(q)
    kc = np.zeros((3, ps, 1, 128), np.uint8)
    keys = {0: (0x38, 0x30, 0x40), 1: (0xB8, 0x38, 0x00), 2: (0x30, 0xB8, 0x38)}  # token -> dims 0..2
    bt = np.array([[2, 0]], np.int32)      # tokens 0, 1 in page 2; token 2 in page 0
    for t, codes in keys.items():
        kc[bt[0, t // ps], t % ps, 0, :3] = codes
    vc = np.zeros((3, ps, 1, 128), np.uint8)
    vals = _cache(22, 3, 1)
    for t in range(3):
        vc[bt[0, t // ps], t % ps] = vals[t, 0]
    out = oracle.paged_decode_attention(q, kc, vc, bt, np.array([3], np.int32), QS, KS, VS, SM)
    # dots by hand: key values (1, .5, 2), (-1, 1, 0), (.5, -1, 1)
    dots = {0: (448 * 1 + 224 * 0.5 + -1 * 2, 448 * -1 + 224 * 1 + 0, 448 * 0.5 + 224 * -1 + -1 * 1),
            1: (-224 * 1 + 1 * 0.5 + 2 * 2, -224 * -1 + 1 * 1 + 0, -224 * 0.5 + 1 * -1 + 2 * 1)}
    assert dots[0] == (558.0, -224.0, -1.0) and dots[1] == (-219.5, 225.0, -111.0)
    f = SM * QS * KS
    for h in (0, 1):
        e = np.exp(f * np.array(dots[h]))
        p = e / e.sum()
        ref = VS * sum(p[t] * _dec(vals[t, 0, 0]) for t in range(3))
        assert np.allclose(out[0, h], ref, rtol=1e-13, atol=1e-15), h
