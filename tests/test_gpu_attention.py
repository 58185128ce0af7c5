"""GPU parity of FP8 paged decode attention against the oracle.

FP8-RL summary page, "Method step details" step 3 and "Experimental results" (full FP8:
linear layers, KV cache and attention).  The recalibrated query scale is bit-exact.
Outputs: every element within half a bf16 ulp of the fp64 oracle plus 2e-3 of the largest
|output| of its (sequence, head) row, the form of the GEMM gate.  The query-key products of
E4M3 values are exact on the bf16 matrix core with fp32 accumulation; softmax and the value
sum are fp32.
"""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import bf16_bits, bf16_to_f64, to_dev_bf16, ulp_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _codes(seed, shape):
    g = np.random.default_rng(seed)
    c = g.integers(0, 0x7F, size=shape, dtype=np.uint8)
    return c | (g.integers(0, 2, size=shape, dtype=np.uint8) << 7)


def _gate(got_bits, ref):
    got = bf16_to_f64(got_bits)
    rowmax = np.max(np.abs(ref), axis=-1, keepdims=True)
    bound = 0.5 * ulp_bf16(ref) + 2e-3 * rowmax
    err = np.abs(got - ref)
    return bool(np.all(err <= bound)), float(np.max(err / np.maximum(bound, 1e-300)))


def _run(q_bits, kc, vc, bt, lens, q_scale, k_scale, v_scale, sm, recal):
    seqs, hq, _ = q_bits.shape
    out = torch.full((seqs, hq, 128), float("nan"), dtype=torch.bfloat16, device=DEV)
    qs = torch.tensor([q_scale], dtype=torch.float32, device=DEV)
    fq.fp8q_paged_decode_attention(to_dev_bf16(q_bits.reshape(seqs, -1)).view(seqs, hq, 128),
                                   torch.from_numpy(kc).to(DEV), torch.from_numpy(vc).to(DEV),
                                   torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV), qs,
                                   torch.tensor([k_scale], device=DEV), torch.tensor([v_scale], device=DEV), sm, out,
                                   recalibrate_q=recal)
    torch.cuda.synchronize()
    return bf16_bits(out), float(qs.item())


@pytest.mark.parametrize("hq,hkv,ps", [(8, 2, 16), (32, 4, 16), (16, 1, 16), (2, 2, 16), (12, 2, 5), (4, 4, 1)])
def test_small_contexts(hq, hkv, ps):
    seqs = 4
    lens = np.array([70, 1, 0, 131], np.int32)
    per = -(-int(lens.max()) // ps)
    pages = seqs * per + 3
    g = np.random.default_rng(hq * 7 + ps)
    bt = g.permutation(pages)[:seqs * per].reshape(seqs, per).astype(np.int32)
    kc, vc = _codes(hq + ps, (pages, ps, hkv, 128)), _codes(hq + ps + 1, (pages, ps, hkv, 128))
    q = synth.activation(5, 1, hq + ps, seqs, hq * 128).reshape(seqs, hq, 128)
    ks, vs, sm = 0.02, 0.015, 128 ** -0.5
    for recal in (False, True):
        qs = 0.01 if not recal else float(oracle.q_scale(q))
        got, qs_dev = _run(q, kc, vc, bt, lens, 0.01, ks, vs, sm, recal)
        if recal:
            assert np.float32(qs_dev) == np.float32(qs)
        ref = oracle.paged_decode_attention(q, kc, vc, bt, lens, qs, ks, vs, sm)
        assert np.all(got[2] == 0), "a sequence of length 0 gives zeros"
        ok, ratio = _gate(got, ref)
        assert ok, f"recal={recal}: worst err/bound {ratio:.3f}"


def _random_attention_cases(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(count):
        hkv = int(g.choice([1, 2, 4, 8]))
        hq = hkv * int(g.choice([1, 2, 3, 4, 8, 16]))
        cases.append((int(g.integers(1, 13)), hq, hkv, int(g.choice([1, 5, 16])), 300 + c))
    return cases


@pytest.mark.parametrize("seqs,hq,hkv,ps,seed", _random_attention_cases(8, 17))
def test_random_contexts(seqs, hq, hkv, ps, seed):
    """Seeded random sequence counts and lengths (empty ones included), query / KV head
    counts, page sizes and scales, with and without query recalibration."""
    g = np.random.Generator(np.random.PCG64(seed))
    lens = g.integers(0, 900, size=seqs).astype(np.int32)
    per = max(1, -(-int(lens.max()) // ps))
    pages = seqs * per + int(g.integers(0, 5))
    bt = g.permutation(pages)[:seqs * per].reshape(seqs, per).astype(np.int32)
    kc, vc = _codes(seed, (pages, ps, hkv, 128)), _codes(seed + 1, (pages, ps, hkv, 128))
    q = synth.activation(5, 2, seed, seqs, hq * 128).reshape(seqs, hq, 128)
    ks, vs = float(g.choice([0.005, 0.02, 0.08])), float(g.choice([0.01, 0.03]))
    sm = 128 ** -0.5
    recal = bool(g.integers(0, 2))
    qs = float(oracle.q_scale(q)) if recal else 0.01
    got, qs_dev = _run(q, kc, vc, bt, lens, 0.01, ks, vs, sm, recal)
    if recal:
        assert np.float32(qs_dev) == np.float32(qs)
    ref = oracle.paged_decode_attention(q, kc, vc, bt, lens, qs, ks, vs, sm)
    ok, ratio = _gate(got, ref)
    assert ok, f"worst err/bound {ratio:.3f}"


@pytest.mark.parametrize("ps", [16, 5])
def test_many_sequences_pair_kv_heads(ps):
    """64 sequences x 8 KV heads with groups of 4 query heads: the kernel reads two KV heads
    per workgroup (32-token chunks).  Lengths span empty, single-token, sub-chunk,
    chunk-boundary and multi-chunk contexts."""
    seqs, hq, hkv = 64, 32, 8
    g = np.random.default_rng(40 + ps)
    lens = g.integers(0, 200, size=seqs).astype(np.int32)
    lens[:8] = [0, 1, 31, 32, 33, 64, 65, 199]
    per = -(-int(lens.max()) // ps)
    pages = seqs * per + 5
    bt = g.permutation(pages)[:seqs * per].reshape(seqs, per).astype(np.int32)
    kc, vc = _codes(50 + ps, (pages, ps, hkv, 128)), _codes(51 + ps, (pages, ps, hkv, 128))
    q = synth.activation(5, 1, 60 + ps, seqs, hq * 128).reshape(seqs, hq, 128)
    ks, vs, sm = 0.02, 0.015, 128 ** -0.5
    qs = float(oracle.q_scale(q))
    got, qs_dev = _run(q, kc, vc, bt, lens, 0.01, ks, vs, sm, True)
    assert np.float32(qs_dev) == np.float32(qs)
    ref = oracle.paged_decode_attention(q, kc, vc, bt, lens, qs, ks, vs, sm)
    assert np.all(got[0] == 0), "a sequence of length 0 gives zeros"
    ok, ratio = _gate(got, ref)
    assert ok, f"worst err/bound {ratio:.3f}"


def test_saturating_stored_query_scale_and_peaked_scores():
    """A stored q_scale smaller than the queries need (codes saturate) and large scores."""
    seqs, hq, hkv, ps, L = 2, 4, 1, 16, 300
    per = -(-L // ps)
    bt = np.arange(seqs * per, dtype=np.int32).reshape(seqs, per)
    kc, vc = _codes(21, (seqs * per, ps, hkv, 128)), _codes(22, (seqs * per, ps, hkv, 128))
    q = synth.activation(5, 2, 3, seqs, hq * 128).reshape(seqs, hq, 128)
    lens = np.array([L, L - 17], np.int32)
    got, _ = _run(q, kc, vc, bt, lens, 2.0 ** -7, 0.05, 0.02, 0.25, False)
    ref = oracle.paged_decode_attention(q, kc, vc, bt, lens, 2.0 ** -7, 0.05, 0.02, 0.25)
    ok, ratio = _gate(got, ref)
    assert ok, f"worst err/bound {ratio:.3f}"


def test_kv_layer_shape_sampled_sequences():
    """64 sequences x 20,000 tokens, 8 KV heads, 32 query heads, 16-token pages (the KV
    workload) with a seeded page table.  Four sampled sequences hold K/V ~N(0, 1) with
    per-head outlier dims written by the oracle's quantizer (recalibrated scales); the rest
    of the cache is random codes.  The sampled outputs are checked against the oracle on a
    host copy of their pages."""
    slots, pages = synth.kv_slot_mapping()
    seqs, L, hkv, hq, ps = 64, 20000, 8, 32, 16
    per = L // ps
    bt = (slots.reshape(seqs, L)[:, ::ps] // ps).astype(np.int32)
    kc = synth.device_fp8_codes((pages, ps, hkv, 128), DEV, 5, 0, 30)
    vc = synth.device_fp8_codes((pages, ps, hkv, 128), DEV, 5, 0, 31)
    sample = (0, 5, 37, 63)
    lens = np.full(seqs, L, np.int32)
    lens[5] = 12345
    n = len(sample) * L
    local = np.arange(n, dtype=np.int64)  # token i of sample j -> local page j*per + i // ps
    kh, vh, ks, vs = oracle.kv_quant(synth.kv_values(5, 0, 40, n), synth.kv_values(5, 0, 41, n), local,
                                     np.zeros((len(sample) * per, ps, hkv, 128), np.uint8),
                                     np.zeros((len(sample) * per, ps, hkv, 128), np.uint8), ps, recalibrate=True)
    for j, b in enumerate(sample):
        idx = torch.from_numpy(bt[b].astype(np.int64)).to(DEV)
        kc[idx] = torch.from_numpy(kh[j * per:(j + 1) * per]).to(DEV)
        vc[idx] = torch.from_numpy(vh[j * per:(j + 1) * per]).to(DEV)
    q = synth.activation(5, 0, 32, seqs, hq * 128).reshape(seqs, hq, 128)
    out = torch.empty((seqs, hq, 128), dtype=torch.bfloat16, device=DEV)
    qs = torch.zeros(1, device=DEV)
    sm = 128 ** -0.5
    fq.fp8q_paged_decode_attention(to_dev_bf16(q.reshape(seqs, -1)).view(seqs, hq, 128), kc, vc,
                                   torch.from_numpy(bt).to(DEV), torch.from_numpy(lens).to(DEV), qs,
                                   torch.tensor([ks], device=DEV), torch.tensor([vs], device=DEV), sm, out,
                                   recalibrate_q=True)
    torch.cuda.synchronize()
    q_scale = float(oracle.q_scale(q))
    assert float(qs.item()) == q_scale
    got = bf16_bits(out)
    for j, b in enumerate(sample):
        ref = oracle.paged_decode_attention(q[b:b + 1], kh[j * per:(j + 1) * per], vh[j * per:(j + 1) * per],
                                            np.arange(per, dtype=np.int32)[None, :], lens[b:b + 1], q_scale, ks,
                                            vs, sm)
        ok, ratio = _gate(got[b:b + 1], ref)
        assert ok, f"sequence {b}: worst err/bound {ratio:.3f}"
