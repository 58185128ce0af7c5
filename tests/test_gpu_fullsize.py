"""Parity at the workloads' full sizes, in the launch configurations the benchmark times.

Sources: FP8-RL summary page, "Prerequisites / FP8 quantization format" (128x128 weight
blocks, E4M3) and "Method step details" steps 1-3 (weights quantized at every sync,
activations per forward, K/V scales recalibrated per step); "1T-parameter RL on 100
GPUs", section 3.4 (paged KV cache, K and V quantized separately).

Inputs are drawn on the GPU by the seeded generators and the oracle is given host copies
of the same bytes; GEMM operands are quantized by the oracle.  Where the oracle would
take minutes on the whole output, outputs are sampled (blocks, rows, tokens) and each
sample is checked against the oracle, and properties that hold at any size are checked
on every output: scales equal the oracle's scale of the exact block / tensor amax, no
code is NaN, and every nonzero block reaches the code for 448 (0x7E)."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import bf16_bits, u8, f32, gemm_gate

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _block_properties(w, q, s):
    """Every block of one quantized weight [n, k]: its scale is the oracle's scale of the
    block amax (max is order-free, so the device reduction is exact), no code is NaN, and
    the largest code magnitude of every nonzero block is 0x7E."""
    n, k = w.shape
    nb, kb = n // 128, k // 128
    amax = w.view(nb, 128, kb, 128).abs().amax(dim=(1, 3)).float().cpu().numpy()
    want = np.array([oracle.scale(a) for a in amax.ravel()], np.float32).reshape(nb, kb)
    got = f32(s)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32)), "block scales differ from the oracle's"
    mag = torch.bitwise_and(q, 0x7F).view(nb, 128, kb, 128)
    assert not bool((mag == 0x7F).any()), "a NaN code was written"
    top = mag.amax(dim=(1, 3)).cpu().numpy()
    assert np.all(top[amax > 0] == 0x7E)


def _check_blocks(w, q, s, picks):
    """Blocks (bi, bj) of one weight against the oracle, codes and scales bit for bit."""
    wb = torch.stack([w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] for bi, bj in picks])
    qb = torch.stack([q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] for bi, bj in picks])
    sb = torch.stack([s[bi, bj] for bi, bj in picks])
    qr, sr = oracle.quant_weight_blk128(bf16_bits(wb).reshape(-1, 128))   # one block per 128 rows
    assert np.array_equal(f32(sb).view(np.uint32), sr[:, 0].view(np.uint32))
    assert np.array_equal(u8(qb).reshape(-1, 128), qr)


DENSE_LINEARS = [(4096, 4096), (1024, 4096), (1024, 4096), (4096, 4096),  # q k v o
                 (12288, 4096), (12288, 4096), (4096, 12288)]            # gate up down


def test_weight_sync_36_layers_one_call():
    """All 252 linears of 36 dense layers (6.95 G parameters) quantized by one batched
    call, as at a weight sync.  Every scale and the code properties are checked on every
    block; three blocks of every tensor (the first and last tensors: also their corner
    blocks) are checked code for code against the oracle."""
    ws, qs, ss = [], [], []
    for layer in range(36):
        for t, (n, k) in enumerate(DENSE_LINEARS):
            ws.append(synth.device_normal_bf16((n, k), 0.02, DEV, 3, layer, t, outlier_p=1e-3, outlier_mult=20.0))
            qs.append(torch.full((n, k), 0x7F, dtype=torch.uint8, device=DEV))
            ss.append(torch.full((n // 128, k // 128), -1.0, dtype=torch.float32, device=DEV))
    assert sum(w.numel() for w in ws) == 6_945_767_424
    _say("sync: generated 252 tensors")
    fq.fp8q_quant_weight_blk128(list(zip(ws, qs, ss)))
    torch.cuda.synchronize()
    _say("sync: quantized")
    g = np.random.Generator(np.random.PCG64(36))
    for i, (w, q, s) in enumerate(zip(ws, qs, ss)):
        nb, kb = s.shape
        picks = [(int(g.integers(nb)), int(g.integers(kb))) for _ in range(3)]
        if i in (0, len(ws) - 1):
            picks += [(0, 0), (0, kb - 1), (nb - 1, 0), (nb - 1, kb - 1)]
        _check_blocks(w, q, s, picks)
        _block_properties(w, q, s)
    _say("sync: checked")


def _grouped_sample_rows(off, g):
    """Per nonempty group: its first and last row and one row between."""
    rows = []
    for e in range(len(off) - 1):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 > r0:
            rows.append(np.unique([r0, r1 - 1, int(g.integers(r0, r1))]))
    return rows


def _check_grouped_rows(y, aq, as_, bq, bs, off, g):
    worst = 0.0
    for rows in _grouped_sample_rows(off, g):
        e = int(np.searchsorted(off, rows[0], side="right") - 1)
        ref = oracle.gemm_w8a8(aq[rows], as_[:, rows], bq[e], bs[e])
        ok, ratio, _ = gemm_gate(y[rows], ref)
        worst = max(worst, ratio)
        assert ok, f"expert {e}, rows {rows}: worst err/bound {ratio:.3f}"
    return worst


def test_moe_layer_full_size():
    """One MoE layer (128 experts, hidden 2048, expert intermediate 768, 4096 tokens
    routed top-8 with Zipf skew): fc1 and fc2 expert weights quantized in one batched
    call and compared with the oracle in full; the routed fc1 input and the fc2 input
    quantized and compared in full; grouped fc1 and fc2 on the oracle's operands, three
    rows of every expert against the oracle."""
    E, H, I = 128, 2048, 768
    row_token, off, _ = synth.moe_routing(0)
    mrows = int(off[-1])
    assert mrows == 4096 * 8
    fc1 = synth.device_normal_bf16((E * 2 * I, H), 0.02, DEV, 4, 0, 0)
    fc2 = synth.device_normal_bf16((E * H, I), 0.02, DEV, 4, 0, 1)
    fc1q = torch.empty(fc1.shape, dtype=torch.uint8, device=DEV)
    fc2q = torch.empty(fc2.shape, dtype=torch.uint8, device=DEV)
    fc1s = torch.empty((E * 2 * I // 128, H // 128), dtype=torch.float32, device=DEV)
    fc2s = torch.empty((E * H // 128, I // 128), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_weight_blk128([(fc1, fc1q, fc1s), (fc2, fc2q, fc2s)])
    torch.cuda.synchronize()
    ref1 = oracle.quant_weight_blk128(bf16_bits(fc1))
    ref2 = oracle.quant_weight_blk128(bf16_bits(fc2))
    for (q, s), (qr, sr) in (((fc1q, fc1s), ref1), ((fc2q, fc2s), ref2)):
        assert np.array_equal(f32(s).view(np.uint32), sr.view(np.uint32))
        assert np.array_equal(u8(q), qr)
    _say("moe: expert weights match")

    x = synth.device_activation(4096, H, DEV, 4, 0, 5)
    xs_rows = x[torch.from_numpy(row_token).to(DEV)]
    a1q = torch.empty((mrows, H), dtype=torch.uint8, device=DEV)
    a1s = torch.empty((H // 128, mrows), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128(xs_rows, a1q, a1s)
    a2 = synth.device_activation(mrows, I, DEV, 4, 0, 6, outlier_channels=0)
    a2q = torch.empty((mrows, I), dtype=torch.uint8, device=DEV)
    a2s = torch.empty((I // 128, mrows), dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128(a2, a2q, a2s)
    torch.cuda.synchronize()
    aq1, as1 = oracle.quant_act_g128(bf16_bits(xs_rows))
    aq2, as2 = oracle.quant_act_g128(bf16_bits(a2))
    for (q, s), (qr, sr) in (((a1q, a1s), (aq1, as1)), ((a2q, a2s), (aq2, as2))):
        assert np.array_equal(f32(s).view(np.uint32), sr.view(np.uint32))
        assert np.array_equal(u8(q), qr)
    _say("moe: activations match")

    offs = _dev(off)
    g = np.random.Generator(np.random.PCG64(48))
    b1q, b1s = ref1[0].reshape(E, 2 * I, H), ref1[1].reshape(E, 2 * I // 128, H // 128)
    b2q, b2s = ref2[0].reshape(E, H, I), ref2[1].reshape(E, H // 128, I // 128)
    for aq, as_, bq, bs, n in ((aq1, as1, b1q, b1s, 2 * I), (aq2, as2, b2q, b2s, H)):
        y = torch.full((mrows, n), float("nan"), dtype=torch.bfloat16, device=DEV)
        fq.fp8q_grouped_gemm_w8a8(_dev(aq), _dev(as_), _dev(bq), _dev(bs), offs, y)
        torch.cuda.synchronize()
        yb = bf16_bits(y)
        assert not np.any((yb & 0x7FFF) > 0x7F80), "a row was not written"
        worst = _check_grouped_rows(yb, aq, as_, bq, bs, off, g)
        _say(f"moe: grouped n={n} worst err/bound {worst:.3f}")


def test_kv_layer_full_size():
    """One KV layer: 64 sequences x 20,000 tokens (1.28 M tokens, 8 heads of 128) in
    16-token pages, recalibrate + write, then a 64-token decode write with the stored
    scales (a quarter of its values pushed past the range, so it saturates).  The scales
    are compared with the oracle's amax over all 2.6 G elements; 4,096 sampled tokens
    (with the first, the last and those holding the K and V maxima) code for code; every
    slot for the properties."""
    slots_np, pages = synth.kv_slot_mapping()
    T = len(slots_np)
    assert T == 64 * 20000 and pages * 16 == T   # every slot is written exactly once
    k = synth.device_kv(T, DEV, 5, 0, 0)
    v = synth.device_kv(T, DEV, 5, 0, 1)
    sl = _dev(slots_np)
    kc = torch.full((pages, 16, 8, 128), 0x7F, dtype=torch.uint8, device=DEV)
    vc = torch.full_like(kc, 0x7F)
    ks = torch.full((1,), 5.0, device=DEV)
    vs = torch.full((1,), 5.0, device=DEV)
    fq.fp8q_kv_quant(k, v, sl, kc, vc, ks, vs, 448.0, recalibrate=True)
    torch.cuda.synchronize()
    _say("kv: written")
    kb = bf16_bits(k).reshape(T, 1024)
    vb = bf16_bits(v).reshape(T, 1024)
    rks, rvs = oracle.kv_scales(kb, vb, slots_np)
    got_ks, got_vs = f32(ks)[0], f32(vs)[0]
    assert np.float32(got_ks).view(np.uint32) == np.float32(rks).view(np.uint32)
    assert np.float32(got_vs).view(np.uint32) == np.float32(rvs).view(np.uint32)
    _say(f"kv: scales match ({rks!r}, {rvs!r})")

    g = np.random.Generator(np.random.PCG64(20000))
    kmax = int(np.argmax(np.max(kb & 0x7FFF, axis=1)))
    vmax = int(np.argmax(np.max(vb & 0x7FFF, axis=1)))
    idx = np.unique(np.concatenate([[0, T - 1, kmax, vmax], g.choice(T, 4096, replace=False)]))
    n = len(idx)
    spages = -(-n // 16)
    sentinel = np.full((spages, 16, 8, 128), 0x7F, np.uint8)
    rk, rv, _, _ = oracle.kv_quant(kb[idx].reshape(n, 8, 128), vb[idx].reshape(n, 8, 128),
                                   np.arange(n, dtype=np.int64), sentinel, sentinel, 16,
                                   k_scale=rks, v_scale=rvs, recalibrate=False)
    sel = _dev(slots_np[idx])
    assert np.array_equal(u8(kc.view(-1, 8, 128)[sel]), rk.reshape(-1, 8, 128)[:n])
    assert np.array_equal(u8(vc.view(-1, 8, 128)[sel]), rv.reshape(-1, 8, 128)[:n])
    for c in (kc, vc):
        mag = torch.bitwise_and(c, 0x7F)
        assert not bool((mag == 0x7F).any()), "a slot was not written or a NaN code was stored"
        assert int(mag.max()) == 0x7E
    _say("kv: sampled tokens match")

    # decode: one new token per sequence at its last position, stored scales
    dec = np.arange(64) * 20000 + 19999
    kd = synth.device_kv(64, DEV, 5, 1, 0)
    vd = synth.device_kv(64, DEV, 5, 1, 1)
    kd[::4] *= 64.0
    vd[1::4] *= 64.0
    fq.fp8q_kv_quant(kd, vd, _dev(slots_np[dec]), kc, vc, ks, vs, 448.0, recalibrate=False)
    torch.cuda.synchronize()
    assert f32(ks)[0] == got_ks and f32(vs)[0] == got_vs, "stored scales changed without the flag"
    sentinel = np.full((4, 16, 8, 128), 0x7F, np.uint8)
    rk, rv, _, _ = oracle.kv_quant(bf16_bits(kd), bf16_bits(vd), np.arange(64, dtype=np.int64), sentinel,
                                   sentinel, 16, k_scale=rks, v_scale=rvs, recalibrate=False)
    sel = _dev(slots_np[dec])
    got_k = u8(kc.view(-1, 8, 128)[sel])
    assert np.array_equal(got_k, rk.reshape(-1, 8, 128))
    assert np.array_equal(u8(vc.view(-1, 8, 128)[sel]), rv.reshape(-1, 8, 128))
    assert np.any((got_k & 0x7F) == 0x7E)
    # the token before each decode slot kept its prefill code
    prev = _dev(slots_np[dec - 1])
    pk, _, _, _ = oracle.kv_quant(kb[dec - 1].reshape(64, 8, 128), vb[dec - 1].reshape(64, 8, 128),
                                  np.arange(64, dtype=np.int64), sentinel, sentinel, 16,
                                  k_scale=rks, v_scale=rvs, recalibrate=False)
    assert np.array_equal(u8(kc.view(-1, 8, 128)[prev]), pk.reshape(-1, 8, 128))


def test_gemm_operand_at_the_2gib_limit():
    """A token operand of exactly 2 GiB (524,288 x 4096 codes), the largest the 32-bit
    buffer ranges address: rows sampled at both ends and between, against the oracle.
    Codes and scales are drawn directly by the seeded generator."""
    m, n, k = (1 << 31) // 4096, 256, 4096
    a = synth.device_fp8_codes((m, k), DEV, 7, 0, 0)
    a_s = synth.device_scales((k // 128, m), DEV, 7, 0, 1)
    b = synth.device_fp8_codes((n, k), DEV, 7, 0, 2)
    b_s = synth.device_scales((n // 128, k // 128), DEV, 7, 0, 3)
    y = torch.full((m, n), float("nan"), dtype=torch.bfloat16, device=DEV)
    fq.fp8q_gemm_w8a8_blkscaled(a, a_s, b, b_s, y)
    torch.cuda.synchronize()
    g = np.random.Generator(np.random.PCG64(31))
    rows = np.unique(np.concatenate([np.arange(64), np.arange(m - 64, m), g.choice(m, 128, replace=False)]))
    sel = _dev(rows)
    ref = oracle.gemm_w8a8(u8(a[sel]), f32(a_s[:, sel]), u8(b), f32(b_s))
    ok, ratio, nrm = gemm_gate(bf16_bits(y[sel]), ref)
    assert ok, f"worst err/bound {ratio:.3f}, normwise {nrm:.2e}"
    assert not bool(torch.isnan(y).any()), "a row was not written"
