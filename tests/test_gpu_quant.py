"""GPU parity of the quantizers against the CPU oracle: FP8 codes and fp32 scales must
match bit for bit (FP8-RL summary page, "Prerequisites / FP8 quantization format" and
"Method step details" steps 1-3).  Every call goes through the C ABI."""
import os
import struct

import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import to_dev_bf16, u8, f32

pytestmark = pytest.mark.gpu
DEV = "cuda"
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_vectors.txt")


def gpu_act(x_bits, ld_s=None):
    m, k = x_bits.shape
    x = to_dev_bf16(x_bits)
    q = torch.empty((m, k), dtype=torch.uint8, device=DEV)
    ld_s = m if ld_s is None else ld_s
    s = torch.full((k // 128, ld_s), -7.0, dtype=torch.float32, device=DEV)
    fq.fp8q_quant_act_g128(x, q, s)
    torch.cuda.synchronize()
    return u8(q), f32(s)


def check_act(x_bits, ld_s=None):
    q, s = gpu_act(x_bits, ld_s)
    qr, sr = oracle.quant_act_g128(x_bits, ld_s)
    m = x_bits.shape[0]
    assert np.array_equal(s[:, :m].view(np.uint32), sr[:, :m].view(np.uint32)), "scales differ"
    bad = np.argwhere(q != qr)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[0]}: gpu {q[tuple(bad[0])]:#x} oracle {qr[tuple(bad[0])]:#x}"
    if ld_s is not None and ld_s > m:
        assert np.all(s[:, m:] == -7.0), "padding of the scale rows was written"


def test_act_hand_vectors():
    rows = []
    want = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].split()
            if len(line) == 6 and line[1] == "group":
                r = np.zeros(128, np.uint16)
                r[0], r[1] = int(line[2], 16), int(line[4], 16)
                rows.append(r)
                want.append((int(line[3], 16), int(line[5], 16)))
    x = np.stack(rows)
    q, s = gpu_act(x)
    for i, (sbits, code) in enumerate(want):
        assert s[0, i].view(np.uint32) == sbits
        assert q[i, 1] == code, f"row {i}: {q[i, 1]:#x} != {code:#x}"
    check_act(x)


def test_act_tiny_and_ragged():
    _, x = synth.tiny()
    check_act(x)
    check_act(synth.activation(2, 0, 7, 13, 384))
    check_act(synth.activation(2, 0, 8, 1, 4096))
    check_act(synth.activation(2, 0, 9, 37, 1024), ld_s=40)


@pytest.mark.parametrize("m", [1, 64, 512, 4096])
def test_act_attention_shapes(m):
    check_act(synth.activation(2, 0, 100 + m, m, 4096))


def test_act_exhaustive_bf16_values():
    """Every finite bf16 value as an element of a group with a few amax choices."""
    allv = np.arange(0, 0x7F80, dtype=np.uint16)
    vals = np.concatenate([allv, allv | 0x8000])
    g = np.random.Generator(np.random.PCG64(3))
    for amax in (0x0008, 0x3DCD, 0x4030, 0x7F7F, int(g.integers(1, 0x7F80))):
        v = vals[(vals & 0x7FFF) <= amax]
        pad = (-len(v)) % 127
        v = np.concatenate([v, np.zeros(pad, np.uint16)]).reshape(-1, 127)
        x = np.zeros((v.shape[0], 128), np.uint16)
        x[:, 0] = amax
        x[:, 1:] = v
        check_act(x)


def test_act_special_values():
    g = np.random.Generator(np.random.PCG64(4))
    x = synth.activation(2, 1, 0, 64, 512)
    x[0, :] = 0                      # all-zero groups -> scale 1
    x[1, :128] = 0x8000              # -0 everywhere
    x[2, :] = x[2, :] & 0x807F       # bf16 subnormals only (tiny-scale path)
    x[3, 128:256] = 0x0001           # smallest subnormal
    x[4, :] = g.integers(0, 0x0100, size=512).astype(np.uint16)  # mixed tiny values
    check_act(x)


def gpu_weight(tensors):
    descs = []
    outs = []
    for w_bits, ld_w, ld_q in tensors:
        n, k = w_bits.shape
        wfull = np.zeros((n, ld_w), np.uint16)
        wfull[:, :k] = w_bits
        w = to_dev_bf16(wfull)[:, :k]
        qfull = torch.full((n, ld_q), 0xA5, dtype=torch.uint8, device=DEV)
        q = qfull[:, :k]
        s = torch.empty((n // 128, k // 128), dtype=torch.float32, device=DEV)
        descs.append((w, q, s))
        outs.append((qfull, s))
    fq.fp8q_quant_weight_blk128(descs)
    torch.cuda.synchronize()
    return [(u8(qf), f32(s)) for qf, s in outs]


def test_act_random_shapes_and_pitches():
    """Seeded random activation shapes with padded row pitches and scale rows: codes and
    scales bit-exact against the oracle, padding untouched."""
    g = np.random.Generator(np.random.PCG64(77))
    for case in range(12):
        m, k = int(g.integers(1, 3000)), 128 * int(g.integers(1, 33))
        ldx, ldq, lds = k + 8 * int(g.integers(0, 5)), k + 16 * int(g.integers(0, 5)), m + int(g.integers(0, 9))
        x_bits = synth.activation(2, 1, case, m, k)
        xfull = np.zeros((m, ldx), np.uint16)
        xfull[:, :k] = x_bits
        x = to_dev_bf16(xfull)[:, :k]
        qfull = torch.full((m, ldq), 0xA5, dtype=torch.uint8, device=DEV)
        sfull = torch.full((k // 128, lds), -7.0, dtype=torch.float32, device=DEV)
        fq.fp8q_quant_act_g128(x, qfull[:, :k], sfull)
        torch.cuda.synchronize()
        q, sc = u8(qfull), f32(sfull)
        qr, sr = oracle.quant_act_g128(x_bits)
        assert np.array_equal(sc[:, :m].view(np.uint32), sr[:, :m].view(np.uint32)), f"case {case}: scales"
        assert np.array_equal(q[:, :k], qr), f"case {case}: codes"
        assert np.all(q[:, k:] == 0xA5) and np.all(sc[:, m:] == -7.0), f"case {case}: padding written"


def test_weight_random_batches():
    """Seeded random batches of weight tensors (1 to 9 per call, random shapes and padded
    pitches): codes and scales bit-exact against the oracle."""
    g = np.random.Generator(np.random.PCG64(78))
    for call in range(6):
        specs = []
        for t in range(int(g.integers(1, 10))):
            n, k = 128 * int(g.integers(1, 13)), 128 * int(g.integers(1, 13))
            specs.append((synth.weight(3, 5 + call, t, n, k), k + 8 * int(g.integers(0, 4)), k + 16 * int(g.integers(0, 4))))
        for (w, _, _), (q, sc) in zip(specs, gpu_weight(specs)):
            k = w.shape[1]
            qr, sr = oracle.quant_weight_blk128(w)
            assert np.array_equal(sc.view(np.uint32), sr.view(np.uint32))
            assert np.array_equal(q[:, :k], qr)
            assert np.all(q[:, k:] == 0xA5)


def test_weight_tiny():
    w, _ = synth.tiny()
    (q, s), = gpu_weight([(w, 256, 256)])
    qr, sr = oracle.quant_weight_blk128(w)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert s[1, 1] == 1.0
    assert np.array_equal(q, qr)


def test_weight_batched_descriptors_and_pitches():
    specs = [(synth.weight(3, 0, i, n, k), ldw, ldq) for i, (n, k, ldw, ldq) in enumerate(
        [(128, 128, 128, 128), (256, 384, 392, 400), (1024, 512, 512, 512), (384, 1280, 1288, 1296)])]
    # more descriptors than fit one launch: 70 small tensors
    specs += [(synth.weight(3, 1, i, 128, 256), 256, 256) for i in range(70)]
    outs = gpu_weight(specs)
    for (w, ldw, ldq), (q, s) in zip(specs, outs):
        k = w.shape[1]
        qr, sr = oracle.quant_weight_blk128(w)
        assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
        assert np.array_equal(q[:, :k], qr)
        assert np.all(q[:, k:] == 0xA5), "bytes beyond k in the row pitch were written"


def test_weight_attention_shapes():
    specs = [(synth.weight(2, 0, 0, 4096, 4096), 4096, 4096), (synth.weight(2, 0, 1, 1024, 4096), 4096, 4096)]
    outs = gpu_weight(specs)
    for (w, _, _), (q, s) in zip(specs, outs):
        qr, sr = oracle.quant_weight_blk128(w)
        assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
        assert np.array_equal(q, qr)


def test_weight_tiny_scale_block():
    w = synth.weight(3, 2, 0, 256, 256)
    w[:128, :128] &= 0x807F   # a block of bf16 subnormals: scale below 2^-116
    w[128:, 128:] = 0x8000    # a block of -0
    (q, s), = gpu_weight([(w, 256, 256)])
    qr, sr = oracle.quant_weight_blk128(w)
    assert np.array_equal(s.view(np.uint32), sr.view(np.uint32))
    assert np.array_equal(q, qr)
    assert np.all(q[128:, 128:] == 0x80)


@pytest.mark.parametrize("ue8m0", [False, True])
def test_weight_wide_launch_equals_per_tensor_calls(ue8m0):
    """A launch of 21846 blocks or more (1 GB of traffic) takes four blocks of a block row per
    workgroup.  Its codes and scales equal per-tensor calls (each below that size: one block per
    workgroup) byte for byte.  K of 1, 2, 3, 5, 6, 7, 24, 32 and 16 blocks covers every count of
    live blocks in a row's last workgroup; pitches are padded and the bytes beyond k must stay
    untouched.  Two blocks of each tensor are also checked against the oracle.  Both the fp32
    and the power-of-two (UE8M0) scale variants."""
    quant = fq.fp8q_quant_weight_blk128_ue8m0 if ue8m0 else fq.fp8q_quant_weight_blk128
    g = torch.Generator(device=DEV)
    g.manual_seed(11)
    shapes = [(12800, 128, 192, 144), (12800, 256, 264, 272), (12800, 384, 384, 400), (12800, 640, 648, 656),
              (8192, 768, 768, 768), (25600, 896, 904, 912), (25600, 3072, 3072, 3072),
              (25600, 4096, 4104, 4112), (51200, 2048, 2048, 2048), (12800, 4096, 4096, 4096)]
    assert sum((n // 128) * (k // 128) for n, k, _, _ in shapes) >= 21846
    ws, wide, single = [], [], []
    for n, k, ldw, ldq in shapes:
        x = torch.randn((n, ldw), generator=g, device=DEV) * 0.02
        x[torch.rand((n, ldw), generator=g, device=DEV) < 1e-3] *= 20.0
        ws.append(x.to(torch.bfloat16)[:, :k])
        for outs in (wide, single):
            qfull = torch.full((n, ldq), 0xA5, dtype=torch.uint8, device=DEV)
            outs.append((qfull, torch.empty((n // 128, k // 128), dtype=torch.float32, device=DEV)))
    quant([(w, q[:, :w.shape[1]], s) for w, (q, s) in zip(ws, wide)])
    for w, (q, s) in zip(ws, single):
        quant([(w, q[:, :w.shape[1]], s)])
    torch.cuda.synchronize()
    for (n, k, _, ldq), w, (qw, sw), (q1, s1) in zip(shapes, ws, wide, single):
        assert torch.equal(sw.view(torch.int32), s1.view(torch.int32)), f"{n}x{k}: scales differ"
        assert torch.equal(qw, q1), f"{n}x{k}: codes differ"
        if ldq > k:
            assert bool(torch.all(qw[:, k:] == 0xA5)), f"{n}x{k}: bytes beyond k were written"
        for bi, bj in ((0, k // 128 - 1), (n // 256, (k // 128) // 2)):
            wb = w[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128].contiguous().view(torch.int16)
            qr, sr = oracle.quant_weight_blk128(wb.cpu().numpy().view(np.uint16), ue8m0=ue8m0)
            assert np.float32(sw[bi, bj].item()).view(np.uint32) == sr.reshape(-1)[0].view(np.uint32)
            assert np.array_equal(u8(qw[128 * bi:128 * bi + 128, 128 * bj:128 * bj + 128]), qr)


# ----------------------------------------------------------------------------- KV
def gpu_kv(k_bits, v_bits, slots, pages, page_size, k_scale=1.0, v_scale=1.0, recal=True, rng=448.0):
    t, h, d = k_bits.shape
    k = to_dev_bf16(k_bits.reshape(t, h * d)).view(t, h, d)
    v = to_dev_bf16(v_bits.reshape(t, h * d)).view(t, h, d)
    kc = torch.full((pages, page_size, h, d), 0x7F, dtype=torch.uint8, device=DEV)
    vc = torch.full((pages, page_size, h, d), 0x7F, dtype=torch.uint8, device=DEV)
    ks = torch.tensor([k_scale], dtype=torch.float32, device=DEV)
    vs = torch.tensor([v_scale], dtype=torch.float32, device=DEV)
    fq.fp8q_kv_quant(k, v, torch.from_numpy(slots).to(DEV), kc, vc, ks, vs, rng, recalibrate=recal)
    torch.cuda.synchronize()
    return u8(kc), u8(vc), f32(ks)[0], f32(vs)[0]


def check_kv(k_bits, v_bits, slots, pages, page_size, **kw):
    kc, vc, ks, vs = gpu_kv(k_bits, v_bits, slots, pages, page_size, **kw)
    h, d = k_bits.shape[1:]
    sentinel = np.full((pages, page_size, h, d), 0x7F, np.uint8)
    rk, rv, rks, rvs = oracle.kv_quant(k_bits, v_bits, slots, sentinel, sentinel, page_size,
                                       k_scale=kw.get("k_scale", 1.0), v_scale=kw.get("v_scale", 1.0),
                                       rng=kw.get("rng", 448.0), recalibrate=kw.get("recal", True))
    assert np.float32(ks).view(np.uint32) == np.float32(rks).view(np.uint32)
    assert np.float32(vs).view(np.uint32) == np.float32(rvs).view(np.uint32)
    assert np.array_equal(kc, rk)
    assert np.array_equal(vc, rv)


def test_kv_small_with_skips():
    g = np.random.Generator(np.random.PCG64(12))
    t, pages = 300, 24
    k = synth.kv_values(5, 0, 0, t)
    v = synth.kv_values(5, 0, 1, t)
    slots = g.permutation(pages * 16)[:t].astype(np.int64)
    slots[g.choice(t, 17, replace=False)] = -1
    k[np.nonzero(slots < 0)[0][0], 0, 0] = 0x4F00  # a large value in a skipped token
    check_kv(k, v, slots, pages, 16)


def test_kv_stored_scale_saturation_and_other_heads():
    g = np.random.Generator(np.random.PCG64(13))
    t, h, pages = 50, 3, 8
    k = synth.to_bf16_bits(8 * g.standard_normal((t, h, 128), dtype=np.float32))
    v = synth.to_bf16_bits(g.standard_normal((t, h, 128), dtype=np.float32))
    slots = g.permutation(pages * 8)[:t].astype(np.int64)
    check_kv(k, v, slots, pages, 8, k_scale=0.0625, v_scale=0.001, recal=False)
    check_kv(k, v, slots, pages, 8, rng=240.0)


def test_kv_hand_vector_p5():
    k = np.zeros((5, 1, 128), np.uint16)
    k[:, 0, 0] = [0x42C8, 0xC270, 0x4266, 0x4264, 0x4268]
    kc, vc, ks, vs = gpu_kv(k, k, np.arange(5, dtype=np.int64), 1, 16, k_scale=0.125, v_scale=0.125,
                            recal=False)
    assert list(kc[0, :5, 0, 0]) == [0x7E, 0xFE, 0x7E, 0x7E, 0x7E]
    assert np.all(kc[0, 5:] == 0x7F)


def test_kv_sequences_pages():
    slots, pages = synth.kv_slot_mapping(5, 0, seqs=8, seq_len=700)
    t = len(slots)
    check_kv(synth.kv_values(5, 1, 0, t), synth.kv_values(5, 1, 1, t), slots, pages, 16)


def test_kv_random_cases():
    """Seeded random token counts, head counts, page sizes, skipped slots, stored or
    recalibrated scales and E4M3 ranges: cache bytes and scales bit-exact."""
    g = np.random.Generator(np.random.PCG64(31))
    for case in range(10):
        t, h = int(g.integers(1, 2500)), int(g.integers(1, 9))
        ps = int(g.choice([1, 5, 8, 16]))
        pages = -(-t // ps) + int(g.integers(0, 4))
        slots = g.permutation(pages * ps)[:t].astype(np.int64)
        slots[g.random(t) < 0.1] = -1
        k = synth.to_bf16_bits(float(g.choice([0.1, 1.0, 30.0])) * g.standard_normal((t, h, 128), dtype=np.float32))
        v = synth.to_bf16_bits(g.standard_normal((t, h, 128), dtype=np.float32))
        recal = bool(g.integers(0, 2))
        check_kv(k, v, slots, pages, ps, recal=recal, rng=float(g.choice([448.0, 240.0])),
                 k_scale=float(g.choice([0.01, 0.25, 2.0])), v_scale=float(g.choice([0.005, 0.125])))


@pytest.mark.parametrize("heads", [9, 12, 16])
def test_kv_rows_longer_than_one_pass(heads):
    """Token rows of more than 1024 elements take several passes of the lane layout."""
    g = np.random.Generator(np.random.PCG64(heads))
    t, pages = 700, 50
    k = synth.to_bf16_bits(g.standard_normal((t, heads, 128), dtype=np.float32))
    v = synth.to_bf16_bits(3 * g.standard_normal((t, heads, 128), dtype=np.float32))
    slots = g.permutation(pages * 16)[:t].astype(np.int64)
    slots[g.random(t) < 0.05] = -1
    check_kv(k, v, slots, pages, 16)
    check_kv(k, v, slots, pages, 16, recal=False, k_scale=0.004, v_scale=0.02)


def test_kv_empty_call_recalibrates_to_one():
    k = np.zeros((0, 8, 128), np.uint16)
    kc, vc, ks, vs = gpu_kv(k, k, np.zeros(0, np.int64), 1, 16, k_scale=3.0, v_scale=3.0)
    assert ks == 1.0 and vs == 1.0


def test_determinism():
    x = synth.activation(2, 3, 0, 512, 4096)
    a = gpu_act(x)
    b = gpu_act(x)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
