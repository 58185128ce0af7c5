"""Oracle GEMMs pinned by brute force, by a library routine and by linearity.

The block-scaled W8A8 product (FP8-RL summary page, "Method step details" step 1:
FP8 weights with one scale per 128x128 block times dynamically quantized
activations) is y[m,n] = sum_kb a_s[kb,m] * b_s[n/128,kb] * sum_{k in kb}
dec(a[m,k]) dec(b[n,k]).  Dequantizing each operand block by block and taking
an ordinary product gives the same real number, so numpy's float64 matmul of the
dequantized operands (decoded with torch's float8_e4m3fn, not the oracle's
table) must agree with the oracle to fp64 rounding.
"""
from fractions import Fraction

import numpy as np
import torch

import oracle
from fp8_block_scaled_weight_amd import synth


def _dec(codes):
    t = torch.from_numpy(np.ascontiguousarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn)
    return t.double().numpy()


def _dequant_a(q, s):  # s: [k/128, m]
    m, k = q.shape
    return _dec(q) * np.repeat(s.T.astype(np.float64)[:, : k // 128], 128, axis=1)[:m]


def _dequant_b(q, s):  # s: [n/128, k/128]
    return _dec(q) * np.kron(s.astype(np.float64), np.ones((128, 128)))


def _e4m3_fraction(code: int) -> Fraction:
    """E4M3FN value from the format definition, as an exact rational."""
    e, m = (code >> 3) & 15, code & 7
    v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


def _tiny():
    w, x = synth.tiny()
    wq, ws = oracle.quant_weight_blk128(w)
    xq, xs = oracle.quant_act_g128(x)
    return xq, xs, wq, ws


def test_tiny_bruteforce_fractions():
    """Exact rational evaluation of a 4 x 256 slice of the Tiny GEMM (2x2 weight blocks)."""
    xq, xs, wq, ws = _tiny()
    y = oracle.gemm_w8a8(xq, xs, wq, ws)
    dec = {c: _e4m3_fraction(c) for c in range(256) if c not in (0x7F, 0xFF)}
    for i in (0, 5, 10, 15):
        for j in range(256):
            tot = Fraction(0)
            for kb in range(2):
                part = sum(dec[int(xq[i, t])] * dec[int(wq[j, t])] for t in range(kb * 128, kb * 128 + 128))
                tot += Fraction(float(xs[kb, i])) * Fraction(float(ws[j // 128, kb])) * part
            ref = float(tot)
            assert abs(y[i, j] - ref) <= 1e-12 * max(abs(ref), 1e-30), (i, j)


def test_matches_numpy_matmul_of_dequantized_operands():
    w = synth.weight(98, 0, 0, 256, 512)
    x = synth.activation(98, 0, 1, 48, 512)
    wq, ws = oracle.quant_weight_blk128(w)
    xq, xs = oracle.quant_act_g128(x)
    y = oracle.gemm_w8a8(xq, xs, wq, ws)
    a = _dequant_a(xq, xs)
    b = _dequant_b(wq, ws)
    ref = a @ b.T
    bound = 1e-12 * (np.abs(a) @ np.abs(b).T)
    assert np.all(np.abs(y - ref) <= bound + 1e-300)


def test_lossless_special_case_equals_matmul_of_inputs():
    """Blocks made of 2^j * (E4M3 values) with max exactly 448 * 2^j quantize losslessly
    (scale 2^j), so the block-scaled GEMM equals the float64 matmul of the bf16 inputs."""
    g = np.random.Generator(np.random.PCG64(21))
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = _dec(finite)

    def make_exact(rows, cols, rb, cb):
        out = np.empty((rows, cols), dtype=np.float32)
        for i in range(0, rows, rb):
            for j in range(0, cols, cb):
                p = 2.0 ** int(g.integers(-3, 4))
                blk = g.choice(vals, size=(rb, cb))
                blk.flat[int(g.integers(0, rb * cb))] = 448.0
                out[i:i + rb, j:j + cb] = blk * p
        return out

    wf = make_exact(256, 384, 128, 128)
    xf = make_exact(16, 384, 1, 128)
    w = synth.to_bf16_bits(wf)
    x = synth.to_bf16_bits(xf)
    assert np.array_equal(synth.bf16_bits_to_f32(w), wf)
    wq, ws = oracle.quant_weight_blk128(w)
    xq, xs = oracle.quant_act_g128(x)
    assert np.all(np.log2(ws) == np.round(np.log2(ws)))
    y = oracle.gemm_w8a8(xq, xs, wq, ws)
    ref = xf.astype(np.float64) @ wf.astype(np.float64).T
    assert np.array_equal(y, ref)


def test_scale_linearity():
    """Doubling one weight block's scale adds exactly that block's contribution once more."""
    xq, xs, wq, ws = _tiny()
    y0 = oracle.gemm_w8a8(xq, xs, wq, ws)
    ws2 = ws.copy()
    ws2[1, 0] *= 2
    y1 = oracle.gemm_w8a8(xq, xs, wq, ws2)
    xs_only0 = xs.copy()
    xs_only0[1, :] = 0
    contrib = oracle.gemm_w8a8(xq, xs_only0, wq, ws)[:, 128:]
    assert np.array_equal(y1[:, :128], y0[:, :128])
    assert np.allclose(y1[:, 128:] - y0[:, 128:], contrib, rtol=1e-13, atol=1e-13 * np.abs(y0).max())


def test_grouped_equals_dense_per_group():
    g = np.random.Generator(np.random.PCG64(8))
    G, n, k = 5, 256, 256
    sizes = np.array([3, 0, 17, 1, 9])  # includes an empty group
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m = int(off[-1])
    b_bits = np.stack([synth.weight(97, e, 0, n, k) for e in range(G)])
    bq = np.empty((G, n, k), np.uint8)
    bs = np.empty((G, n // 128, k // 128), np.float32)
    for e in range(G):
        bq[e], bs[e] = oracle.quant_weight_blk128(b_bits[e])
    x = synth.to_bf16_bits(g.standard_normal((m, k), dtype=np.float32))
    aq, as_ = oracle.quant_act_g128(x)
    y = oracle.grouped_gemm_w8a8(aq, as_, bq, bs, off)
    for e in range(G):
        r0, r1 = off[e], off[e + 1]
        if r1 == r0:
            continue
        ye = oracle.gemm_w8a8(aq[r0:r1], as_[:, r0:r1], bq[e], bs[e])
        assert np.array_equal(y[r0:r1], ye)


def test_blockwise_matmul_form_equals_the_scalar_oracle():
    """The full-size form (one float64 matrix product per K block, then the scaled outer
    sum in K-block order) gives the scalar oracle's numbers bit for bit: every block sum is
    exact in fp64, and the outer sum takes the same operations in the same order.  Codes
    span the whole finite range, with the largest magnitudes forced into one row and one
    column so block sums reach their largest values."""
    g = np.random.Generator(np.random.PCG64(31))
    m, n, k = 70, 256, 640
    codes = np.concatenate([np.arange(0, 0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    a = g.choice(codes, size=(m, k))
    b = g.choice(codes, size=(n, k))
    a[5], b[7] = 0x7E, 0x7E          # 128 * 448 * 448 block sums
    b[9] = 0xFE
    a_s = np.zeros((k // 128, m + 6), np.float32)   # padded ld_as
    a_s[:, :m] = g.uniform(1e-4, 3.0, size=(k // 128, m)).astype(np.float32)
    b_s = g.uniform(1e-5, 1e-2, size=(n // 128, k // 128)).astype(np.float32)
    y_ref = oracle.gemm_w8a8(a, a_s, b, b_s)
    y = oracle.gemm_w8a8_blockwise(a, a_s, b, b_s)
    assert np.array_equal(y, y_ref)
    assert np.abs(y).max() > 1e3


def test_e4m3_table_matches_the_format_definition():
    t = oracle.e4m3_table()
    for c in range(256):
        if c & 0x7F == 0x7F:
            assert np.isnan(t[c])
        else:
            assert t[c] == float(_e4m3_fraction(c))
