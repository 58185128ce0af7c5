"""Property-based pins of the oracle (hypothesis): random inputs checked against
definitions written out here with exact rationals, independent of the oracle's code.

- 1x128 quantization (FP8-RL summary page, "Prerequisites / FP8 quantization format" and
  "Method step details" step 1, with the readings scale = fl32(amax / 448), an all-zero group
  scale 1, and the exact quotient rounded once to the nearest E4M3FN value, ties to even):
  any finite bf16 group, subnormals and -0 included.
- The block-scaled GEMM: random small shapes and codes against the exact rational sum.
- The KV scales (step 3: recalibrated per step): amax over the tokens actually written.
"""
from fractions import Fraction

import numpy as np
import torch
from hypothesis import HealthCheck, given, settings, strategies as st

import oracle
from fp8_block_scaled_weight_amd import synth

SETTINGS = settings(max_examples=40, deadline=None, suppress_health_check=[HealthCheck.too_slow])


def _e4m3(code: int) -> Fraction:
    """E4M3FN value of a code from the format definition (bias 7, 3 mantissa bits)."""
    e, m = (code >> 3) & 15, code & 7
    v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


_POS = [(c, _e4m3(c)) for c in range(0x7F)]  # finite non-negative codes, increasing


def _nearest(q: Fraction, negative: bool) -> int:
    """Nearest E4M3FN code to the real q (ties to the even code; |q| clamps to 448)."""
    a = min(abs(q), Fraction(448))
    best = None
    for c, v in _POS:
        d = abs(v - a)
        if best is None or d < best[1] or (d == best[1] and c % 2 == 0):
            best = (c, d)
    return best[0] | (0x80 if negative else 0)


def _f32_nearest(fr: Fraction) -> np.float32:
    """The binary32 value nearest to a positive rational (ties to the even significand),
    decided with exact comparisons."""
    c = np.float32(float(fr))
    cands = {c, np.nextafter(c, np.float32(0)), np.nextafter(c, np.float32(np.inf))}
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr), int(np.float32(v).view(np.uint32)) & 1))
    return np.float32(best)


def _bf16_value(bits: int) -> Fraction:
    f = np.array([bits], np.uint16).astype(np.uint32) << 16
    return Fraction(float(f.view(np.float32)[0]))


finite_bf16 = st.integers(0, 0xFFFF).filter(lambda b: (b & 0x7F80) != 0x7F80)


@SETTINGS
@given(st.lists(finite_bf16, min_size=128, max_size=128), st.integers(0, 3))
def test_group_quantization_is_the_exact_rounding(bits, shift):
    # shift the group toward small magnitudes now and then (subnormal scales and codes)
    x = np.array(bits, np.uint16)
    if shift:
        x = np.where((x & 0x7F80) > (shift << 7) * 8, x - ((shift * 8) << 7), x).astype(np.uint16)
    q, s = oracle.quant_act_g128(x.reshape(1, 128))
    vals = [_bf16_value(int(b)) for b in x]
    amax = max(abs(v) for v in vals)
    scale = np.float32(1.0) if amax == 0 else _f32_nearest(amax / 448)
    assert s[0, 0].view(np.uint32) == scale.view(np.uint32)
    sc = Fraction(float(scale))
    for i, v in enumerate(vals):
        neg = bool(int(x[i]) & 0x8000)
        assert q[0, i] == _nearest(v / sc, neg), (i, hex(int(x[i])), float(v), float(sc))


@SETTINGS
@given(st.integers(1, 5), st.integers(1, 2), st.integers(1, 2), st.integers(0, 2 ** 32 - 1))
def test_gemm_is_the_exact_block_scaled_sum(m, nb, kb, seed):
    g = np.random.default_rng(seed)
    n, k = 128 * nb, 128 * kb
    codes = np.concatenate([np.arange(0, 0x7F), np.arange(0x80, 0xFF)]).astype(np.uint8)
    a = g.choice(codes, size=(m, k))
    b = g.choice(codes, size=(n, k))
    a_s = g.uniform(1e-3, 2.0, size=(kb, m)).astype(np.float32)
    b_s = g.uniform(1e-4, 1e-1, size=(nb, kb)).astype(np.float32)
    y = oracle.gemm_w8a8(a, a_s, b, b_s)
    dec = [_e4m3(c) for c in range(256)]
    for i in range(m):
        for j in range(0, n, 37):
            terms = [Fraction(float(a_s[t, i])) * Fraction(float(b_s[j // 128, t]))
                     * sum(dec[a[i, kk]] * dec[b[j, kk]] for kk in range(128 * t, 128 * t + 128))
                     for t in range(kb)]
            exact = sum(terms)
            # fp64 rounds each scaled block sum and the outer sum once: a few ulps of sum |terms|
            tol = sum(abs(x) for x in terms) * Fraction(1, 2 ** 50) + Fraction(1, 2 ** 1000)
            assert abs(Fraction(y[i, j]) - exact) <= tol


@SETTINGS
@given(st.integers(1, 40), st.integers(0, 2 ** 32 - 1), st.floats(1.0, 1000.0))
def test_kv_scales_are_the_amax_of_the_written_tokens(t, seed, rng):
    g = np.random.default_rng(seed)
    k = synth.to_bf16_bits(g.standard_normal((t, 256)).astype(np.float32) * g.uniform(0.01, 50))
    v = synth.to_bf16_bits(g.standard_normal((t, 256)).astype(np.float32) * g.uniform(0.01, 50))
    slots = g.permutation(64)[:t].astype(np.int64)
    slots[g.random(t) < 0.3] = -1
    ks, vs = oracle.kv_scales(k, v, slots, rng)
    rng32 = np.float32(rng)
    for bits, got in ((k, ks), (v, vs)):
        live = synth.bf16_bits_to_f32(bits)[slots >= 0]
        amax = float(np.abs(live).max()) if live.size else 0.0
        want = np.float32(1.0) if amax == 0 else _f32_nearest(Fraction(amax) / Fraction(float(rng32)))
        assert np.float32(got).view(np.uint32) == want.view(np.uint32)
