"""Oracle of the power-of-two (UE8M0) scale variant, pinned without the oracle itself.

FP8-RL summary page, "Experimental results" (scale-format ablation): FP32 scale
factors give the lowest mismatch, UE8M0 (power-of-two) scales a coarser
granularity.  Reading taken: scale = the smallest power of two 2^e with
448 * 2^e >= amax (so the block maximum still fits the E4M3 range), e in the E8M0
range [-127, 127]; 1 for an all-zero block.  With a power-of-two scale the quotient
x / scale is exact, so the codes are the E4M3 roundings of exactly representable
values: they are pinned against torch's float8_e4m3fn cast.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from fp8_block_scaled_weight_amd import synth

BF16_MAX = float(np.frombuffer(np.uint32(0x7F7F0000).tobytes(), np.float32)[0])


def _rule(amax: float) -> Fraction:
    """Brute force in exact rationals: the smallest e with 448 * 2^e >= amax, clamped."""
    if amax == 0:
        return Fraction(1)
    a = Fraction(amax)
    e = -200
    while Fraction(448) * Fraction(2) ** e < a:
        e += 1
    e = max(-127, min(127, e))
    return Fraction(2) ** e


@pytest.mark.parametrize("amax,expected", [
    (448.0, 1.0), (449.0, 2.0), (224.0, 0.5), (224.5, 1.0), (1.0, 2.0 ** -8), (0.0, 1.0),
    (2.0 ** -133, 2.0 ** -127),          # below the E8M0 range: clamped to 2^-127 (a binary32 subnormal)
    (BF16_MAX, 2.0 ** 120),              # largest bf16: 448 * 2^119 < 3.39e38 <= 448 * 2^120
    (0.10009765625, 2.0 ** -12),         # 448 * 2^-12 = 0.109 >= 0.1001 > 448 * 2^-13
])
def test_hand_scales(amax, expected):
    assert float(oracle.scale_ue8m0(amax)) == expected


def test_scale_rule_brute_force():
    g = np.random.Generator(np.random.PCG64(11))
    bits = g.integers(1, 0x7F80, size=3000, dtype=np.uint32).astype(np.uint16)
    vals = list(synth.bf16_bits_to_f32(bits).astype(np.float64))
    # boundaries: 448 * 2^k and its bf16 neighbours
    for k in (-40, -9, -1, 0, 1, 7, 60):
        b = 448.0 * 2.0 ** k
        vals += [b, float(np.nextafter(np.float32(b), np.float32(0))), float(np.nextafter(np.float32(b), np.float32(np.inf)))]
    for a in vals:
        assert Fraction(float(oracle.scale_ue8m0(a))) == _rule(a), a


def _torch_codes(x_f64, s_f64):
    """E4M3 codes of the exact quotients through torch's float8_e4m3fn cast (RNE)."""
    u = torch.from_numpy(x_f64 / s_f64).float()  # exact: power-of-two scale, <= 8 significant bits
    return u.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_weight_blocks_match_library_cast():
    w = synth.weight(3, 0, 0, 256, 384)
    w[:128, 128:256] = 0  # one all-zero block
    q, s = oracle.quant_weight_blk128(w, ue8m0=True)
    x = synth.bf16_bits_to_f32(w).astype(np.float64)
    for bi in range(2):
        for bj in range(3):
            blk = x[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            sc = float(s[bi, bj])
            amax = np.abs(blk).max()
            assert Fraction(sc) == _rule(amax)
            if amax == 0:
                assert sc == 1.0 and np.all(q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] == 0)
                continue
            # power of two with the block maximum in (224, 448]
            assert 224 < amax / sc <= 448
            got = q[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128]
            assert np.array_equal(got, _torch_codes(blk, sc))


def test_activation_groups_match_library_cast():
    x_bits = synth.activation(2, 0, 3, 24, 512)
    q, s = oracle.quant_act_g128(x_bits, ld_s=29, ue8m0=True)
    x = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    for r in range(24):
        for g in range(4):
            grp = x[r, g * 128:(g + 1) * 128]
            sc = float(s[g, r])
            assert Fraction(sc) == _rule(np.abs(grp).max())
            assert np.array_equal(q[r, g * 128:(g + 1) * 128], _torch_codes(grp, sc))


def test_power_of_two_blocks_agree_with_fp32_scales():
    """Where amax / 448 is itself a power of two, both scale rules give the same scale
    and codes (the FP32-scale oracle is pinned separately)."""
    w = synth.weight(3, 0, 1, 128, 256)
    x = synth.bf16_bits_to_f32(w)
    for bj, k in ((0, -7), (1, -6)):
        blk = x[:, bj * 128:(bj + 1) * 128]
        idx = np.unravel_index(np.argmax(np.abs(blk)), blk.shape)
        amax_bits = synth.to_bf16_bits(np.array([448.0 * 2.0 ** k], np.float32))[0]
        w[idx[0], bj * 128 + idx[1]] = amax_bits  # exact 448 * 2^k, still the maximum
    q8, s8 = oracle.quant_weight_blk128(w, ue8m0=True)
    q32, s32 = oracle.quant_weight_blk128(w)
    assert np.array_equal(s8, s32) and np.array_equal(q8, q32)


# ------------------------------------------------- SwiGLU + 1x128 quantization, UE8M0
def test_swiglu_saturated_gate_reduces_to_activation_quantizer():
    """Every gate >= 40 makes the SiLU factor exactly 1 in fp64, so up = 1 turns the
    power-of-two SwiGLU quantization into the power-of-two activation quantizer of the
    gate values (pinned above against torch's cast), and up = -1 flips every sign."""
    m, n = 6, 384
    g = synth.bf16_bits_to_f32(synth.activation(4, 2, 17, m, n)).astype(np.float64)
    gate = synth.to_bf16_bits((40.0 + np.abs(g) * 30.0).astype(np.float32))
    for up, flip in ((1.0, 0x00), (-1.0, 0x80)):
        h = np.concatenate([gate, synth.to_bf16_bits(np.full((m, n), up, np.float32))], axis=1)
        q, s = oracle.swiglu_quant_g128(h, ue8m0=True)
        q_ref, s_ref = oracle.quant_act_g128(gate, ue8m0=True)
        assert np.array_equal(s, s_ref)
        assert np.array_equal(q, q_ref ^ flip)


def test_swiglu_scales_and_codes_exact_rational():
    """Each group's scale is the rule's power of two for the exact fp64 group maximum
    (brute force in rationals), and every code is the E4M3 nearest of a / scale."""
    from tests.test_oracle_bruteforce import brute_code
    m, n = 10, 256
    h = np.concatenate([synth.activation(4, 3, 11, m, n), synth.activation(4, 3, 12, m, n)], axis=1)
    h[0, :128] = 0                                                  # zero gate group: scale 1
    h[1, n:n + 128] = synth.to_bf16_bits(np.full(128, 2.0 ** -130, np.float32))  # tiny: clamped
    q, s, amax = oracle.swiglu_quant_g128(h, ld_s=m + 1, with_amax=True, ue8m0=True)
    x = synth.bf16_bits_to_f32(h).astype(np.float64)
    a = np.array([[oracle.silu_times_up(x[r, c], x[r, n + c]) for c in range(n)] for r in range(m)])
    assert s[0, 0] == 1.0 and np.all(q[0, :128] & 0x7F == 0)
    assert s[0, 1] == np.float32(2.0 ** -127)
    for r in range(m):
        for gi in range(n // 128):
            grp = a[r, gi * 128:(gi + 1) * 128]
            am = float(np.abs(grp).max())
            assert amax[gi, r] == am
            assert Fraction(float(s[gi, r])) == _rule(am)
            for c in range(128):
                assert q[r, gi * 128 + c] == brute_code(grp[c], float(s[gi, r]))
