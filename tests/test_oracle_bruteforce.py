"""Oracle pinned by brute force and by a library routine.

* Exhaustive bf16 sweeps: for each amax in a seeded set, every finite bf16 x
  with |x| <= amax (both signs) is quantized by the oracle and by an exact
  rational nearest-value search written here from the E4M3FN definition (FP8-RL
  summary page, "Prerequisites / FP8 quantization format").  They must agree on
  every code and on the scale.
* torch's CPU float8_e4m3fn cast (round to nearest even) must agree with the
  oracle's encoder on every float32 value of magnitude <= 448 that is tested,
  including exact midpoints and their fp32 neighbours.
"""
import bisect
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle


def _e4m3_value(code: int) -> Fraction:
    e, m = (code >> 3) & 15, code & 7
    v = Fraction(m, 512) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
    return -v if code & 0x80 else v


POS = [_e4m3_value(c) for c in range(127)]
MIDS = [(POS[i] + POS[i + 1]) / 2 for i in range(126)]


def brute_code(x: float, s: float) -> int:
    """Nearest E4M3FN code to the exact rational x/s; ties to even; clamp to 448."""
    q = Fraction(x) / Fraction(s)
    a = min(abs(q), Fraction(448))
    i = bisect.bisect_left(MIDS, a)  # MIDS[i-1] < a <= MIDS[i]
    if i < 126 and MIDS[i] == a and (i & 1):
        i += 1
    return i | (0x80 if math.copysign(1.0, x) < 0 else 0)


def _bf16_f32(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32)


ALL_POS_BF16 = np.arange(0, 0x7F80, dtype=np.uint32)  # +0 .. largest finite


def _amax_set():
    fixed = [0x0001, 0x0003, 0x0008, 0x0080, 0x00FF, 0x0A31, 0x1F00, 0x3700, 0x3DCD, 0x3DD0,
             0x3F80, 0x4030, 0x4060, 0x43E0, 0x4C1B, 0x7F7F]
    g = np.random.Generator(np.random.PCG64(7))
    rand = [int(v) for v in g.integers(0x0001, 0x7F80, size=40)]
    return fixed + rand


@pytest.mark.slow
@pytest.mark.parametrize("amax_bits", _amax_set())
def test_exhaustive_bf16_sweep(amax_bits):
    xs = ALL_POS_BF16[ALL_POS_BF16 <= amax_bits]
    xs = np.concatenate([xs, xs | 0x8000]).astype(np.uint16)  # both signs, -0 included
    per = 127
    pad = (-len(xs)) % per
    xs_p = np.concatenate([xs, np.zeros(pad, dtype=np.uint16)])
    groups = xs_p.reshape(-1, per)
    grid = np.zeros((groups.shape[0], 128), dtype=np.uint16)
    grid[:, 0] = amax_bits
    grid[:, 1:] = groups
    q, s = oracle.quant_act_g128(grid)
    amax = float(_bf16_f32(amax_bits))
    s_ref = np.float32(np.float32(amax) / np.float32(448.0))
    assert np.all(s.view(np.uint32) == s_ref.view(np.uint32))
    got = q[:, 1:].reshape(-1)[: len(xs)]
    xf = _bf16_f32(xs)
    sf = float(s_ref)
    want = np.array([brute_code(float(x), sf) for x in xf], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"first mismatch x={xf[bad[0]]!r} oracle={got[bad[0]]:#x} brute={want[bad[0]]:#x}"


def _torch_e4m3(v: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def _encode_many(v: np.ndarray) -> np.ndarray:
    return np.array([oracle.e4m3_encode(float(x)) for x in v], dtype=np.uint8)


def test_encoder_matches_torch_cast_on_bf16_grid():
    xs = _bf16_f32(ALL_POS_BF16)
    xs = xs[xs <= 448.0]
    xs = np.concatenate([xs, -xs])
    assert np.array_equal(_encode_many(xs), _torch_e4m3(xs))


def test_encoder_matches_torch_cast_at_midpoints():
    pos = np.array([float(v) for v in POS], dtype=np.float64)
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)  # exact in fp32
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(0))
    xs = np.concatenate([mids, up, dn, pos.astype(np.float32)])
    xs = xs[np.abs(xs) <= 448.0]
    xs = np.concatenate([xs, -xs])
    assert np.array_equal(_encode_many(xs), _torch_e4m3(xs))


def test_encoder_matches_torch_cast_random():
    g = np.random.Generator(np.random.PCG64(11))
    mag = np.exp2(g.uniform(-14, math.log2(448.0), size=60000)).astype(np.float32)
    xs = np.where(g.random(60000) < 0.5, -mag, mag).astype(np.float32)
    assert np.array_equal(_encode_many(xs), _torch_e4m3(xs))


def test_decode_anchors():
    anchors = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0,
               0x40: 2.0, 0x70: 128.0, 0x76: 224.0, 0x7E: 448.0, 0xFE: -448.0, 0xB8: -1.0}
    for c, v in anchors.items():
        assert oracle.e4m3_decode(c) == v
    assert math.isnan(oracle.e4m3_decode(0x7F)) and math.isnan(oracle.e4m3_decode(0xFF))
    assert math.copysign(1.0, oracle.e4m3_decode(0x80)) < 0
    # decode agrees with torch's float8_e4m3fn view for every finite code
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    tv = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    ov = np.array([oracle.e4m3_decode(int(c)) for c in codes])
    assert np.array_equal(tv.astype(np.float64), ov)


def test_encoder_never_emits_nan_and_saturates():
    for u in (448.0, 463.999, 464.0, 480.0, 1e30, float(np.finfo(np.float64).max)):
        assert oracle.e4m3_encode(u) == 0x7E
        assert oracle.e4m3_encode(-u) == 0xFE
    assert oracle.e4m3_encode(-0.0) == 0x80
    assert oracle.e4m3_encode(0.0) == 0x00
