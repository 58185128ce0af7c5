"""Oracle pinned to hand-computed E4M3FN encodings (tests/golden/e4m3_hand_vectors.txt).

The vectors follow the blockwise rule of the FP8-RL summary page, section
"Prerequisites / FP8 quantization format", under the readings listed in the
fixture header.  P3, P7 and P8 separate the exact-quotient reading from the
fp32-division and reciprocal shortcuts.
"""
import os
import struct

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "e4m3_hand_vectors.txt")


def _cases():
    out = []
    with open(GOLDEN) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            case, kind, amax, scale, x, code = line.split()
            out.append((case, kind, int(amax, 16), int(scale, 16), int(x, 16), int(code, 16)))
    return out


CASES = _cases()


def _f32_bits(v) -> int:
    return struct.unpack("<I", struct.pack("<f", float(v)))[0]


def test_fixture_has_all_cases():
    names = {c[0] for c in CASES}
    for need in ("P1d", "P1f", "P3", "P4", "P5e", "P6a", "P7", "P8"):
        assert need in names


@pytest.mark.parametrize("case,kind,amax,scale,x,code", CASES, ids=[c[0] for c in CASES])
def test_hand_vector(case, kind, amax, scale, x, code):
    if kind == "group":
        g = np.zeros((1, 128), dtype=np.uint16)
        g[0, 0] = amax
        g[0, 1] = x
        q, s = oracle.quant_act_g128(g)
        assert _f32_bits(s[0, 0]) == scale, f"{case}: scale {_f32_bits(s[0, 0]):#010x}"
        assert q[0, 1] == code, f"{case}: code {q[0, 1]:#04x} != {code:#04x}"
        assert q[0, 0] == 0x7E  # the amax element always maps to 448
    elif kind == "zero_block":
        w = np.zeros((128, 128), dtype=np.uint16)
        q, s = oracle.quant_weight_blk128(w)
        assert _f32_bits(s[0, 0]) == scale
        assert np.all(q == code)
    elif kind == "stored":
        sc = struct.unpack("<f", struct.pack("<I", scale))[0]
        k = np.zeros((1, 1, 128), dtype=np.uint16)
        k[0, 0, 0] = x
        cache = np.full((1, 16, 1, 128), 0x7F, dtype=np.uint8)
        kc, vc, ks, vs = oracle.kv_quant(k, k, np.array([3]), cache, cache, 16, k_scale=sc,
                                         v_scale=sc, recalibrate=False)
        assert kc[0, 3, 0, 0] == code
        assert vc[0, 3, 0, 0] == code
        assert ks == np.float32(sc)
    else:
        raise AssertionError(kind)


def test_p1_whole_group():
    vals = [0x4060, 0x3F80, 0xBF00, 0x3E08, 0x3E18, 0x37C0, 0x3700, 0xB700]
    want = [0x7E, 0x70, 0xE8, 0x58, 0x5A, 0x02, 0x00, 0x80]
    g = np.zeros((1, 128), dtype=np.uint16)
    g[0, :8] = vals
    q, s = oracle.quant_act_g128(g)
    assert _f32_bits(s[0, 0]) == 0x3C000000
    assert list(q[0, :8]) == want
    assert np.all(q[0, 8:] == 0)


def test_shortcuts_disagree_where_the_pins_say():
    """P3, P7, P8: rounding fl32(x/s) instead of the exact quotient gives another code."""
    for amax_b, x_b, exact, shortcut in ((0x3DCD, 0x35CD, 0x03, 0x04), (0x4030, 0x3D84, 0x53, 0x52),
                                        (0x3DD0, 0x369C, 0x0B, 0x0A)):
        amax = (np.uint32(amax_b) << 16).view(np.float32)
        x = (np.uint32(x_b) << 16).view(np.float32)
        s = oracle.scale(amax)
        assert oracle.quantize_value(x, s) == exact
        assert oracle.e4m3_encode(float(np.float32(x / s))) == shortcut
