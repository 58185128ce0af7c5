"""GPU parity of the block-scaled W8A8 GEMM, dense and grouped, against the fp64 oracle
(FP8-RL summary page, "Method step details" step 1; the output is rounded to bf16
once, per "Where rounding happens matters").  Gate: every element within half a bf16
ulp of the exact value plus 2e-3 of max|y|.  Operands are quantized by the oracle so
the GEMM is tested on its own."""
import numpy as np
import pytest
import torch

import oracle
import fp8_block_scaled_weight_amd as fq
from fp8_block_scaled_weight_amd import synth
from tests._helpers import bf16_bits, gemm_gate

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def quantized_operands(m, n, k, cfg=2, layer=0, tensor=0):
    w = synth.weight(cfg, layer, tensor, n, k)
    x = synth.activation(cfg, layer, tensor + 50, m, k)
    wq, ws = oracle.quant_weight_blk128(w)
    xq, xs = oracle.quant_act_g128(x)
    return xq, xs, wq, ws


def gpu_gemm(xq, xs, wq, ws, ld_y=None):
    m, k = xq.shape
    n = wq.shape[0]
    ld_y = n if ld_y is None else ld_y
    yfull = torch.full((max(m, 1), ld_y), float("nan"), dtype=torch.bfloat16, device=DEV)[:m]
    y = yfull[:, :n]
    fq.fp8q_gemm_w8a8_blkscaled(_dev_u8(xq), _dev_f32(xs), _dev_u8(wq), _dev_f32(ws), y)
    torch.cuda.synchronize()
    return bf16_bits(y), bf16_bits(yfull)


def check(xq, xs, wq, ws, rows=None, ld_y=None, blockwise=False):
    """blockwise: the oracle's full-size form (one float64 product per K block), which
    gives the scalar oracle's numbers bit for bit in seconds at 4096-token shapes."""
    y, yfull = gpu_gemm(xq, xs, wq, ws, ld_y)
    if blockwise:
        ref = oracle.gemm_w8a8_blockwise(xq, xs, wq, ws)
        got = y
    elif rows is None:
        ref = oracle.gemm_w8a8(xq, xs, wq, ws)
        got = y
    else:
        ref = oracle.gemm_w8a8(xq[rows], xs[:, rows], wq, ws)
        got = y[rows]
    ok, ratio, nrm = gemm_gate(got, ref)
    assert ok, f"gate exceeded: worst err/bound {ratio:.3f}, normwise {nrm:.2e}"
    assert nrm < 4e-3
    return yfull


def test_tiny():
    w, x = synth.tiny()
    wq, ws = oracle.quant_weight_blk128(w)
    xq, xs = oracle.quant_act_g128(x)
    check(xq, xs, wq, ws)


@pytest.mark.parametrize("m", [1, 5, 64, 130, 512])
@pytest.mark.parametrize("n", [1024, 4096])
def test_attention_shapes(m, n):
    check(*quantized_operands(m, n, 4096, tensor=n))


@pytest.mark.parametrize("n", [4096, 2048, 1024])
def test_m4096_all_rows(n):
    """4096 tokens, every output: q/o (4096x4096), k and v stacked (2048x4096), k (1024x4096)."""
    check(*quantized_operands(4096, n, 4096, tensor=n + 1), blockwise=True)


@pytest.mark.parametrize("n,k", [(12288, 4096), (4096, 12288)])
def test_mlp_m4096_all_rows(n, k):
    """The dense MLP at 4096 tokens, every output: gate/up (12288x4096, 256x256 tiles over
    32 K steps) and down (4096x12288, 96 K steps)."""
    check(*quantized_operands(4096, n, k, cfg=3, tensor=3 + n // 4096), blockwise=True)


def test_mlp_shapes_sampled():
    g = np.random.Generator(np.random.PCG64(2))
    xq, xs, wq, ws = quantized_operands(64, 12288, 4096, cfg=3)
    check(xq, xs, wq, ws)
    xq, xs, wq, ws = quantized_operands(300, 4096, 12288, cfg=3, tensor=2)
    check(xq, xs, wq, ws, rows=np.sort(g.choice(300, 40, replace=False)))


@pytest.mark.parametrize("m,n,k", [
    (4000, 4096, 1024),   # 256x256 tiles, ragged last token tile
    (2000, 4096, 512),    # 128x128 tiles, two workgroups per CU, ragged
    (1100, 2048, 384),    # 128x128 tiles, four-stage copy ring, ragged
    (1000, 1024, 512),    # 128x64 tiles (m < 1024), ragged
    (700, 1024, 640),     # 128x64 tiles, ragged
    (900, 1024, 1152),    # 128x64 tiles in two K groups, odd K-block count: one group's last step is empty
    (200, 4096, 1024),    # two K groups, four steps each
    (700, 512, 1024),     # few tiles (48 of 128x64): the few-token kernel, 22 tiles of 32 tokens, ragged
    (1000, 512, 4096),    # 64 tiles: the few-token kernel at its largest tile count
    (65536, 384, 256),    # n not a multiple of 256 with enough rows for 256x256 tiles
    (4000, 4096, 128),    # 256x256 tiles, one K step: the only step is also the last
    (4000, 4096, 256),    # 256x256 tiles, two K steps
])
def test_tile_configs_ragged(m, n, k):
    g = np.random.Generator(np.random.PCG64(m + n))
    xq, xs, wq, ws = quantized_operands(m, n, k, tensor=20 + n // 128)
    edges = [0, 1, 127, 128, 255, 256, m - 129, m - 128, m - 2, m - 1]
    rows = np.unique(np.concatenate([np.array([r for r in edges if 0 <= r < m]), g.choice(m, 40, replace=False)]))
    check(xq, xs, wq, ws, rows=rows)


@pytest.mark.parametrize("m,n,k", [
    (64, 512, 1024),      # the last few-token size
    (65, 512, 1024),      # 8 tiles of 128x64: the few-token kernel past 64 tokens
    (65, 8192, 1024),     # 128 tiles: 128x64 tiles in two K groups
    (1023, 512, 1024),    # 64 tiles: still the few-token kernel
    (1024, 512, 1024),    # 128x128 tiles from 1024 tokens
    (300, 512, 896),      # 24 tiles but K < 1024: 128x64 tiles, one K group
    (129, 1024, 1024),    # 32 tiles, a 1-token last tile of 32 tokens
])
def test_dispatch_boundaries(m, n, k):
    """Each side of every size rule that picks a GEMM kernel, sampled rows against the oracle."""
    g = np.random.Generator(np.random.PCG64(m * 7 + n + k))
    xq, xs, wq, ws = quantized_operands(m, n, k, tensor=30 + m % 7)
    edges = [0, 1, 31, 32, 63, 64, 127, 128, m - 2, m - 1]
    rows = np.unique(np.concatenate([np.array([r for r in edges if 0 <= r < m]),
                                     g.choice(m, min(m, 24), replace=False)]))
    check(xq, xs, wq, ws, rows=rows)


@pytest.mark.parametrize("m,n,k", [
    (40, 12288, 1024),    # 64 tokens x 48 weight rows, 256 workgroups, 40 live rows
    (500, 1024, 1024),    # 64 x 32, 256 workgroups, a 52-row last token tile
    (64, 6144, 1024),     # 64 x 32 at exactly 192 workgroups
    (64, 6016, 1024),     # 188 such workgroups: 32 x 32 instead
    (33, 4096, 1024),     # 32 x 32, 256 workgroups, a 1-row last token tile
    (17, 12288, 1024),    # 32 x 48 from 17 tokens
    (320, 1024, 2048),    # 160 workgroups of 64 x 32: 32 x 32
    (16, 12288, 1024),    # 16 tokens: 16 weight rows per workgroup
    (64, 12288, 1024),    # 64 x 48: 256 workgroups, tiles straddling 128-row scale blocks
    (50, 12288, 256),     # 64 x 48, a 50-row token tile
    (64, 9216, 512),      # 64 x 48 at exactly 192 workgroups
    (64, 9600, 512),      # 64 x 48, 200 workgroups
    (64, 6272, 512),      # n not a multiple of 48: 64 x 32
    (20, 12288, 1024),    # 32 x 48
])
def test_few_token_weight_row_pairs(m, n, k):
    """The few-token kernel with 32 or 48 weight rows per workgroup (48-row tiles straddle
    128-row scale blocks), both token heights and each side of the workgroup-count rules:
    every output against the oracle."""
    check(*quantized_operands(m, n, k, tensor=40 + m % 5))


def _random_shapes(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    shapes = []
    while len(shapes) < count:
        m = int(g.choice([g.integers(1, 65), g.integers(65, 1024), g.integers(1024, 5000)]))
        n, k = 128 * int(g.integers(1, 65)), 128 * int(g.integers(1, 41))
        if m * k <= 16 << 20 and n * k <= 16 << 20:
            shapes.append((m, n, k))
    return shapes


@pytest.mark.parametrize("m,n,k", _random_shapes(24, 2024))
def test_random_shapes(m, n, k):
    """Seeded random shapes across every kernel-selection branch (few tokens, few tiles,
    128x64 tiles with one or two K groups, 128x128 and 256x256 tiles), sampled rows
    against the oracle."""
    g = np.random.Generator(np.random.PCG64(m + 3 * n + 7 * k))
    xq, xs, wq, ws = quantized_operands(m, n, k, tensor=40 + (m + n + k) % 9)
    edges = [0, 1, 127, 128, 255, 256, m - 1]
    rows = np.unique(np.concatenate([np.array([r for r in edges if 0 <= r < m]),
                                     g.choice(m, min(m, 16), replace=False)]))
    check(xq, xs, wq, ws, rows=rows)


def test_padded_output_pitch_untouched():
    xq, xs, wq, ws = quantized_operands(40, 256, 384, tensor=9)
    yfull = check(xq, xs, wq, ws, ld_y=264)
    assert np.all(yfull[:, 256:] == 0x7FC0)  # NaN fill beyond n is untouched


def test_zero_scales_and_zero_rows():
    xq, xs, wq, ws = quantized_operands(48, 256, 256, tensor=11)
    xq[3] = 0
    ws[1, 0] = 0.0
    check(xq, xs, wq, ws)


def test_deterministic():
    ops = quantized_operands(256, 1024, 2048, tensor=12)
    a, _ = gpu_gemm(*ops)
    b, _ = gpu_gemm(*ops)
    assert np.array_equal(a, b)


def test_stacked_weights_equal_separate_gemms():
    """k and v stored as one weight (rows stacked, 128-row scale blocks kept apart): the one
    GEMM's column slices equal the two separate GEMMs byte for byte, although the two layouts
    run different tile configurations (4096 x 2048: 512 128x128 tiles on a 2-stage ring, two
    workgroups per CU; 4096 x 1024: 256 tiles on a 4-stage ring).  Sampled rows are also
    checked against the oracle."""
    m, kd, h = 4096, 1024, 4096
    xq, xs, wk, sk = quantized_operands(m, kd, h, tensor=13)
    _, _, wv, sv = quantized_operands(8, kd, h, tensor=14)
    wkv, skv = np.concatenate([wk, wv]), np.concatenate([sk, sv])
    yk, _ = gpu_gemm(xq, xs, wk, sk)
    yv, _ = gpu_gemm(xq, xs, wv, sv)
    ykv, _ = gpu_gemm(xq, xs, wkv, skv)
    assert np.array_equal(ykv[:, :kd], yk) and np.array_equal(ykv[:, kd:], yv)
    rows = np.array([0, 1, 127, 128, 2047, 4095])
    check(xq, xs, wkv, skv, rows=rows)


# ------------------------------------------------------------------------- grouped
def grouped_case(sizes, n, k, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    G = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    m = int(off[-1])
    bq = np.empty((G, n, k), np.uint8)
    bs = np.empty((G, n // 128, k // 128), np.float32)
    for e in range(G):
        bq[e], bs[e] = oracle.quant_weight_blk128(synth.weight(4, 0, e, n, k, outlier_frac=0.0))
    x = synth.to_bf16_bits(g.standard_normal((max(m, 1), k), dtype=np.float32))[:m]
    aq, as_ = oracle.quant_act_g128(x) if m else (np.zeros((0, k), np.uint8), np.zeros((k // 128, 0), np.float32))
    return aq, as_, bq, bs, off


def gpu_grouped(aq, as_, bq, bs, off):
    m, k = aq.shape
    n = bq.shape[1]
    y = torch.full((max(m, 1), n), float("nan"), dtype=torch.bfloat16, device=DEV)[:m]
    fq.fp8q_grouped_gemm_w8a8(_dev_u8(aq), _dev_f32(as_), _dev_u8(bq), _dev_f32(bs),
                              torch.from_numpy(off).to(DEV), y)
    torch.cuda.synchronize()
    return bf16_bits(y)


def check_grouped(case, rows=None):
    aq, as_, bq, bs, off = case
    y = gpu_grouped(*case)
    if rows is None:
        ref = oracle.grouped_gemm_w8a8(aq, as_, bq, bs, off)
        ok, ratio, nrm = gemm_gate(y, ref)
        assert ok, f"worst err/bound {ratio:.3f}"
        return
    for gi in rows:
        r0, r1 = off[gi], off[gi + 1]
        if r1 == r0:
            continue
        ref = oracle.gemm_w8a8(aq[r0:r1], as_[:, r0:r1], bq[gi], bs[gi])
        ok, ratio, nrm = gemm_gate(y[r0:r1], ref)
        assert ok, f"group {gi}: worst err/bound {ratio:.3f}"


def test_grouped_small_with_empty_groups():
    check_grouped(grouped_case([3, 0, 130, 1, 0, 257, 64], 256, 384, 5))


def test_grouped_long_k_large_tiles():
    """K = 2048 with n % 256 == 0 takes the 256x256 tile: empty groups, groups smaller than
    a tile and groups spanning several tiles with ragged ends."""
    check_grouped(grouped_case([3, 0, 300, 1, 0, 513, 64, 256], 512, 2048, 8))


def test_grouped_mixed_tile_heights():
    """K >= 2048 covers a group with 256-row tiles while more than 128 rows are left and a
    remainder of at most 128 rows with one 128-row tile: remainders of 128 (a full short
    tile), 129 and 200 (one 256-row tile), 127, 255 and 1, exact multiples of 256, empty."""
    check_grouped(grouped_case([200, 128, 129, 0, 384, 255, 257, 127, 512, 1], 256, 2048, 11))


def test_grouped_all_empty_but_one():
    check_grouped(grouped_case([0, 0, 200, 0], 128, 256, 6))


def test_grouped_many_groups():
    g = np.random.Generator(np.random.PCG64(7))
    sizes = g.integers(0, 90, size=70)
    check_grouped(grouped_case(list(sizes), 256, 256, 7))


def test_grouped_many_groups_large_tiles():
    """300 experts (five 64-group passes of the tile search), about a third of them empty,
    on the K >= 2048 path of 256- and 128-row tiles."""
    g = np.random.Generator(np.random.PCG64(12))
    sizes = g.integers(0, 30, size=300) * (g.random(300) > 0.33)
    check_grouped(grouped_case(list(sizes), 256, 2048, 12))


def _random_grouped_cases(count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    cases = []
    for c in range(count):
        groups = int(g.integers(1, 41))
        sizes = [int(x) for x in g.integers(0, 300, size=groups) * (g.random(groups) > 0.2)]
        n = int(g.choice([128, 256, 384, 512]))
        k = int(g.choice([128, 256, 768, 1024, 2048, 2560]))
        cases.append((tuple(sizes), n, k, 100 + c))
    return cases


@pytest.mark.parametrize("sizes,n,k,seed", _random_grouped_cases(10, 31))
def test_grouped_random(sizes, n, k, seed):
    """Seeded random expert counts, group sizes (a fifth of them empty), N and K: both tile
    paths (128x128, and 256/128-row tiles for K >= 2048 with N a multiple of 256), every row
    against the oracle."""
    check_grouped(grouped_case(list(sizes), n, k, seed))


def test_grouped_moe_routing_fc2_subset():
    """Zipf-skewed top-8 routing over 128 experts (4096 tokens); fc2 shape n=2048, k=768.
    Checks a subset of groups (smallest, largest, a few others) against the oracle."""
    row_token, off, _ = synth.moe_routing(0)
    sizes = np.diff(off)
    n, k = 2048, 768
    G = 128
    bq = np.empty((G, n, k), np.uint8)
    bs = np.empty((G, n // 128, k // 128), np.float32)
    rng = np.random.Generator(np.random.PCG64(9))
    # expert weights: quantize a few distinct tensors and reuse them to keep the oracle fast
    base = [oracle.quant_weight_blk128(synth.weight(4, 0, e, n, k, outlier_frac=0.0)) for e in range(4)]
    for e in range(G):
        bq[e], bs[e] = base[e % 4]
    x = synth.to_bf16_bits(rng.standard_normal((int(off[-1]), k), dtype=np.float32))
    aq, as_ = oracle.quant_act_g128(x)
    pick = sorted({int(np.argmin(sizes)), int(np.argmax(sizes)), 0, 17, 64, 127})
    check_grouped((aq, as_, bq, bs, off), rows=pick)
