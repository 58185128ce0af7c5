"""Seeded synthetic inputs for the FP8 rollout hot path.

This module generates inputs only: it holds none of the method's arithmetic (no
amax, no scales, no FP8 encoding, no GEMM).  Both the HIP library's callers
(tests, benchmark) and the CPU oracle's callers take their inputs from here, so
the two sides see the same bytes.

Shapes and distributions follow the workloads the pages describe: the dense
model is Qwen3-8B-like (hidden 4096, 8 KV heads of 128, MLP 12288, 36 layers),
the MoE model Qwen3-30B-A3B-like (128 experts, top-8, hidden 2048, expert
intermediate 768, 48 layers), responses of up to 20,000 tokens.  No dataset item
and no trained weight is used: every value is drawn from a seeded generator.

Host generators use numpy's PCG64 seeded with SeedSequence([260118150, cfg,
layer, tensor]); fp32 samples become bf16 by round-to-nearest-even (torch CPU
conversion).  Inputs too large for a host RNG are drawn on the GPU with a seeded
torch generator, and the oracle is given host copies of those exact bytes.
"""
from __future__ import annotations

import numpy as np
import torch

ROOT_SEED = 260118150

# Dense model (Qwen3-8B-like)
HIDDEN = 4096
KV_DIM = 1024           # 8 KV heads x 128
MLP = 12288
LAYERS_DENSE = 36
# MoE model (Qwen3-30B-A3B-like)
MOE_EXPERTS = 128
MOE_TOPK = 8
MOE_HIDDEN = 2048
MOE_INTER = 768
LAYERS_MOE = 48
# KV workload
KV_HEADS = 8
HEAD_DIM = 128
KV_SEQS = 64
KV_SEQ_LEN = 20000
PAGE_SIZE = 16


def rng(cfg: int, layer: int = 0, tensor: int = 0) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([ROOT_SEED, cfg, layer, tensor])))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 (round to nearest even), returned as uint16 bit patterns."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def weight(cfg: int, layer: int, tensor: int, n: int, k: int, std: float = 0.02,
           outlier_frac: float = 1e-3, outlier_mult: float = 20.0,
           zero_block: tuple[int, int] | None = None) -> np.ndarray:
    """bf16 [n, k] ~ N(0, std^2); round(outlier_frac * n * k) entries, drawn without
    replacement, multiplied by outlier_mult; optional all-zero 128x128 block (+0)."""
    g = rng(cfg, layer, tensor)
    w = g.standard_normal((n, k), dtype=np.float32) * np.float32(std)
    cnt = int(round(outlier_frac * n * k))
    if cnt:
        idx = g.choice(n * k, size=cnt, replace=False)
        w.reshape(-1)[idx] *= np.float32(outlier_mult)
    if zero_block is not None:
        bi, bj = zero_block
        w[bi * 128:(bi + 1) * 128, bj * 128:(bj + 1) * 128] = 0.0
    return to_bf16_bits(w)


def activation(cfg: int, layer: int, tensor: int, m: int, k: int, outlier_channels: int = 4,
               outlier_mult: float = 50.0) -> np.ndarray:
    """bf16 [m, k] ~ N(0, 1) with `outlier_channels` seeded columns multiplied by outlier_mult."""
    g = rng(cfg, layer, tensor)
    x = g.standard_normal((m, k), dtype=np.float32)
    if outlier_channels:
        cols = g.choice(k, size=outlier_channels, replace=False)
        x[:, cols] *= np.float32(outlier_mult)
    return to_bf16_bits(x)


def tiny():
    """Config 'tiny': one 256x256 weight with 66 outliers x20 and block (1,1) all
    zero; 16x256 activations ~N(0,1) (no outlier channels)."""
    w = weight(1, 0, 0, 256, 256, zero_block=(1, 1))
    x = activation(1, 0, 1, 16, 256, outlier_channels=0)
    return w, x


# ---------------------------------------------------------------- MoE routing
def moe_topk(layer: int, tokens: int = 4096, experts: int = MOE_EXPERTS, topk: int = MOE_TOPK,
             zipf_s: float = 1.1):
    """Skewed top-k routing as a router would record it: expert e gets popularity rank
    r_e (a seeded permutation of 1..E); logits[t, e] = -s ln(r_e) + Gumbel(0, 1); each
    token takes its top-k logits (ties to the lower expert id), which samples k experts
    without replacement with probability proportional to r_e^-s.  The routing weights
    are the softmax of the k chosen logits.

    Returns (topk_ids int16 [tokens, topk], topk_weights fp32 [tokens, topk])."""
    g = rng(4, layer, 1000)
    rank = g.permutation(experts) + 1
    logits = -zipf_s * np.log(rank.astype(np.float64))[None, :] + g.gumbel(size=(tokens, experts))
    # top-k with ties to the lower id: stable sort on -logit keeps id order for equal keys
    order = np.argsort(-logits, axis=1, kind="stable")[:, :topk]
    chosen = np.take_along_axis(logits, order, axis=1)
    w = np.exp(chosen - chosen.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return order.astype(np.int16), w.astype(np.float32)


def moe_routing(layer: int, tokens: int = 4096, experts: int = MOE_EXPERTS, topk: int = MOE_TOPK,
                zipf_s: float = 1.1):
    """The routing of moe_topk laid out for a grouped GEMM that takes pre-sorted rows
    (rows sorted by expert, stable by token id).

    Returns (row_token [tokens*topk] int64: token feeding each expert-sorted row,
    offsets [experts+1] int32, expert_of_row [tokens*topk] int32)."""
    ids, _ = moe_topk(layer, tokens, experts, topk, zipf_s)
    tok = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    exp = ids.reshape(-1).astype(np.int32)
    perm = np.lexsort((tok, exp))
    row_token = tok[perm]
    expert_of_row = exp[perm]
    counts = np.bincount(exp, minlength=experts)
    offsets = np.zeros(experts + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return row_token, offsets, expert_of_row


# ---------------------------------------------------------------- KV workload
def kv_slot_mapping(cfg: int = 5, layer: int = 0, seqs: int = KV_SEQS, seq_len: int = KV_SEQ_LEN,
                    page_size: int = PAGE_SIZE):
    """Sequence-major tokens; each sequence owns ceil(seq_len/page_size) pages taken
    from a seeded permutation of all page ids.  Returns (slot_mapping int64 [T], pages)."""
    pages_per_seq = -(-seq_len // page_size)
    pages = seqs * pages_per_seq
    g = rng(cfg, layer, 2000)
    table = g.permutation(pages).astype(np.int64).reshape(seqs, pages_per_seq)
    pos = np.arange(seq_len, dtype=np.int64)
    slots = table[:, pos // page_size] * page_size + (pos % page_size)[None, :]
    return slots.reshape(-1), pages


def kv_values(cfg: int, layer: int, tensor: int, tokens: int, heads: int = KV_HEADS,
              head_dim: int = HEAD_DIM, outlier_dims: int = 4, outlier_mult: float = 30.0):
    """bf16 [tokens, heads, head_dim] ~ N(0, 1); per head, `outlier_dims` seeded dims x30."""
    g = rng(cfg, layer, tensor)
    x = g.standard_normal((tokens, heads, head_dim), dtype=np.float32)
    for h in range(heads):
        dims = g.choice(head_dim, size=outlier_dims, replace=False)
        x[:, h, dims] *= np.float32(outlier_mult)
    return to_bf16_bits(x)


# ---------------------------------------------------------------- device-side
def device_generator(device, *key: int) -> torch.Generator:
    seed = ROOT_SEED
    for k in key:
        seed = (seed * 1000003 + int(k)) % (2 ** 63 - 1)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    return gen


def device_normal_bf16(shape, std: float, device, *key: int, outlier_p: float = 0.0,
                       outlier_mult: float = 1.0) -> torch.Tensor:
    """bf16 tensor on `device`, N(0, std^2); each entry independently an outlier
    (x outlier_mult) with probability outlier_p.  Drawn in fp32, rounded once."""
    gen = device_generator(device, *key)
    x = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    x.mul_(std)
    if outlier_p > 0:
        mask = torch.rand(shape, generator=gen, device=device) < outlier_p
        x = torch.where(mask, x * outlier_mult, x)
    return x.to(torch.bfloat16)


def device_activation(m: int, k: int, device, *key: int, outlier_channels: int = 4,
                      outlier_mult: float = 50.0) -> torch.Tensor:
    gen = device_generator(device, *key)
    x = torch.randn((m, k), generator=gen, device=device, dtype=torch.float32)
    if outlier_channels:
        cols = torch.randperm(k, generator=gen, device=device)[:outlier_channels]
        x[:, cols] *= outlier_mult
    return x.to(torch.bfloat16)


def device_kv(tokens: int, device, *key: int, heads: int = KV_HEADS, head_dim: int = HEAD_DIM,
              outlier_dims: int = 4, outlier_mult: float = 30.0) -> torch.Tensor:
    gen = device_generator(device, *key)
    x = torch.randn((tokens, heads, head_dim), generator=gen, device=device, dtype=torch.float32)
    for h in range(heads):
        dims = torch.randperm(head_dim, generator=gen, device=device)[:outlier_dims]
        x[:, h, dims] *= outlier_mult
    return x.to(torch.bfloat16)


def device_fp8_codes(shape, device, *key: int) -> torch.Tensor:
    """uint8 tensor on `device` of finite OCP E4M3FN byte codes, each drawn uniformly
    from the 254 codes other than the two NaN patterns (0x7F, 0xFF)."""
    gen = device_generator(device, *key)
    c = torch.randint(0, 254, shape, generator=gen, device=device, dtype=torch.int16)
    c = c + (c >= 0x7F).to(torch.int16)      # skip 0x7F
    return c.to(torch.uint8)


def device_scales(shape, device, *key: int) -> torch.Tensor:
    """fp32 tensor on `device` of positive scale factors, log-uniform in [2^-12, 2^-4]."""
    gen = device_generator(device, *key)
    u = torch.rand(shape, generator=gen, device=device, dtype=torch.float32)
    return torch.exp2(-12.0 + 8.0 * u)
