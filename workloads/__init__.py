"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module draws random numbers and lays them out; it holds none of the MXFP8
arithmetic (no scale selection, rounding to E4M3 or GEMM).  Inputs are drawn
from numpy's PCG64 ``default_rng(seed)`` in fp32 and rounded to BF16 with
round-to-nearest-even, the precision the learner's linear layers receive
("End-to-End MXFP8 RL on Blackwell" (verl blog), section "The pipeline": BF16
master weights; every decoder linear of Qwen3-8B / Qwen3-30B-A3B is quantized).

Shapes are the Qwen3-8B and Qwen3-30B-A3B decoder-linear shapes the page's
experiments run on (section "Setup"); no dataset is used.
"""
from __future__ import annotations

import numpy as np

# Qwen3-8B decoder linears: hidden 4096, qkv out 6144 (32 q heads + 2x8 kv
# heads of 128), MLP intermediate 12288 (gate_up fused -> 24576), 36 layers.
QWEN3_8B = dict(hidden=4096, qkv=6144, inter=12288, layers=36)
# Qwen3-30B-A3B experts: hidden 2048, expert intermediate 768 (gate_up 1536),
# 128 experts, top-8 routing.
QWEN3_30B_A3B = dict(hidden=2048, expert_inter=768, experts=128, topk=8)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> BF16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + rounding) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal_bf16(rng: np.random.Generator, shape, std: float = 1.0,
                outlier_frac: float = 0.0, outlier_mult: float = 20.0) -> np.ndarray:
    """N(0, std^2) in fp32; optionally an element-wise Bernoulli(outlier_frac)
    mask multiplies entries by outlier_mult (activation outliers); then BF16."""
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if outlier_frac > 0.0:
        mask = rng.random(size=shape, dtype=np.float32) < outlier_frac
        x[mask] *= np.float32(outlier_mult)
    return f32_to_bf16_bits(x)


# ---------------------------------------------------------------- configs

def tiny(seed: int = 0):
    """W[256x256] ~ N(0, 0.02^2), X[64x256] ~ N(0, 1)."""
    rng = np.random.default_rng(seed)
    W = normal_bf16(rng, (256, 256), std=0.02)
    X = normal_bf16(rng, (64, 256))
    return dict(W=W, X=X)


def qkv(seed: int = 0, tokens: int = 4096):
    """Qwen3-8B qkv_proj: W[6144x4096] ~ N(0, 0.02^2); X[tokens x 4096] ~ N(0,1)
    with 1% of entries multiplied by 20."""
    rng = np.random.default_rng(seed)
    W = normal_bf16(rng, (QWEN3_8B["qkv"], QWEN3_8B["hidden"]), std=0.02)
    X = normal_bf16(rng, (tokens, QWEN3_8B["hidden"]), outlier_frac=0.01)
    return dict(W=W, X=X)


def mlp(seed: int = 0, tokens: int = 8192):
    """Qwen3-8B MLP training micro-batch of `tokens` (multiple of 32):
    W_gu[24576x4096], W_d[4096x12288] ~ N(0, 0.02^2); X[tokens x 4096] and
    h[tokens x 12288] ~ N(0,1) with 1% x20 outliers; dY_gu[tokens x 24576] and
    dY_d[tokens x 4096] ~ N(0,1) * 2^-10 (small gradients)."""
    assert tokens % 32 == 0
    H, I = QWEN3_8B["hidden"], QWEN3_8B["inter"]
    rng = np.random.default_rng(seed)
    return dict(
        W_gu=normal_bf16(rng, (2 * I, H), std=0.02),
        W_d=normal_bf16(rng, (H, I), std=0.02),
        X=normal_bf16(rng, (tokens, H), outlier_frac=0.01),
        h=normal_bf16(rng, (tokens, I), outlier_frac=0.01),
        dY_gu=normal_bf16(rng, (tokens, 2 * I), std=2.0 ** -10),
        dY_d=normal_bf16(rng, (tokens, H), std=2.0 ** -10),
    )


def zipf_topk_routing(rng: np.random.Generator, tokens: int, experts: int,
                      topk: int, s: float = 1.1) -> np.ndarray:
    """Expert popularity p_i proportional to i^-s (i = 1..experts); each token
    draws `topk` distinct experts by Gumbel-top-k.  Returns int32 [tokens, topk]."""
    logp = -s * np.log(np.arange(1, experts + 1, dtype=np.float64))
    g = rng.gumbel(size=(tokens, experts))
    keys = logp[None, :] + g
    top = np.argpartition(-keys, topk - 1, axis=1)[:, :topk]
    return top.astype(np.int32)


def group_layout(route: np.ndarray, experts: int, pad: int = 32):
    """Rows sorted stably by (expert, token); each expert's group padded with
    zero rows to a multiple of `pad`.  Returns (offsets int32 [G+1], row_token
    int64 [M_total] with -1 for padding rows, counts int64 [G])."""
    tokens, topk = route.shape
    flat_e = route.reshape(-1).astype(np.int64)
    flat_t = np.repeat(np.arange(tokens, dtype=np.int64), topk)
    order = np.lexsort((flat_t, flat_e))
    flat_e, flat_t = flat_e[order], flat_t[order]
    counts = np.bincount(flat_e, minlength=experts).astype(np.int64)
    padded = (counts + pad - 1) // pad * pad
    offsets = np.zeros(experts + 1, np.int64)
    offsets[1:] = np.cumsum(padded)
    row_token = np.full(int(offsets[-1]), -1, np.int64)
    start = np.zeros(experts + 1, np.int64)
    start[1:] = np.cumsum(counts)
    for g in range(experts):
        n = counts[g]
        row_token[offsets[g]:offsets[g] + n] = flat_t[start[g]:start[g] + n]
    return offsets.astype(np.int32), row_token, counts


def moe(seed: int = 0, tokens: int = 8192, experts: int | None = None,
        hidden: int | None = None, inter: int | None = None, topk: int | None = None):
    """Qwen3-30B-A3B MoE layer: per expert gate_up [2*inter x hidden] and down
    [hidden x inter] ~ N(0, 0.02^2); X[tokens x hidden] ~ N(0,1); Zipf(1.1)
    top-k routing; rows gathered per expert and padded to 32 with zero rows.
    The down-projection input (the activation of the gate_up output) is drawn
    as N(0,1) per real row, zero on padding rows."""
    cfg = QWEN3_30B_A3B
    E = experts or cfg["experts"]
    H = hidden or cfg["hidden"]
    I = inter or cfg["expert_inter"]
    k = topk or cfg["topk"]
    rng = np.random.default_rng(seed)
    W_gu = normal_bf16(rng, (E, 2 * I, H), std=0.02)
    W_d = normal_bf16(rng, (E, H, I), std=0.02)
    X = normal_bf16(rng, (tokens, H))
    route = zipf_topk_routing(rng, tokens, E, k)
    offsets, row_token, counts = group_layout(route, E)
    real = row_token >= 0
    A_gu = np.zeros((row_token.size, H), np.uint16)
    A_gu[real] = X[row_token[real]]
    A_d = np.zeros((row_token.size, I), np.uint16)
    A_d[real] = normal_bf16(rng, (int(real.sum()), I))
    return dict(W_gu=W_gu, W_d=W_d, X=X, route=route, offsets=offsets,
                row_token=row_token, counts=counts, A_gu=A_gu, A_d=A_d)


def sync_layer_shapes():
    """(name, N, K) of the four quantized linears of one Qwen3-8B decoder
    layer, as the weight synchronization quantizes them."""
    H, Q, I = QWEN3_8B["hidden"], QWEN3_8B["qkv"], QWEN3_8B["inter"]
    return [("qkv", Q, H), ("o", H, H), ("gate_up", 2 * I, H), ("down", H, I)]


def torch_normal_bf16(shape, std: float, seed: int, device):
    """Device-side draw for the multi-GB weight-sync workload: torch's
    Philox generator seeded with `seed`, N(0, std^2) in fp32, rounded to BF16.
    (Too large to draw on the host in a benchmark; a host copy of any sample
    can be taken for checking.)"""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(0.0, std, generator=g)
    return x.to(torch.bfloat16)
