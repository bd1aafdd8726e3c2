"""Seeded synthetic inputs shaped like the linear layers of the 7B/8B/70B
LLMs that the FP8 pages discuss.

This module holds none of the FP8 method's arithmetic: it only draws random
numbers (numpy PCG64 ``default_rng``) and rounds them to the storage dtype.
Both the HIP path and the CPU oracle consume the same bytes made here.

Recipe (distribution parameters are standard deviations):
  * tiny:   X, W [256 x 256] fp32 ~ N(0,1), seed 0, X drawn first then W.
  * mlp8b:  seed 2.  X [4096 x 4096] ~ N(0,1) with round(0.001*K) outlier
            columns (a seeded permutation picks them) multiplied by 50;
            W [14336 x 4096] ~ N(0, 0.02).  bf16.
  * qkv:    seed 3.  X [8192 x 4096] like mlp8b's X; W [6144 x 4096]
            ~ N(0, 0.02).  bf16.
  * mlp70b: seed 4.  X [2048 x 8192] ~ Student-t(df=4), unit scale, not
            renormalised; W [28672 x 8192] ~ N(0, 0.015).  bf16.
  * wgrad:  per step t in 0..19: dY [8192 x 4096] = 1e-3 * Student-t(df=3)
            from seed 500+t, multiplied by 100 at t = 12; X [8192 x 4096]
            ~ N(0,1) from seed 600+t.  bf16.
  * kv:     an 8B-style model's attention K/V of one layer: kv_heads 8,
            head_dim 128, cache capacity 32768 tokens in pages of 16 rows,
            a prefill chunk of 8192 new tokens.  K [tokens x 8*128] ~ N(0,1)
            with 4 fixed channels per head (seeded choice) x 16 and every
            (token, head) vector x a log-uniform gain in [2^-2, 2^2]; V
            ~ N(0,1).  kv_pages: a seeded permutation of the cache's pages
            (a page table) mapping logical row i to a cache row; the new
            tokens are the last 8192 logical rows (a context filled to
            32768).  Seed 11 (K), 12 (V), 13 (pages).  bf16.
  * moe:    a Mixtral-style expert up-projection: 8 experts, hidden 4096,
            ffn 14336, 4096 tokens each routed to its top-2 experts of
            seeded logits N(0,1) + log(p_e), p ~ Dirichlet(2) (uneven
            expert loads).  X [4096 x 4096] like mlp8b's X; the routed rows
            (each token once per chosen expert) are sorted by expert, group
            offsets [9]; W_e [14336 x 4096] ~ N(0, 0.02) from seed 100+e.
            Seed 8.  bf16.
Values are drawn in float32 (Student-t in float64, then float32) and rounded
to bf16 with round-to-nearest-even by torch's CPU cast.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "to_bf16_bits", "bf16_bits_to_f32", "normal", "activation_with_outliers",
    "student_t", "tiny", "mlp8b", "qkv", "mlp70b", "wgrad_step", "dgrad", "kv_keys", "kv_values",
    "kv_pages", "moe_routing", "moe_weight", "CONFIGS",
]

CONFIGS = {
    "tiny": dict(M=256, N=256, K=256),
    "mlp8b": dict(M=4096, N=14336, K=4096),
    "qkv": dict(M=8192, N=6144, K=4096),
    "mlp70b": dict(M=2048, N=28672, K=8192),
    "wgrad": dict(tokens=8192, hidden=4096, steps=20, spike_step=12, spike=100.0),
    "kv": dict(heads=8, head_dim=128, capacity=32768, new_tokens=8192, page=16),
    "moe": dict(tokens=4096, top_k=2, experts=8, N=14336, K=4096),
}


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns (uint16), round-to-nearest-even."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.asarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def normal(rng: np.random.Generator, rows: int, cols: int, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal((rows, cols), dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return x


def activation_with_outliers(rng: np.random.Generator, rows: int, cols: int,
                             frac: float = 0.001, factor: float = 50.0) -> np.ndarray:
    """N(0,1) activations; round(frac*cols) whole columns (at least one) x factor."""
    x = normal(rng, rows, cols)
    n_out = max(1, int(round(frac * cols)))
    cols_idx = rng.permutation(cols)[:n_out]
    x[:, cols_idx] *= np.float32(factor)
    return x


def student_t(rng: np.random.Generator, rows: int, cols: int, df: float,
              scale: float = 1.0) -> np.ndarray:
    x = rng.standard_t(df, size=(rows, cols)).astype(np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return x


# --------------------------------------------------------------- workloads --
def tiny(seed: int = 0):
    rng = np.random.default_rng(seed)
    X = normal(rng, 256, 256)
    W = normal(rng, 256, 256)
    return X, W


def mlp8b(M: int = 4096, N: int = 14336, K: int = 4096, seed: int = 2):
    rng = np.random.default_rng(seed)
    X = to_bf16_bits(activation_with_outliers(rng, M, K))
    W = to_bf16_bits(normal(rng, N, K, 0.02))
    return X, W


def qkv(M: int = 8192, N: int = 6144, K: int = 4096, seed: int = 3):
    rng = np.random.default_rng(seed)
    X = to_bf16_bits(activation_with_outliers(rng, M, K))
    W = to_bf16_bits(normal(rng, N, K, 0.02))
    return X, W


def mlp70b(M: int = 2048, N: int = 28672, K: int = 8192, seed: int = 4):
    rng = np.random.default_rng(seed)
    X = to_bf16_bits(student_t(rng, M, K, 4.0))
    W = to_bf16_bits(normal(rng, N, K, 0.015))
    return X, W


def wgrad_step(t: int, tokens: int = 8192, hidden: int = 4096,
               spike_step: int = 12, spike: float = 100.0):
    """(dY, X) for step t, both bf16 bit patterns of shape [tokens x hidden]."""
    rg = np.random.default_rng(500 + t)
    dy = student_t(rg, tokens, hidden, 3.0, 1e-3)
    if t == spike_step:
        dy *= np.float32(spike)
    rx = np.random.default_rng(600 + t)
    x = normal(rx, tokens, hidden)
    return to_bf16_bits(dy), to_bf16_bits(x)


def dgrad(M: int = 4096, N: int = 14336, K: int = 4096, seed: int = 7):
    """(dY, W) for the data gradient of the 8B-style MLP up-projection
    Y = X W^T: dY [M x N] = 1e-3 * t(3) (the gradient recipe of wgrad_step),
    W [N x K] N(0, 0.02); bf16 bit patterns."""
    rg = np.random.default_rng(seed)
    dy = student_t(rg, M, N, 3.0, 1e-3)
    w = normal(rg, N, K, 0.02)
    return to_bf16_bits(dy), to_bf16_bits(w)


def kv_keys(tokens: int = 8192, heads: int = 8, head_dim: int = 128, seed: int = 11):
    """K vectors [tokens x heads*head_dim], bf16 bits: N(0,1), 4 outlier
    channels per head x 16, a log-uniform per-(token, head) gain in
    [2^-2, 2^2]."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((tokens, heads, head_dim), dtype=np.float32)
    for h in range(heads):
        k[:, h, rng.permutation(head_dim)[:min(4, head_dim)]] *= np.float32(16.0)
    k *= (2.0 ** rng.uniform(-2.0, 2.0, size=(tokens, heads, 1))).astype(np.float32)
    return to_bf16_bits(k.reshape(tokens, heads * head_dim))


def kv_values(tokens: int = 8192, heads: int = 8, head_dim: int = 128, seed: int = 12):
    """V vectors [tokens x heads*head_dim], bf16 bits, N(0,1)."""
    rng = np.random.default_rng(seed)
    return to_bf16_bits(rng.standard_normal((tokens, heads * head_dim), dtype=np.float32))


def kv_pages(capacity: int = 32768, page: int = 16, seed: int = 13):
    """A page table over the cache: row i of the logical sequence lives in
    cache row perm[i // page] * page + i % page (int64 [capacity])."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(capacity // page).astype(np.int64)
    i = np.arange(capacity, dtype=np.int64)
    return perm[i // page] * page + i % page


def moe_routing(tokens: int = 4096, top_k: int = 2, experts: int = 8, K: int = 4096, seed: int = 8):
    """(X_routed bf16 bits [tokens*top_k x K], offsets int64 [experts+1],
    token index of each routed row): every token's top_k experts by seeded
    logits N(0,1) + log(p_e), p ~ Dirichlet(2); routed rows sorted by
    expert (stable in token order)."""
    rng = np.random.default_rng(seed)
    x = activation_with_outliers(rng, tokens, K)
    p = rng.dirichlet(np.full(experts, 2.0))
    logits = rng.standard_normal((tokens, experts)) + np.log(p)[None, :]
    choice = np.argsort(-logits, axis=1, kind="stable")[:, :top_k]        # [tokens, top_k]
    expert = choice.reshape(-1)
    token = np.repeat(np.arange(tokens), top_k)
    order = np.argsort(expert, kind="stable")
    counts = np.bincount(expert, minlength=experts)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    return to_bf16_bits(x[token[order]]), offsets, token[order]


def moe_weight(e: int, N: int = 14336, K: int = 4096):
    """Expert e's weight [N x K], bf16 bits, N(0, 0.02) from seed 100+e."""
    return to_bf16_bits(normal(np.random.default_rng(100 + e), N, K, 0.02))
