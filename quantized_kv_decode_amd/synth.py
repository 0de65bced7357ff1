"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle's callers.

This module draws random numbers and nothing else: it holds none of the quantization,
packing, masking or attention arithmetic. Both the HIP path and the fp64 oracle receive
the tensors it returns, so neither side can influence the other's inputs.

The shapes and distributions stand in for the serving workloads of the LoopKV paper
("Loop-Aware KV Cache Compression for Serving Looped Transformers"): Ouro-1.4B has 24
layers, 4 loops and 16 KV heads of dimension 128 without grouped-query attention (§2.1),
Ouro-2.6B has 48 layers (Appendix, "Ouro-2.6B, served"). No model weights or dataset
items are used; keys, values and queries are Gaussian, with a few outlier key channels
per (cell, head) scaled up, the structure KIVI's per-channel key quantization targets.
"""
from __future__ import annotations

import numpy as np
import torch

REUSE, INT2, INT4 = 0, 2, 4


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def outlier_channels(seed: int, num_heads: int, head_dim: int, count: int = 4) -> np.ndarray:
    """Per head, `count` distinct channels drawn uniformly without replacement."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.choice(head_dim, size=count, replace=False) for _ in range(num_heads)])


def keys(batch: int, tokens: int, heads: int, head_dim: int, seed: int, *, device="cpu",
         outliers: int = 4, outlier_scale: float = 10.0, heavy_tail: bool = False,
         token_offset: int = 0, total_tokens: int | None = None) -> torch.Tensor:
    """bf16 keys [batch, tokens, heads, head_dim]: N(0,1), with `outliers` channels per head
    scaled by `outlier_scale`. With `heavy_tail`, those channels are Student-t(3) draws
    (Z / sqrt(chi2_3 / 3)) times the scale instead of Gaussian ones.

    The outlier channels depend only on `seed`, so a cache generated in token chunks
    (`token_offset`) keeps the same channels; each chunk draws from its own sub-seed.
    """
    g = _gen(seed * 1000003 + token_offset, device)
    x = torch.randn(batch, tokens, heads, head_dim, generator=g, device=device, dtype=torch.float32)
    ch = torch.as_tensor(outlier_channels(seed, heads, head_dim, outliers), device=device)
    if heavy_tail:
        z = torch.randn(batch, tokens, heads, outliers, generator=g, device=device)
        chi = torch.randn(batch, tokens, heads, outliers, 3, generator=g, device=device).pow(2).sum(-1)
        t3 = z / torch.sqrt(chi / 3.0)
        vals = t3 * outlier_scale
    else:
        vals = torch.gather(x, 3, ch.view(1, 1, heads, outliers).expand(batch, tokens, heads, outliers))
        vals = vals * outlier_scale
    x.scatter_(3, ch.view(1, 1, heads, outliers).expand(batch, tokens, heads, outliers), vals)
    return x.to(torch.bfloat16)


def values(batch: int, tokens: int, heads: int, head_dim: int, seed: int, *, device="cpu",
           token_offset: int = 0) -> torch.Tensor:
    """bf16 values [batch, tokens, heads, head_dim], N(0,1)."""
    g = _gen(seed * 1000033 + 7 + token_offset, device)
    return torch.randn(batch, tokens, heads, head_dim, generator=g, device=device).to(torch.bfloat16)


def queries(batch: int, heads: int, head_dim: int, seed: int, *, device="cpu") -> torch.Tensor:
    """bf16 decode queries [batch, heads, head_dim], N(0,1)."""
    g = _gen(seed * 1000037 + 11, device)
    return torch.randn(batch, heads, head_dim, generator=g, device=device).to(torch.bfloat16)


def seeds(batch: int, heads: int, seed: int, scale: float = 2.0) -> torch.Tensor:
    """fp32 running-max seeds [batch, heads] (score units), N(0, scale^2)."""
    g = _gen(seed * 1000039 + 13, "cpu")
    return torch.randn(batch, heads, generator=g) * scale


def plan(num_layers: int, num_loops: int, seed: int, p_int4: float, p_reuse: float = 0.25) -> np.ndarray:
    """uint8 plan [num_loops, num_layers] with codes REUSE=0 / INT2=2 / INT4=4.

    round(p_reuse * cells) cells reuse the final loop's KV, drawn uniformly among loops
    before the final one; round(p_int4 * cells) of the rest are INT4; the others INT2.
    """
    rng = np.random.default_rng(seed)
    cells = num_layers * num_loops
    p = np.full((num_loops, num_layers), INT2, dtype=np.uint8)
    early = np.arange((num_loops - 1) * num_layers)
    n_reuse = int(round(p_reuse * cells))
    reuse = rng.choice(early, size=n_reuse, replace=False)
    p.reshape(-1)[reuse] = REUSE
    rest = np.setdiff1d(np.arange(cells), reuse)
    n4 = int(round(p_int4 * cells))
    p.reshape(-1)[rng.choice(rest, size=n4, replace=False)] = INT4
    return p


def named_plan(name: str, num_layers: int, num_loops: int) -> np.ndarray:
    """The paper's fixed plans by name (uint8 [num_loops, num_layers], final loop never REUSE):
    "kivi4" every cell INT4; "kivi4_loop3_share" loop 3 reuses the final loop's KV;
    "int2_loops123" INT2 before the final loop; "loopkv_r" 25 of the 72 cells before the final
    loop INT2, taken in loop-major order from the first and last 6 layers; "loopkv_m" the first
    26 of those 72 cells (loop-major) reuse the final loop, the next 20 are INT2."""
    p = np.full((num_loops, num_layers), INT4, dtype=np.uint8)
    early = [(t, l) for t in range(num_loops - 1) for l in range(num_layers)]
    if name == "kivi4":
        pass
    elif name == "kivi4_loop3_share":
        p[num_loops - 2, :] = REUSE
    elif name == "int2_loops123":
        p[:num_loops - 1, :] = INT2
    elif name == "loopkv_r":
        edge = list(range(6)) + list(range(num_layers - 6, num_layers))
        cells = [(t, l) for t in range(num_loops - 1) for l in edge]
        for t, l in cells[:25]:
            p[t, l] = INT2
    elif name == "loopkv_m":
        for t, l in early[:26]:
            p[t, l] = REUSE
        for t, l in early[26:46]:
            p[t, l] = INT2
    else:
        raise ValueError(f"unknown plan {name!r}")
    return p


def lengths(batch: int, lo: int, hi: int, seed: int) -> np.ndarray:
    """int32 per-request context lengths, uniform on [lo, hi]."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=batch).astype(np.int32)


def page_table(lens_tokens, page_tokens: int, seed: int, stride: int | None = None,
               shuffle: bool = True) -> tuple[np.ndarray, int]:
    """A page table [batch, stride] (int32) giving each request ceil(len / page_tokens)
    distinct physical pages, drawn from one pool in shuffled (or sequential) order.
    Unused entries are -1. Returns (table, num_pages)."""
    lens_tokens = np.asarray(lens_tokens, dtype=np.int64)
    npages = (lens_tokens + page_tokens - 1) // page_tokens
    total = int(npages.sum())
    ids = np.arange(total, dtype=np.int32)
    if shuffle:
        np.random.default_rng(seed).shuffle(ids)
    if stride is None:
        stride = int(npages.max()) if len(npages) else 1
    tab = np.full((len(lens_tokens), max(stride, 1)), -1, dtype=np.int32)
    pos = 0
    for b, n in enumerate(npages):
        tab[b, :n] = ids[pos:pos + n]
        pos += n
    return tab, total


def damage_table(num_layers: int, num_loops: int, seed: int) -> np.ndarray:
    """A synthetic per-cell damage profile, float64 [num_loops, num_layers, 3] for the options
    (INT4, INT2, REUSE), shaped like the properties the paper reports for Ouro: a few middle
    layers are far more sensitive than the rest; 2-bit codes cost about an order of magnitude
    more than 4-bit ones; reusing the final loop's KV is expensive in the first loop and cheap
    in the late loops (often cheaper than 2-bit codes in the loop before the last). The final
    loop's REUSE entry is NaN (it has nothing to reuse). Lognormal noise, seeded."""
    rng = np.random.default_rng(seed)
    L, T = num_layers, num_loops
    pos = (np.arange(L) + 0.5) / L
    sens = 1.0 + 9.0 * np.exp(-((pos - 0.5) / 0.12) ** 2)          # sensitive middle layers
    sens *= np.exp(rng.normal(0, 0.4, size=L))
    d = np.empty((T, L, 3))
    for t in range(T):
        loop_w = np.exp(rng.normal(0, 0.2, size=L)) * (1.3 if t == 0 else 1.0)
        d[t, :, 0] = 0.004 * sens * loop_w * np.exp(rng.normal(0, 0.3, size=L))
        d[t, :, 1] = d[t, :, 0] * 10.0 * np.exp(rng.normal(0, 0.4, size=L))
        frac = t / max(T - 1, 1)                                      # 0 first loop .. 1 final
        share = 3.0 * (1.0 - frac) ** 2 + 0.25
        d[t, :, 2] = d[t, :, 1] * share * np.exp(rng.normal(0, 0.5, size=L))
    d[T - 1, :, 2] = np.nan
    return d
