"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  This module only draws and shapes data (Gaussian rows, outlier
channels, rotary position encoding, planted needles, page-table layouts); it
holds none of the decode method's arithmetic.

Every tensor comes from its own torch generator whose seed is a hash of
(seed, key...), so any piece can be regenerated independently.  Draws happen
in fp32 on the requested device (torch's CPU and GPU generators give
different streams for the same seed: inputs are generated once and copied
wherever they are needed) and are rounded to the target dtype at the end.
"""
from __future__ import annotations

import hashlib
import math

import torch

ROPE_THETA = 500000.0
OUTLIER_CHANNELS = 4
OUTLIER_SCALE = 6.0


def sub_seed(seed: int, *key) -> int:
    h = hashlib.sha256(repr((int(seed),) + tuple(key)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def generator(seed: int, *key, device="cpu") -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(sub_seed(seed, *key))
    return g


def randn(shape, seed: int, *key, device="cpu") -> torch.Tensor:
    return torch.randn(shape, generator=generator(seed, *key, device=device), device=device,
                       dtype=torch.float32)


def outlier_channels(seed: int, layer: int, n_kv_heads: int, head_dim: int) -> torch.Tensor:
    """[Hkv, 4] distinct channel ids per (layer, KV head), on the CPU."""
    g = generator(seed, "outliers", layer)
    return torch.stack([torch.randperm(head_dim, generator=g)[:OUTLIER_CHANNELS]
                        for _ in range(n_kv_heads)])


def unit_direction(seed: int, *key, dim: int, device="cpu") -> torch.Tensor:
    v = randn((dim,), seed, "direction", *key, device=device)
    return v / v.norm()


def apply_outliers(x: torch.Tensor, channels: torch.Tensor) -> torch.Tensor:
    """x [Hkv, ..., d]: multiplies each head's outlier channels by 6 in place."""
    for h in range(x.shape[0]):
        x[h, ..., channels[h].to(x.device)] *= OUTLIER_SCALE
    return x


def rope(x: torch.Tensor, positions: torch.Tensor) -> torch.Tensor:
    """Rotate-half rotary encoding, base 500000, no frequency scaling.
    x [..., n, d] fp32; positions [n] (broadcast over leading dims)."""
    d = x.shape[-1]
    half = d // 2
    inv = ROPE_THETA ** (-torch.arange(0, half, dtype=torch.float64, device=x.device) * 2.0 / d)
    ang = positions.to(device=x.device, dtype=torch.float64)[:, None] * inv[None, :]
    cos, sin = torch.cos(ang).to(torch.float32), torch.sin(ang).to(torch.float32)
    x1, x2 = x[..., :half], x[..., half:]
    return torch.cat([x1 * cos - x2 * sin, x2 * cos + x1 * sin], dim=-1)


def gaussian_rows(seed: int, key: tuple, n_heads: int, n: int, d: int, *, device="cpu",
                  outliers: torch.Tensor | None = None,
                  positions: torch.Tensor | None = None) -> torch.Tensor:
    """[n_heads, n, d] fp32 N(0,1) rows, outlier channels x6, RoPE'd when
    positions are given."""
    x = randn((n_heads, n, d), seed, *key, device=device)
    if outliers is not None:
        apply_outliers(x, outliers)
    if positions is not None:
        x = rope(x, positions)
    return x


def page_table(seed: int, n_seqs: int, pages_per_seq, max_pages: int, *, shuffle: bool = True):
    """Seeded block layout: sequence b owns pages_per_seq[b] physical blocks
    (a random permutation of the pool when shuffle), unused entries -1.
    Returns (table [B, max_pages] int32 on the CPU, number of blocks)."""
    counts = [int(c) for c in pages_per_seq]
    total = sum(counts)
    perm = torch.randperm(total, generator=generator(seed, "blocks")) if shuffle \
        else torch.arange(total)
    table = torch.full((n_seqs, max_pages), -1, dtype=torch.int32)
    at = 0
    for b, c in enumerate(counts):
        assert c <= max_pages
        table[b, :c] = perm[at:at + c].to(torch.int32)
        at += c
    return table, max(total, 1)


def to_bits(x: torch.Tensor):
    """Host numpy view for the oracle: fp32 as float32, bf16 as uint16 bits."""
    import numpy as np
    x = x.detach().cpu().contiguous()
    if x.dtype == torch.bfloat16:
        return x.view(torch.int16).numpy().view(np.uint16)
    if x.dtype == torch.float32:
        return x.numpy()
    raise TypeError(x.dtype)


def head_dim_scale(d: int) -> float:
    """fp32 value of 1/sqrt(d), the logit scale used everywhere."""
    return float(torch.tensor(1.0 / math.sqrt(d), dtype=torch.float32))
