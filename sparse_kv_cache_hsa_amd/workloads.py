"""The five synthetic workloads (sizes and data recipes).

They stand in for the pages' long-context evaluations (LongBench, needle in a
haystack, RULER, SCBench with Llama3.1-8B-Instruct) with seeded Gaussian data
of the same shapes: Llama3.1-8B attention layers have 32 query heads, 8 KV
heads and head_dim 128.  Data recipe (all seeded, seed 0 by default):
  - K and V rows ~ N(0,1) in fp32 with 4 fixed outlier channels per
    (layer, KV head) scaled x6 in both K and V;
  - keys and queries of the Llama-shaped workloads are rotary-encoded at their
    true positions (rotate-half, base 500000);
  - queries ~ N(0,1); where a workload plants needles, the needle keys are
    3*sqrt(d) times a seeded unit direction of their (layer, KV head) and the
    queries that should find them get sqrt(d) times that direction added;
  - decode tokens are appended at their true positions (prompt length plus
    step), one per step, sequence and layer;
  - values are rounded to the workload's dtype at the end.
This module draws data only; the split of the compression ratio, eviction and
selection are computed by the library (or by the oracle in tests).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import torch

from . import synth


@dataclass(frozen=True)
class Workload:
    name: str
    dtype: torch.dtype
    layers: int
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    page_size: int
    k1: int
    k2: int
    decode_steps: int
    rope: bool = True
    # stage 1 (SnapKV++) workloads
    prompt_len: int = 0                      # fixed prompt length
    prompt_len_range: tuple = ()             # (lo, hi) inclusive, seeded per sequence
    budget: int = 0                          # total token budget per sequence
    window: int = 32
    pool_kernel: int = 63
    # decode-only workloads (no eviction): the cache as generated
    cache_len: int = 0
    turns: int = 1
    turn_append: int = 0
    # needles
    needle_tokens: int = 0                   # scattered single needle rows
    needle_span: int = 0                     # contiguous needle span length
    queries_align: bool = False              # queries point at the needle
    seed: int = 0
    description: str = field(default="", compare=False)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def evicts(self) -> bool:
        return self.budget > 0

    def prompt_lens(self) -> list[int]:
        if self.prompt_len_range:
            lo, hi = self.prompt_len_range
            g = synth.generator(self.seed, self.name, "prompt_lens")
            return [int(x) for x in torch.randint(lo, hi + 1, (self.batch,), generator=g)]
        if self.prompt_len:
            return [self.prompt_len] * self.batch
        return [self.cache_len] * self.batch

    def compression_ratio(self, L: int) -> float:
        return L / self.budget

    # ---- data ---------------------------------------------------------------
    def _outliers(self, layer):
        return synth.outlier_channels(self.seed, layer, self.n_kv_heads, self.head_dim)

    def needle_direction(self, layer: int, h: int, which: int = 0, device="cpu"):
        return synth.unit_direction(self.seed, self.name, layer, h, which, dim=self.head_dim,
                                    device=device)

    def needle_rows(self, layer: int, seq: int, n: int, which: int = 0) -> list[int]:
        """Positions (< n) that carry needle `which` of (layer, seq)."""
        g = synth.generator(self.seed, self.name, "needle_pos", layer, seq, which)
        if self.needle_span:
            hi = max(1, n - self.window - self.needle_span)
            start = int(torch.randint(0, hi, (1,), generator=g))
            return list(range(start, start + self.needle_span))
        if self.needle_tokens:
            return sorted(int(x) for x in torch.randperm(n, generator=g)[:self.needle_tokens])
        return []

    def _plant(self, k: torch.Tensor, layer: int, rows: list[int], which: int) -> None:
        if not rows:
            return
        idx = torch.tensor(rows, device=k.device)
        for h in range(self.n_kv_heads):
            u = self.needle_direction(layer, h, which, device=k.device)
            k[h, idx, :] = 3.0 * math.sqrt(self.head_dim) * u

    def _align(self, q: torch.Tensor, layer: int, which: int) -> torch.Tensor:
        """q [Hq, ..., d]: adds sqrt(d) * u of the KV head of each query head."""
        if not self.queries_align:
            return q
        for hq in range(self.n_q_heads):
            u = self.needle_direction(layer, hq // self.group, which, device=q.device)
            q[hq] += math.sqrt(self.head_dim) * u
        return q

    def _pos(self, start: int, n: int, device) -> torch.Tensor | None:
        return torch.arange(start, start + n, device=device) if self.rope else None

    def prompt_kv(self, layer: int, seq: int, L: int, device="cpu"):
        """Prompt (or retained cache) rows: k, v [Hkv, L, d] in dtype."""
        o = self._outliers(layer)
        pos = self._pos(0, L, device)
        k = synth.gaussian_rows(self.seed, (self.name, "k", layer, seq), self.n_kv_heads, L,
                                self.head_dim, device=device, outliers=o, positions=pos)
        v = synth.gaussian_rows(self.seed, (self.name, "v", layer, seq), self.n_kv_heads, L,
                                self.head_dim, device=device, outliers=o)
        if self.turns == 1:  # multi-turn needles arrive with each turn's rows
            self._plant(k, layer, self.needle_rows(layer, seq, L, 0), 0)
        return k.to(self.dtype), v.to(self.dtype)

    def window_q(self, layer: int, seq: int, L: int, device="cpu"):
        """Observation-window queries [Hq, w, d] at positions L-w .. L-1."""
        w = self.window
        q = synth.gaussian_rows(self.seed, (self.name, "qwin", layer, seq), self.n_q_heads, w,
                                self.head_dim, device=device, positions=self._pos(L - w, w, device))
        return self._align(q, layer, 0).to(self.dtype)

    def turn_rows(self, layer: int, seq: int, turn: int, start: int, device="cpu"):
        """Rows appended at the start of a turn: k, v [Hkv, turn_append, d] at
        positions start..; needle `turn` is planted at a seeded row among them."""
        n = self.turn_append
        o = self._outliers(layer)
        k = synth.gaussian_rows(self.seed, (self.name, "turn_k", layer, seq, turn),
                                self.n_kv_heads, n, self.head_dim, device=device, outliers=o,
                                positions=self._pos(start, n, device))
        v = synth.gaussian_rows(self.seed, (self.name, "turn_v", layer, seq, turn),
                                self.n_kv_heads, n, self.head_dim, device=device, outliers=o)
        at = self.turn_needle_offset(layer, seq, turn)
        self._plant(k, layer, list(range(at, at + max(1, self.needle_span))), turn)
        return k.to(self.dtype), v.to(self.dtype)

    def turn_window_q(self, layer: int, seq: int, turn: int, end: int, device="cpu"):
        """A turn's last w queries [Hq, w, d] at positions end-w .. end-1,
        aligned with the turn's needle where queries align."""
        w = self.window
        q = synth.gaussian_rows(self.seed, (self.name, "turn_qwin", layer, seq, turn),
                                self.n_q_heads, w, self.head_dim, device=device,
                                positions=self._pos(end - w, w, device))
        return self._align(q, layer, turn).to(self.dtype)

    def turn_needle_offset(self, layer: int, seq: int, turn: int) -> int:
        """Row offset, within a turn's appended rows, of that turn's needle."""
        g = synth.generator(self.seed, self.name, "turn_needle", layer, seq, turn)
        span = max(1, self.needle_span)
        return int(torch.randint(0, max(1, self.turn_append - span), (1,), generator=g))

    def decode_tokens(self, layer: int, step: int, positions: torch.Tensor, turn: int = 0,
                      device="cpu"):
        """One decode step for every sequence of a layer.  positions [B] are the
        tokens' true positions.  Returns k, v [B, Hkv, d] and q [B, Hq, d]."""
        B, d = positions.shape[0], self.head_dim
        o = self._outliers(layer)
        k = synth.randn((self.n_kv_heads, B, d), self.seed, self.name, "tok_k", layer, turn, step,
                        device=device)
        v = synth.randn((self.n_kv_heads, B, d), self.seed, self.name, "tok_v", layer, turn, step,
                        device=device)
        q = synth.randn((self.n_q_heads, B, d), self.seed, self.name, "tok_q", layer, turn, step,
                        device=device)
        synth.apply_outliers(k, o)
        synth.apply_outliers(v, o)
        if self.rope:
            pos = positions.to(device)
            k = synth.rope(k, pos)
            q = synth.rope(q, pos)
        q = self._align(q, layer, turn)
        return (k.transpose(0, 1).contiguous().to(self.dtype),
                v.transpose(0, 1).contiguous().to(self.dtype),
                q.transpose(0, 1).contiguous().to(self.dtype))


TINY = Workload(
    name="tiny-hsa-fp32", dtype=torch.float32, layers=1, batch=1, n_q_heads=8, n_kv_heads=2,
    head_dim=64, page_size=16, k1=16, k2=16, decode_steps=32, rope=False, cache_len=2048,
    needle_tokens=8,
    description="1 layer, batch 1, 2 KV heads x GQA 4, d 64, 2,048 cached tokens, page 16, "
                "k1 16, k2 16, 32 decode steps, 8 needle tokens")

LLAMA_32K = Workload(
    name="llama8b-32k-1layer", dtype=torch.bfloat16, layers=1, batch=1, n_q_heads=32,
    n_kv_heads=8, head_dim=128, page_size=16, k1=32, k2=32, decode_steps=128,
    prompt_len=32768, budget=512,
    description="Llama3.1-8B layer, batch 1, 32,768-token prompt, SnapKV++ (w 32, pool 63, "
                "c 64), 128 HSA steps, page 16, k1 32, k2 32")

EXTREME_109K = Workload(
    name="llama8b-109k-budget256", dtype=torch.bfloat16, layers=1, batch=1, n_q_heads=32,
    n_kv_heads=8, head_dim=128, page_size=8, k1=16, k2=32, decode_steps=256,
    prompt_len=109568, budget=256, needle_span=64, queries_align=True,
    description="Llama3.1-8B layer, batch 1, 109,568 tokens, budget 256 (c ~428), 64-token "
                "needle, page 8, k1 16, k2 32, 256 steps")

BATCHED_32L = Workload(
    name="llama8b-32layer-b32-ctx16k-32k", dtype=torch.bfloat16, layers=32, batch=32,
    n_q_heads=32, n_kv_heads=8, head_dim=128, page_size=16, k1=32, k2=64, decode_steps=64,
    prompt_len_range=(16384, 32768), budget=1024,
    description="all 32 Llama3.1-8B layers, batch 32, contexts 16K-32K, budget 1,024 per "
                "sequence, page 16, k1 32, k2 64, 64 steps")

MT_131K = Workload(
    name="llama8b-mt-131k-b4", dtype=torch.bfloat16, layers=1, batch=4, n_q_heads=32,
    n_kv_heads=8, head_dim=128, page_size=32, k1=32, k2=128, decode_steps=64,
    cache_len=131072, turns=4, turn_append=2048, needle_span=32, queries_align=True,
    description="batch 4, full 131,072-token cache kept, HSA alone (page 32, k1 32, k2 128), "
                "4 turns x (append 2,048 rows + 64 steps)")

ALL = {w.name: w for w in (TINY, LLAMA_32K, EXTREME_109K, BATCHED_32L, MT_131K)}
