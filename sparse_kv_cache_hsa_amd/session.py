"""A decode session over one workload: allocates the per-layer paged caches
and page summaries, runs the prefill (SnapKV++ eviction, or a plain append
for workloads that keep the whole cache), and runs decode steps -- for every
layer, append the new token's K/V and fold it into the summaries, then HSA
decode.  All compute is librkv; torch supplies memory and the stream.
"""
from __future__ import annotations

import math

import torch

from . import rkv, synth
from .workloads import Workload


class Session:
    """layers: how many layers to hold (the first ones of the model), or
    layer_ids: which of the model's layers (their seeded data) the session's
    layer slots hold."""

    def __init__(self, wl: Workload, extra_rows: int, device="cuda", layers: int | None = None,
                 layer_ids=None):
        self.wl = wl
        self.dev = torch.device(device)
        if layer_ids is None:
            layer_ids = range(wl.layers if layers is None else layers)
        self.layer_ids = [int(x) for x in layer_ids]
        self.n_layers = len(self.layer_ids)
        self.B, self.Hkv, self.G, self.d = wl.batch, wl.n_kv_heads, wl.group, wl.head_dim
        self.Hq, self.P = wl.n_q_heads, wl.page_size
        self.g = rkv.gqa(self.Hkv, self.G, self.d)
        self.scale = synth.head_dim_scale(self.d)
        self.prompt_lens = wl.prompt_lens()
        if wl.evicts:
            self.keep = [rkv.rkv_split_ratio(L / wl.budget, L, wl.window)[3]
                         for L in self.prompt_lens]
        else:
            self.keep = list(self.prompt_lens)
        turn_rows = wl.turns * (wl.turn_append + wl.decode_steps)
        self.capacity = [k + extra_rows + turn_rows for k in self.keep]
        pages = [math.ceil(c / self.P) for c in self.capacity]
        # a multiple of 8 keeps every summary row 16-byte aligned (wide loads)
        self.max_pages = -(-max(pages) // 8) * 8
        table, self.num_blocks = synth.page_table(wl.seed, self.B, pages, self.max_pages)
        self.page_table = table.to(self.dev)
        shape = (self.num_blocks, self.Hkv, self.P, self.d)
        self.caches, self.summ = [], []
        for _ in range(self.n_layers):
            self.caches.append(rkv.PagedCache(torch.zeros(shape, dtype=wl.dtype, device=self.dev),
                                              torch.zeros(shape, dtype=wl.dtype, device=self.dev),
                                              self.page_table))
            self.summ.append(torch.zeros((self.B, self.Hkv, 2, self.d, self.max_pages),
                                         dtype=wl.dtype, device=self.dev))
        self.rows = list(self.keep)  # rows currently in the cache (all layers alike)
        self.ws = rkv.hsa_workspace(self.g, self.B, self.P, self.max_pages, wl.k1, wl.k2,
                                    self.dev)
        self.out = torch.zeros((self.B, self.Hq, self.d), dtype=torch.float32, device=self.dev)
        self.page_idx = [torch.zeros((self.B, self.Hkv, wl.k2), dtype=torch.int32,
                                     device=self.dev) for _ in range(self.n_layers)]
        # execution options of every decode call, per layer (None = automatic)
        self.opts = [None] * self.n_layers

    # ---- prefill -----------------------------------------------------------
    def prompt_batch(self, layer: int):
        """Prompt K/V [B, Hkv, L_max, d] and window queries [B, Hq, w, d]."""
        wl, L_max = self.wl, max(self.prompt_lens)
        k = torch.zeros((self.B, self.Hkv, L_max, self.d), dtype=wl.dtype, device=self.dev)
        v = torch.zeros_like(k)
        qw = torch.zeros((self.B, self.Hq, wl.window, self.d), dtype=wl.dtype, device=self.dev) \
            if wl.evicts else None
        lid = self.layer_ids[layer]
        for b, L in enumerate(self.prompt_lens):
            kb, vb = wl.prompt_kv(lid, b, L, device=self.dev)
            k[b, :, :L] = kb
            v[b, :, :L] = vb
            if qw is not None:
                qw[b] = wl.window_q(lid, b, L, device=self.dev)
        return k, v, qw

    def evict_workspace(self):
        return torch.empty(rkv.rkv_prefill_evict_workspace_bytes(
            self.g, self.B, max(self.prompt_lens), self.wl.window), dtype=torch.uint8,
            device=self.dev)

    def prefill_layer(self, layer: int, ws=None, kept_idx=None, pooled=None, timer=None):
        """Fills layer's cache and summaries from its prompt.  timer, if given,
        is a pair of CUDA events recorded around the library call."""
        k, v, qw = self.prompt_batch(layer)
        if timer:
            timer[0].record()
        if self.wl.evicts:
            rkv.rkv_prefill_evict(self.g, self.prompt_lens, self.keep, qw, k, v,
                                  self.wl.window, self.wl.pool_kernel, self.scale,
                                  self.caches[layer], summaries=self.summ[layer],
                                  kept_idx=kept_idx, pooled_scores=pooled,
                                  ws=ws if ws is not None else self.evict_workspace())
        else:
            n_old = torch.zeros(self.B, dtype=torch.int32, device=self.dev)
            n_new = torch.tensor(self.prompt_lens, dtype=torch.int32, device=self.dev)
            rkv.rkv_append_summaries(self.g, self.caches[layer], n_old, n_new, k.shape[2],
                                     self.summ[layer], k_src=k, v_src=v)
        if timer:
            timer[1].record()
        return k, v, qw

    def turn_source(self, layer: int, turn: int):
        """Multi-turn workloads: the turn's rows k, v [B, Hkv, turn_append, d]
        and the row counts n_old, n_new of the append (device tensors)."""
        n = self.wl.turn_append
        k = torch.zeros((self.B, self.Hkv, n, self.d), dtype=self.wl.dtype, device=self.dev)
        v = torch.zeros_like(k)
        for b in range(self.B):
            k[b], v[b] = self.wl.turn_rows(self.layer_ids[layer], b, turn, self.positions()[b],
                                           device=self.dev)
        n_old = torch.tensor(self.rows, dtype=torch.int32, device=self.dev)
        return k, v, n_old, n_old + n

    def append_source(self, layer: int, src) -> None:
        """Enqueues the append of a turn_source result to layer's cache."""
        k, v, n_old, n_new = src
        rkv.rkv_append_summaries(self.g, self.caches[layer], n_old, n_new, k.shape[2],
                                 self.summ[layer], k_src=k, v_src=v)

    def append_turn(self, layer: int, turn: int):
        """Appends the turn's rows to every sequence of layer (rows are not
        advanced); returns them."""
        src = self.turn_source(layer, turn)
        self.append_source(layer, src)
        return src[0], src[1]

    # ---- multi-turn view (RocketKV-MT) --------------------------------------
    def enable_turn_view(self, keep_rows: int, extra_rows: int):
        """Adds a view cache per layer for the per-turn filter: capacity
        keep_rows + extra_rows, its own shuffled page table and summaries."""
        pages = -(-(keep_rows + extra_rows) // self.P)
        self.view_max_pages = -(-pages // 8) * 8
        table, nblk = synth.page_table(self.wl.seed + 1, self.B, [pages] * self.B,
                                       self.view_max_pages)
        self.view_table = table.to(self.dev)
        shape = (nblk, self.Hkv, self.P, self.d)
        self.views, self.view_summ = [], []
        for _ in range(self.n_layers):
            self.views.append(rkv.PagedCache(torch.zeros(shape, dtype=self.wl.dtype, device=self.dev),
                                             torch.zeros(shape, dtype=self.wl.dtype, device=self.dev),
                                             self.view_table))
            self.view_summ.append(torch.zeros((self.B, self.Hkv, 2, self.d, self.view_max_pages),
                                              dtype=self.wl.dtype, device=self.dev))
        self.view_rows = [0] * self.B
        self.view_ws = rkv.hsa_workspace(self.g, self.B, self.P, self.view_max_pages, self.wl.k1,
                                         self.wl.k2, self.dev)

    def turn_window_q(self, layer: int, turn: int):
        """The turn's last w queries [B, Hq, w, d] (aligned with the turn's
        needle), at the positions of the turn's last w rows."""
        wl = self.wl
        qw = torch.zeros((self.B, self.Hq, wl.window, self.d), dtype=wl.dtype, device=self.dev)
        for b in range(self.B):
            qw[b] = wl.turn_window_q(self.layer_ids[layer], b, turn, self.positions()[b],
                                     device=self.dev)
        return qw

    def turn_view_keep(self, budget: int):
        """Rows of every sequence's view: stage 1's share of a total token
        budget under the adaptive split, at the current history length."""
        return [rkv.rkv_split_ratio(n / budget, n, self.wl.window)[3] if n > budget else n
                for n in self.rows]

    def turn_filter_workspace(self, max_rows: int | None = None):
        """Workspace of turn_filter for histories of up to max_rows rows
        (default: the current ones)."""
        L_max = max(self.rows) if max_rows is None else max_rows
        return torch.empty(rkv.rkv_turn_filter_workspace_bytes(self.g, self.B, L_max,
                                                               self.wl.window),
                           dtype=torch.uint8, device=self.dev)

    def turn_filter(self, layer: int, qw, keep, ws):
        """SnapKV++ over the whole retained history of `layer` into its view
        (enqueue only); keep: rows per sequence."""
        rkv.rkv_turn_filter(self.g, self.rows, keep, qw, self.wl.window, self.wl.pool_kernel,
                            self.scale, self.caches[layer], self.views[layer],
                            view_summaries=self.view_summ[layer], ws=ws)

    def view_step(self, inp):
        """One decode step on the views (every layer): the token is appended
        to the full cache and, with HSA, decoded on the view."""
        per_layer, n_old, n_new, src, view_n = inp
        for l in range(self.n_layers):
            k, v, q = per_layer[l]
            rkv.rkv_append_summaries(self.g, self.caches[l], n_old, n_new, 1, self.summ[l],
                                     k_src=src[l][0], v_src=src[l][1])
            rkv.rkv_decode_step(self.g, q, k, v, self.views[l], view_n, self.view_summ[l],
                                self.wl.k1, self.wl.k2, self.scale, self.out, self.view_ws,
                                page_idx=self.page_idx[l], opts=self.opts[l])

    def make_view_inputs(self, steps: int, turn: int):
        """make_inputs plus the per-step row counts of the views and the new
        rows shaped [B, Hkv, 1, d] for the full cache's append."""
        base = self.make_inputs(steps, turn=turn)
        v0 = torch.tensor(self.view_rows, dtype=torch.int32)
        out = []
        for s, (per_layer, n_old, n_new) in enumerate(base):
            src = [(k[:, :, None].contiguous(), v[:, :, None].contiguous()) for k, v, _ in per_layer]
            out.append((per_layer, n_old, n_new, src, (v0 + s + 1).to(self.dev)))
        return out

    def positions(self):
        """True position of the next token of every sequence."""
        return [L + (r - k) for L, r, k in zip(self.prompt_lens, self.rows, self.keep)]

    # ---- decode ------------------------------------------------------------
    def make_inputs(self, steps: int, turn: int = 0):
        """Per step and layer: new K/V rows [B, Hkv, d], queries [B, Hq, d],
        and the row counts before/after the step."""
        pos0 = torch.tensor(self.positions(), dtype=torch.int64)
        rows0 = torch.tensor(self.rows, dtype=torch.int32)
        inputs = []
        for s in range(steps):
            per_layer = []
            for l in range(self.n_layers):
                k, v, q = self.wl.decode_tokens(self.layer_ids[l], s, pos0 + s, turn=turn,
                                                device=self.dev)
                per_layer.append((k, v, q))
            n_old = (rows0 + s).to(self.dev)
            n_new = (rows0 + s + 1).to(self.dev)
            inputs.append((per_layer, n_old, n_new))
        return inputs

    def step(self, inp):
        """One decode step over every layer (enqueue only): per layer, append
        the token and run HSA decode in one library call."""
        per_layer, _, n_new = inp
        for l in range(self.n_layers):
            k, v, q = per_layer[l]
            rkv.rkv_decode_step(self.g, q, k, v, self.caches[l], n_new, self.summ[l],
                                self.wl.k1, self.wl.k2, self.scale, self.out, self.ws,
                                page_idx=self.page_idx[l], opts=self.opts[l])

    def advance(self, steps: int):
        self.rows = [r + steps for r in self.rows]
