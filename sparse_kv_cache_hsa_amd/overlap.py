"""Selection quality of HSA against exact top-k at a matched token budget.

The RocketKV pages compare hybrid sparse attention with one-dimensional
reductions ("RocketKV-adapted -- Two-Stage Compression", "Where it sits":
SparQ-style channel selection along the head dimension, Quest-style page
summaries along the sequence dimension).  This measurement runs the four
selections as parameterisations of the same library calls on a workload's
real cache after stage-1 eviction:

  hsa    : page P, k1 channels, k2 pages           (the configured method)
  quest  : page P, every channel (k1 = d), k2 pages
  sparq  : page 1, k1 channels, k2 * P tokens
  exact  : page 1, every channel, k2 * P tokens    (exact top-k of sum_j q_j.k)

and reports, per method, the token recall against `exact` and the share of
the true softmax mass (per query head, averaged) that its tokens carry.
Selections come from librkv; only the reference softmax mass is computed
with plain torch, as a measurement.

  python -m sparse_kv_cache_hsa_amd.overlap --workload llama8b-32k-1layer --steps 16
"""
from __future__ import annotations

import argparse
import json
import sys

import torch

from . import rkv, workloads
from .session import Session


def logical_rows(sess: Session, layer: int, b: int, n: int):
    """K, V rows [Hkv, n, d] of sequence b from the paged cache."""
    P = sess.P
    r = torch.arange(n, device=sess.dev)
    blk = sess.page_table[b, r // P].long()
    c = sess.caches[layer]
    k = c.k_pool[blk, :, r % P].transpose(0, 1)
    v = c.v_pool[blk, :, r % P].transpose(0, 1)
    return k, v


def measure(wl: workloads.Workload, steps: int, device="cuda") -> dict:
    rkv.load_library()
    sess = Session(wl, extra_rows=steps, device=device, layers=1)
    sess.prefill_layer(0)
    B, Hkv, G, d, P = sess.B, sess.Hkv, sess.G, sess.d, sess.P
    budget = wl.k2 * P
    if budget > rkv.RKV_MAX_K2:
        raise SystemExit(f"token budget {budget} exceeds the library's k2 limit of "
                         f"{rkv.RKV_MAX_K2}")
    g = sess.g
    # page-1 copy of the same logical rows (identity page table)
    cap = max(sess.capacity)
    flat_table = (torch.arange(B * cap, dtype=torch.int32, device=device).view(B, cap))
    fk = torch.zeros((B * cap, Hkv, 1, d), dtype=wl.dtype, device=device)
    fv = torch.zeros_like(fk)
    flat = rkv.PagedCache(fk, fv, flat_table)
    fsumm = torch.zeros((B, Hkv, 2, d, cap), dtype=wl.dtype, device=device)
    n0 = list(sess.rows)
    ksrc = torch.zeros((B, Hkv, max(n0), d), dtype=wl.dtype, device=device)
    vsrc = torch.zeros_like(ksrc)
    for b in range(B):
        ksrc[b, :, :n0[b]], vsrc[b, :, :n0[b]] = logical_rows(sess, 0, b, n0[b])
    zeros = torch.zeros(B, dtype=torch.int32, device=device)
    rkv.rkv_append_summaries(g, flat, zeros, torch.tensor(n0, dtype=torch.int32, device=device),
                             max(n0), fsumm, k_src=ksrc, v_src=vsrc)
    del ksrc, vsrc
    ws_p = rkv.hsa_workspace(g, B, P, sess.max_pages, d, wl.k2, device)
    ws_f = rkv.hsa_workspace(g, B, 1, cap, d, budget, device)
    sel = {m: torch.zeros((B, Hkv, wl.k2 if m in ("hsa", "quest") else budget),
                          dtype=torch.int32, device=device) for m in ("hsa", "quest", "sparq", "exact")}
    stats = {m: {"recall": [], "mass": []} for m in sel}
    inputs = sess.make_inputs(steps)
    for s in range(steps):
        per_layer, n_old, n_new = inputs[s]
        kt, vt, qt = per_layer[0]
        rkv.rkv_decode_step(g, qt, kt, vt, sess.caches[0], n_new, sess.summ[0], wl.k1, wl.k2,
                            sess.scale, sess.out, sess.ws, page_idx=sel["hsa"])
        rkv.rkv_append_summaries(g, flat, n_old, n_new, 1, fsumm, k_src=kt[:, :, None].contiguous(),
                                 v_src=vt[:, :, None].contiguous())
        rkv.rkv_hsa_select(g, qt, n_new, P, sess.summ[0], d, wl.k2, sel["quest"], ws_p)
        rkv.rkv_hsa_select(g, qt, n_new, 1, fsumm, wl.k1, budget, sel["sparq"], ws_f)
        rkv.rkv_hsa_select(g, qt, n_new, 1, fsumm, d, budget, sel["exact"], ws_f)
        torch.cuda.synchronize()
        n = n_new.cpu().tolist()
        for b in range(B):
            tok = {}
            for m, t in sel.items():
                idx = t[b].long()
                if m in ("hsa", "quest"):  # pages -> their valid rows
                    rows = (idx[..., None] * P + torch.arange(P, device=device)).view(Hkv, -1)
                    ok = (idx[..., None] >= 0).expand(-1, -1, P).reshape(Hkv, -1) & (rows < n[b])
                else:
                    rows, ok = idx, idx >= 0
                # invalid entries (padding, rows past the end of a partial
                # last page) all go to a spare column n, so every write is in
                # bounds and no invalid entry can clear a selected row
                tok[m] = torch.where(ok & (rows >= 0) & (rows < n[b]), rows,
                                     torch.full_like(rows, n[b]))
            for m, rows in tok.items():
                lo, hi = int(rows.min()), int(rows.max())
                assert 0 <= lo and hi <= n[b], (m, lo, hi, n[b])
            k, _ = logical_rows(sess, 0, b, n[b])
            q = qt[b].float().view(Hkv, G, d)
            kT = k.float().transpose(1, 2).contiguous()
            p = torch.softmax(torch.matmul(q, kT) * sess.scale, dim=-1)

            def to_mask(rows):
                mk = torch.zeros((Hkv, n[b] + 1), dtype=torch.bool, device=device)
                mk.scatter_(1, rows, True)
                return mk[:, :n[b]]

            ex_mask = to_mask(tok["exact"])
            for m, rows in tok.items():
                mask = to_mask(rows)
                stats[m]["recall"].append(((mask & ex_mask).sum(1).float() /
                                           ex_mask.sum(1).clamp(min=1).float()).mean().item())
                stats[m]["mass"].append((p * mask[:, None, :]).sum(-1).mean().item())
    out = {"workload": wl.name, "steps": steps, "sequences": B, "kv_heads": Hkv,
           "budget_tokens": budget, "page_size": P, "k1": wl.k1, "k2": wl.k2,
           "cache_rows": [int(x) for x in n0]}
    for m, st in stats.items():
        r, ms = torch.tensor(st["recall"]), torch.tensor(st["mass"])
        out[m] = {"recall_vs_exact_mean": round(r.mean().item(), 4),
                  "recall_vs_exact_min": round(r.min().item(), 4),
                  "attention_mass_mean": round(ms.mean().item(), 4),
                  "attention_mass_min": round(ms.min().item(), 4)}
    return out


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default=workloads.LLAMA_32K.name)
    ap.add_argument("--steps", type=int, default=16)
    a = ap.parse_args(argv)
    res = measure(workloads.ALL[a.workload], a.steps)
    json.dump(res, sys.stdout)
    print()


if __name__ == "__main__":
    main()
