"""Parity at the workloads' full sizes, on every unit and every decode step.

Each test drives the library through the C ABI exactly as the benchmark's
session does (same cache layout, same launch shapes) and checks every
(sequence, KV head) unit against the oracle, which gets its inputs from the
seeded generator only:
  - the split ratio and keep counts (exact integers);
  - SnapKV++ kept sets: bit-exact, except boundary swaps whose oracle score
    gap is under 1e-6 relative, which are counted and reported;
  - at every decode step: the channel set, the page set (bit-exact) and the
    attention output (within OUT_ATOL);
  - the page summaries after the last step (bit-exact).
When a unit's kept set differs by an accepted near-tie swap, the library's
cache for that sequence is rewritten with the oracle's kept rows (through
rkv_append_summaries), so both sides decode over the same cache and no unit
drops out of the decode checks.  The oracle's calls, which are independent
per unit, run on a pool of host threads (the oracle is C and releases the
interpreter lock); each unit's arithmetic is unchanged.

Near-tie swap counts, the units they touched and needle recall are written
to gpurun_out/parity/<workload>.json under the repository root.
"""
from __future__ import annotations

import concurrent.futures as cf
import json
import os

import numpy as np
import pytest
import torch

import oracle
from _helpers import OUT_ATOL, bits, check_kept, gpu_summaries, lib, max_abs_err, n_pages
from sparse_kv_cache_hsa_amd import workloads
from sparse_kv_cache_hsa_amd.session import Session

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
THREADS = max(1, min(16, len(os.sched_getaffinity(0))))
_POOL = cf.ThreadPoolExecutor(THREADS)


def say(*a):
    """Progress: printed, and appended to gpurun_out/parity/progress.log so
    that a run whose output pytest captures still shows it is alive."""
    print(*a, flush=True)
    d = os.path.join(ROOT, "gpurun_out", "parity")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "progress.log"), "a") as f:
        print(*a, file=f, flush=True)


def pmap(fn, items):
    return list(_POOL.map(fn, items))


def write_report(name: str, rec: dict) -> None:
    d = os.path.join(ROOT, "gpurun_out", "parity")
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, f"{name}.json"), "w") as f:
        json.dump(rec, f, indent=1, sort_keys=True)


class OracleUnit:
    """The oracle's view of one (sequence, KV head): logical rows, summaries."""

    def __init__(self, k_rows, v_rows, cap, P):
        n, d = k_rows.shape
        self.P = P
        self.K = np.zeros((cap, d), k_rows.dtype)
        self.V = np.zeros((cap, d), v_rows.dtype)
        self.K[:n], self.V[:n] = k_rows, v_rows
        npg = n_pages(cap, P)
        self.smax = np.zeros((npg, d), k_rows.dtype)
        self.smin = np.zeros((npg, d), k_rows.dtype)
        self.n = 0
        self.append(None, None, n)

    def append(self, k_rows, v_rows, count=None):
        n0 = self.n
        if k_rows is not None:
            count = k_rows.shape[0]
            self.K[n0:n0 + count], self.V[n0:n0 + count] = k_rows, v_rows
        oracle.summaries_append(self.K, n0, n0 + count, self.P, self.smax, self.smin)
        self.n = n0 + count


def evict_layer(sess, slot, stats):
    """Runs the library's prefill eviction for layer slot `slot`, checks every
    unit's kept set against the oracle and returns {(b, h): OracleUnit}.  A
    sequence with an accepted near-tie swap gets the oracle's kept rows
    written into the library's cache."""
    rkv = lib()
    wl = sess.wl
    B, Hkv, G, w, P = sess.B, sess.Hkv, sess.G, wl.window, sess.P
    L_max = max(sess.prompt_lens)
    kept = torch.full((B, Hkv, max(sess.keep)), -7, dtype=torch.int32, device="cuda")
    pooled = torch.zeros((B, Hkv, L_max), dtype=torch.float32, device="cuda")
    k, v, qw = sess.prefill_layer(slot, kept_idx=kept, pooled=pooled)
    torch.cuda.synchronize()
    kept_h = kept.cpu().numpy()
    cap = max(sess.capacity)
    lid = sess.layer_ids[slot]
    res, kept_o, swapped_seqs = {}, {}, set()
    keep_o = [oracle.split_ratio(L / wl.budget, L, w)[3] for L in sess.prompt_lens]
    assert sess.keep == keep_o, (sess.keep, keep_o)
    host = [(bits(k[b, :, :L].cpu()), bits(v[b, :, :L].cpu()), bits(qw[b].cpu()))
            for b, L in enumerate(sess.prompt_lens)]
    del k, v, qw

    def one(bh):
        b, h = bh
        kb, _, qb = host[b]
        return oracle.snapkv_group(qb[h * G:(h + 1) * G], kb[h], wl.pool_kernel, keep_o[b],
                                   sess.scale)

    units = [(b, h) for b in range(B) for h in range(Hkv)]
    for (b, h), (k_o, _, pl_o) in zip(units, pmap(one, units)):
        L = sess.prompt_lens[b]
        s = check_kept(kept_h[b, h, :keep_o[b]], k_o, pl_o, w)
        stats["stage1_units"] += 1
        if s:
            stats["near_tie_swaps"] += s
            stats["units_with_swaps"].append([lid, b, h, s])
            swapped_seqs.add(b)
        res[(b, h)] = OracleUnit(host[b][0][h][k_o], host[b][1][h][k_o], cap, P)
        kept_o[(b, h)] = k_o
        if wl.needle_span:
            needle = np.asarray(wl.needle_rows(lid, b, L, 0))
            hit = int(np.isin(needle, k_o).sum())
            stats.setdefault("stage1_needle_rows_kept", []).append([lid, b, h, hit,
                                                                   len(needle)])
    for b in sorted(swapped_seqs):
        # both sides continue from the oracle's kept rows
        keep_b = sess.keep[b]
        kk = torch.from_numpy(np.stack([res[(b, h)].K[:keep_b] for h in range(Hkv)])[None])
        vv = torch.from_numpy(np.stack([res[(b, h)].V[:keep_b] for h in range(Hkv)])[None])
        if sess.wl.dtype == torch.bfloat16:
            kk, vv = kk.view(torch.bfloat16), vv.view(torch.bfloat16)
        z = torch.zeros(1, dtype=torch.int32, device="cuda")
        rkv.rkv_append_summaries(sess.g, sess.caches[slot].row_slice(b, b + 1), z, z + keep_b,
                                 keep_b, sess.summ[slot][b:b + 1], k_src=kk.cuda(),
                                 v_src=vv.cuda())
    torch.cuda.synchronize()
    say(f"  layer {lid}: stage-1 units {B * Hkv}, near-tie swaps so far "
        f"{stats['near_tie_swaps']} (sequences rewritten: {sorted(swapped_seqs)})")
    return res, kept_o


def decode_and_check(sess, ounits, steps, when=None, turn=0, stats=None, needle=None):
    """Runs `steps` decode steps of every layer slot with rkv_decode_step (the
    session's call) and compares the oracle units ounits[(slot, b, h)] at
    the steps where when(unit, step) holds (None: every unit at every step).
    needle(slot, b, h) -> logical pages or None, if given, counts the checked
    steps whose page set holds one of those pages."""
    rkv = lib()
    wl = sess.wl
    G, B, Hkv = sess.G, sess.B, sess.Hkv
    nl = sess.n_layers
    chan = [torch.zeros((B, Hkv, wl.k1), dtype=torch.int32, device="cuda") for _ in range(nl)]
    pidx = [torch.zeros((B, Hkv, wl.k2), dtype=torch.int32, device="cuda") for _ in range(nl)]
    outs = [torch.zeros((B, sess.Hq, sess.d), dtype=torch.float32, device="cuda")
            for _ in range(nl)]
    inputs = sess.make_inputs(steps, turn=turn)
    stats = {} if stats is None else stats
    checked = 0
    for s in range(steps):
        per_layer, _, n_new = inputs[s]
        for l in range(nl):
            kt, vt, qt = per_layer[l]
            rkv.rkv_decode_step(sess.g, qt, kt, vt, sess.caches[l], n_new, sess.summ[l], wl.k1,
                                wl.k2, sess.scale, outs[l], sess.ws, chan_idx=chan[l],
                                page_idx=pidx[l])
        torch.cuda.synchronize()
        host = []
        for l in range(nl):
            kt, vt, qt = per_layer[l]
            host.append((bits(kt.cpu()), bits(vt.cpu()), bits(qt.cpu()), chan[l].cpu().numpy(),
                         pidx[l].cpu().numpy(), outs[l].cpu().double().numpy()))
        for (l, b, h), o in ounits.items():
            o.append(host[l][0][b, h][None], host[l][1][b, h][None])
        todo = [(u, o) for u, o in ounits.items() if when is None or when(u, s)]

        def one(item):
            (l, b, h), o = item
            kc, vc, qc, gc, gp, go = host[l]
            c_o, p_o, _, out_o = oracle.hsa_group(qc[b, h * G:(h + 1) * G], o.K, o.V, o.smax,
                                                  o.smin, o.n, sess.P, wl.k1, wl.k2, sess.scale)
            bad = []
            if not np.array_equal(gc[b, h], c_o):
                bad.append(f"channels {gc[b, h]} != {c_o}")
            if not np.array_equal(gp[b, h], p_o):
                bad.append(f"pages {gp[b, h]} != {p_o}")
            err = float(np.abs(go[b, h * G:(h + 1) * G] - out_o).max())
            if err > OUT_ATOL:
                bad.append(f"max abs error {err}")
            return (l, b, h), bad, err

        for (l, b, h), bad, err in pmap(one, todo):
            assert not bad, (sess.layer_ids[l], b, h, s, bad)
            stats["max_abs_err"] = max(stats.get("max_abs_err", 0.0), err)
            if needle is not None:
                pages = needle(l, b, h)
                if pages is not None:
                    hit = bool(np.isin(host[l][4][b, h], pages).any())
                    stats["needle_page_hits"] = stats.get("needle_page_hits", 0) + int(hit)
                    stats["needle_page_checks"] = stats.get("needle_page_checks", 0) + 1
            checked += 1
        if s % 4 == 0:
            say(f"  step {s}: checks so far {checked}")
    sess.advance(steps)
    torch.cuda.synchronize()
    for (l, b, h), o in ounits.items():
        NP = n_pages(o.n, sess.P)
        gmax, gmin = gpu_summaries(sess.summ[l], b, h, NP)
        np.testing.assert_array_equal(gmax, o.smax[:NP])
        np.testing.assert_array_equal(gmin, o.smin[:NP])
    return checked


def new_stats(wl):
    return {"workload": wl.name, "stage1_units": 0, "near_tie_swaps": 0,
            "units_with_swaps": [], "near_tie_rule": "relative gap < 1e-6 of the oracle's "
                                                     "pooled score at the keep boundary"}


def test_llama_32k_one_layer():
    """Prompt 32,768, budget 512 (keep 3,191), all 8 KV heads, 128 steps,
    every unit at every step."""
    wl = workloads.LLAMA_32K
    say(f"case {wl.name}")
    sess = Session(wl, extra_rows=wl.decode_steps, device="cuda")
    assert sess.keep == [3191]
    stats = new_stats(wl)
    ou, _ = evict_layer(sess, 0, stats)
    ou = {(0, b, h): o for (b, h), o in ou.items()}
    n = decode_and_check(sess, ou, wl.decode_steps, stats=stats)
    stats["decode_checks"] = n
    say(f"  decode checks {n}")
    assert n == wl.decode_steps * sess.B * sess.Hkv
    write_report(wl.name, stats)


def test_llama_109k_budget256():
    """Prompt 109,568, budget 256 (keep 1,359), page 8, 64-row needle, 256
    steps, every unit at every step.  Reported: the needle rows stage 1 keeps
    per head, and the share of checked steps whose page set holds a page
    with a kept needle row."""
    wl = workloads.EXTREME_109K
    say(f"case {wl.name}")
    sess = Session(wl, extra_rows=wl.decode_steps, device="cuda")
    assert sess.keep == [1359]
    stats = new_stats(wl)
    ou, kept = evict_layer(sess, 0, stats)
    needle = np.asarray(wl.needle_rows(0, 0, sess.prompt_lens[0], 0))
    pages = {}
    for (b, h), k_o in kept.items():
        logical = np.nonzero(np.isin(k_o, needle))[0]
        pages[(0, b, h)] = np.unique(logical // sess.P) if len(logical) else None
    ou = {(0, b, h): o for (b, h), o in ou.items()}
    n = decode_and_check(sess, ou, wl.decode_steps, stats=stats,
                         needle=lambda l, b, h: pages[(l, b, h)])
    stats["decode_checks"] = n
    say(f"  decode checks {n}; needle page hits {stats.get('needle_page_hits')} of "
        f"{stats.get('needle_page_checks')}")
    assert n == wl.decode_steps * sess.B * sess.Hkv
    write_report(wl.name, stats)


@pytest.mark.timeout(1500)
def test_batched_32k_launch_shape():
    """The benchmark's launch shape: all 32 layers, batch 32, prompts
    16K-32K, budget 1,024, page 16, k1 32, k2 64, the fused kernel over all
    256 (sequence, head) units per layer, 68 steps (4 warm-up + 64 timed).
    Stage 1 on every unit of every layer; every unit of every layer checked
    at every step; then the same decode twice, bit for bit."""
    wl = workloads.BATCHED_32L
    rkv = lib()
    say(f"case {wl.name} (all {wl.layers} layers)")
    steps = 68
    sess = Session(wl, extra_rows=steps, device="cuda")
    assert rkv.fused_path(sess.g, sess.B, sess.P, sess.max_pages, wl.k2)
    stats = new_stats(wl)
    ou = {}
    for slot in range(sess.n_layers):
        res, _ = evict_layer(sess, slot, stats)
        for (b, h), o in res.items():
            ou[(slot, b, h)] = o
    n = decode_and_check(sess, ou, steps, stats=stats)
    stats["decode_checks"] = n
    stats["decode_checks_rule"] = "every unit of every layer at every step"
    say(f"  decode checks {n}")
    units = sess.B * sess.Hkv
    assert n == steps * units * sess.n_layers
    # determinism at the launch shape: the same decode, twice, bit for bit
    q = sess.wl.decode_tokens(0, steps, torch.tensor(sess.positions()), device="cuda")[2]
    n_now = torch.tensor(sess.rows, dtype=torch.int32, device="cuda")
    res = []
    for _ in range(2):
        out = torch.zeros((sess.B, sess.Hq, sess.d), dtype=torch.float32, device="cuda")
        pidx = torch.zeros((sess.B, sess.Hkv, wl.k2), dtype=torch.int32, device="cuda")
        rkv.rkv_hsa_decode(sess.g, q, sess.caches[0], n_now, sess.summ[0], wl.k1, wl.k2,
                           sess.scale, out, sess.ws, page_idx=pidx)
        torch.cuda.synchronize()
        res.append((out.view(torch.int32).clone(), pidx.clone()))
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])
    stats["repeat_bitwise_equal"] = True
    write_report(wl.name, stats)


def test_multiturn_131k():
    """Batch 4, 131,072 cached rows kept whole, page 32, k1 32, k2 128, four
    turns of (append 2,048 rows, 64 steps); every unit at every step of every
    turn.  The turn's needle (planted in the turn's rows, the turn's queries
    aligned with it) is reported as the share of checked steps whose page set
    holds one of its pages."""
    wl = workloads.MT_131K
    say(f"case {wl.name}")
    steps = wl.decode_steps
    sess = Session(wl, extra_rows=0, device="cuda")
    k, v, _ = sess.prefill_layer(0)
    torch.cuda.synchronize()
    cap = max(sess.capacity)
    ou = {}
    for b in range(sess.B):
        L = sess.prompt_lens[b]
        kb, vb = bits(k[b, :, :L].cpu()), bits(v[b, :, :L].cpu())
        for h in range(sess.Hkv):
            ou[(0, b, h)] = OracleUnit(kb[h], vb[h], cap, sess.P)
    del k, v
    stats = new_stats(wl)
    total = 0
    per_turn = []
    span = max(1, wl.needle_span)
    for turn in range(wl.turns):
        start = list(sess.rows)
        kt, vt = sess.append_turn(0, turn)
        torch.cuda.synchronize()
        kc, vc = bits(kt.cpu()), bits(vt.cpu())
        for (_, b, h), o in ou.items():
            o.append(kc[b, h], vc[b, h])
        sess.advance(wl.turn_append)
        pages = {}
        for b in range(sess.B):
            at = start[b] + wl.turn_needle_offset(0, b, turn)
            pages[b] = np.unique(np.arange(at, at + span) // sess.P)
        tstats = {}
        n = decode_and_check(sess, ou, steps, turn=turn, stats=tstats,
                             needle=lambda l, b, h: pages[b])
        total += n
        per_turn.append({"turn": turn, "decode_checks": n,
                         "needle_page_hits": tstats.get("needle_page_hits", 0),
                         "needle_page_checks": tstats.get("needle_page_checks", 0),
                         "max_abs_err": tstats.get("max_abs_err", 0.0)})
        say(f"  turn {turn}: checks {n}, needle page hits {tstats.get('needle_page_hits')}"
            f"/{tstats.get('needle_page_checks')}")
    stats["turns"] = per_turn
    stats["decode_checks"] = total
    say(f"  decode checks {total}")
    assert total == wl.turns * steps * sess.B * sess.Hkv
    write_report(wl.name, stats)
