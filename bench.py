"""Decode throughput of the RocketKV path on one MI355X.

A step is one decode step of the whole model: for every layer, append the new
token's K/V (and fold it into the page summaries), then Hybrid Sparse
Attention (channel ranking, page bound scores, page top-k2, attention over
the selected pages).  Caches are first pruned by SnapKV++ (timed separately,
reported as stage1).  Steps are HIP-graph replays of the captured launches;
inputs are resident in HBM before the timed region starts.

Default workload: all 32 Llama3.1-8B layers, batch 32, contexts 16K-32K,
budget 1,024 tokens per sequence.  Prints one JSON line on stdout.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "HSA decode steps/s + attended tokens/s, achieved HBM GB/s vs peak, 32K ctx"
DEFAULT_WORKLOAD = "llama8b-32layer-b32-ctx16k-32k"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def attended_rows(sess, layer_page_idx, rows_now):
    """Valid rows in the selected pages, per (sequence, KV head), summed."""
    import torch
    P = sess.P
    pidx = layer_page_idx.cpu().to(torch.int64)            # [B, Hkv, k2]
    n = torch.tensor(rows_now, dtype=torch.int64)[:, None, None]
    valid = (pidx >= 0)
    rows = torch.clamp(n - pidx * P, min=0, max=P) * valid
    return int(rows.sum())


def step_bytes(sess, rows_now, per_head_rows):
    """Algorithmic HBM bytes of one decode step over every layer, and the
    attention share (gathered K/V + q + out) of layer 0.
    per_head_rows[l]: attended rows of layer l summed over (sequence, KV head)."""
    wl = sess.wl
    s = 2 if wl.dtype.itemsize == 2 else 4
    B, Hkv, Hq, d, P = sess.B, sess.Hkv, sess.Hq, sess.d, sess.P
    pages = sum((n + P - 1) // P for n in rows_now)
    q = B * Hq * d * s
    summaries = Hkv * wl.k1 * pages * 2 * s
    kv = [r * d * 2 * s for r in per_head_rows]
    out = B * Hq * d * 4
    append = B * 3 * Hkv * d * 2 * s
    return (q + summaries + out + append) * sess.n_layers + sum(kv), kv[0] + q + out


def measured_copy_gbs(dev, nbytes: int = 1 << 30, reps: int = 5) -> float:
    """Read + write bandwidth of a plain device-to-device copy: the practical
    HBM ceiling on this device, reported beside the 8 TB/s spec."""
    import torch
    x = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    y.copy_(x)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        y.copy_(x)
    e1.record()
    torch.cuda.synchronize()
    gbs = reps * 2 * nbytes / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del x, y
    torch.cuda.empty_cache()
    return gbs


def measured_read_gbs(dev, nbytes: int = 2 << 30, reps: int = 5) -> tuple[float, float]:
    """The library's read probe over a 2 GiB buffer (eight times the 256 MB
    last-level cache): a plain stream of every 4 KB chunk, and a gather of
    half of them in a seeded random order (4 KB page slices at scattered
    offsets, the decode kernel's K/V pattern).  Returns both rates, GB/s."""
    import torch
    from sparse_kv_cache_hsa_amd import rkv
    chunk = rkv.RKV_READ_PROBE_CHUNK
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(rkv.RKV_READ_PROBE_SINK_WORDS, dtype=torch.int32, device=dev)
    n = nbytes // chunk
    g = torch.Generator().manual_seed(0)
    offsets = (torch.randperm(n, generator=g)[: n // 2] * chunk).to(dev)
    rates = []
    for offs, nread in ((None, n * chunk), (offsets, (n // 2) * chunk)):
        rkv.rkv_read_probe(buf, sink, offs)  # warm-up; checks the offsets
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            rkv.rkv_read_probe(buf, sink, offs, check_offsets=False)
        e1.record()
        torch.cuda.synchronize()
        rates.append(reps * nread / (e0.elapsed_time(e1) * 1e-3) / 1e9)
    del buf, sink, offsets
    torch.cuda.empty_cache()
    return rates[0], rates[1]


def counted_traffic(kernel: str, workload: str, build_id: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, copy-calibrated), or None when there is none for
    this workload or it was taken on another build of the kernels."""
    key = kernel.replace(" + ", "+").replace(" ", "-")
    path = os.path.join(ROOT, "profiles", f"{key}_{workload}_counters.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("build_id") != build_id or rec.get("workload") != workload:
        return None
    return int(rec["traffic_bytes_per_launch"])


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def host_threads() -> tuple[int, int]:
    """(nproc, threads used): the host's CPUs and the pool size, which stays
    within the 16-core share of one GPU on a shared host."""
    n = len(os.sched_getaffinity(0))
    return n, max(1, min(16, n))


def _pool_run(fn, items, threads: int, budget_s: float, max_reps: int = 100000):
    """Runs fn over items (repeatedly, until about budget_s seconds) on a
    thread pool; returns (repetitions, seconds).  The oracle is C and
    releases the interpreter lock, so units run in parallel."""
    import concurrent.futures as cf
    pool = cf.ThreadPoolExecutor(threads) if threads > 1 else None
    t0 = time.perf_counter()
    reps = 0
    while True:
        if pool:
            list(pool.map(fn, items))
        else:
            for u in items:
                fn(u)
        reps += 1
        el = time.perf_counter() - t0
        if el >= budget_s or reps >= max_reps:
            break
    if pool:
        pool.shutdown()
    return reps, el


def read_units(sess, layer: int, q):
    """The GPU run's bytes of one layer, per (sequence, KV head): cache rows
    k, v [n, d], summaries smax, smin [NP, d] and the step's queries [G, d],
    read back from HBM (bf16 as raw bits)."""
    import numpy as np

    from sparse_kv_cache_hsa_amd import synth
    c, P, G = sess.caches[layer], sess.P, sess.G
    table = c.page_table.cpu()
    units = []
    for b in range(sess.B):
        n = sess.rows[b]
        np_ = (n + P - 1) // P
        blocks = table[b, :np_].to(c.k_pool.device).long()
        kb = c.k_pool[blocks].permute(1, 0, 2, 3).reshape(sess.Hkv, np_ * P, sess.d)[:, :n]
        vb = c.v_pool[blocks].permute(1, 0, 2, 3).reshape(sess.Hkv, np_ * P, sess.d)[:, :n]
        sm = sess.summ[layer][b, :, :, :, :np_].transpose(-1, -2)      # [Hkv, 2, NP, d]
        kb, vb, sm = synth.to_bits(kb.cpu()), synth.to_bits(vb.cpu()), synth.to_bits(sm.cpu())
        qb = synth.to_bits(q[b].cpu())
        for h in range(sess.Hkv):
            units.append((np.ascontiguousarray(kb[h]), np.ascontiguousarray(vb[h]),
                          np.ascontiguousarray(qb[h * G:(h + 1) * G]),
                          np.ascontiguousarray(sm[h, 0]), np.ascontiguousarray(sm[h, 1]), n))
    return units


def cpu_baseline(wl, sess, q_last, budget_s: float):
    """The oracle's decode step (fold the step's row into the summaries, then
    HSA) on the host cores, on the GPU run's own bytes: layer 0's cache,
    summaries and last-step queries read back, every (sequence, KV head) unit
    repeated until about budget_s seconds, scaled to every layer.  Also the
    host's stage-1 (SnapKV++) time for one layer, from a sample of units on
    the workload's prompts.  The oracle computes in fp64 with plain loops and
    a sort: a stated baseline, not a tuned CPU implementation."""
    import oracle
    nproc, threads = host_threads()
    units = read_units(sess, 0, q_last)

    def one(u):
        k, v, q, smax, smin, n = u
        oracle.summaries_append(k, n - 1, n, sess.P, smax, smin)
        oracle.hsa_group(q, k, v, smax, smin, n, sess.P, wl.k1, wl.k2, sess.scale)

    res = {"cpu_model": cpu_model(), "nproc": nproc}
    for tag, th, bud in (("", threads, budget_s), ("_1thread", 1, budget_s / 3)):
        reps, el = _pool_run(one, units, th, bud)
        per_layer_step = el / reps
        res["value" + tag] = round(1.0 / (per_layer_step * sess.n_layers), 4)
        res["sample" + tag] = (f"{reps} repetitions of layer 0's decode step over all "
                               f"{len(units)} (sequence, KV head) units, on the GPU run's cache "
                               f"bytes read back, scaled to {sess.n_layers} layers; {el:.1f} s on "
                               f"{th} thread(s); the oracle as it stands: fp64 "
                               f"arithmetic, plain loops, untuned")
    res.update({"unit": "steps/s", "cores": threads, "kind": "oracle",
                "sample": res.pop("sample"), "value": res.pop("value")})
    if wl.evicts:
        res["stage1"] = host_stage1(wl, sess, threads, budget_s / 2)
    return res


def host_stage1(wl, sess, threads: int, budget_s: float):
    """Host SnapKV++ for one layer: the oracle on whole sequences' prompts of
    layer 0 (all KV heads of as many sequences as fill the pool), its rate
    scaled to the layer's B x Hkv units."""
    import oracle
    from sparse_kv_cache_hsa_amd import synth
    n_seq = max(1, -(-threads // sess.Hkv))
    units = []
    for b in range(n_seq):
        L = sess.prompt_lens[b]
        k, _ = wl.prompt_kv(sess.layer_ids[0], b, L, device=sess.dev)
        qw = wl.window_q(sess.layer_ids[0], b, L, device=sess.dev)
        kb, qb = synth.to_bits(k.cpu()), synth.to_bits(qw.cpu())
        for h in range(sess.Hkv):
            units.append((qb[h * sess.G:(h + 1) * sess.G].copy(), kb[h].copy(), sess.keep[b]))

    def one(u):
        oracle.snapkv_group(u[0], u[1], wl.pool_kernel, u[2], sess.scale)

    reps, el = _pool_run(one, units, threads, budget_s, max_reps=20)
    rate = reps * len(units) / el                       # units per second
    layer_s = sess.B * sess.Hkv / rate
    return {"s_per_layer": round(layer_s, 3),
            "sample": f"{reps} x {len(units)} units (sequences 0..{n_seq - 1}, every KV head, "
                      f"prompts of {min(sess.prompt_lens[:n_seq])}..{max(sess.prompt_lens[:n_seq])} "
                      f"rows) in {el:.1f} s on {threads} thread(s), scaled to the layer's "
                      f"{sess.B * sess.Hkv} units"}


def graph_of(torch, fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    return g


def turn_plan(sess, steps_per_turn: int, view_budget: int = 0):
    """Inputs of every turn, generated before anything is timed: the turn's
    append sources per layer, its decode-step inputs and, with a view budget,
    the turn's window queries and view sizes.  Row counts are simulated and
    restored, so the session is left as it was."""
    rows0 = list(sess.rows)
    plan = []
    for t in range(sess.wl.turns):
        tp = {"src": [sess.turn_source(l, t) for l in range(sess.n_layers)]}
        sess.advance(sess.wl.turn_append)
        if view_budget:
            tp["keep"] = sess.turn_view_keep(view_budget)
            tp["n_rows"] = list(sess.rows)
            tp["qw"] = [sess.turn_window_q(l, t) for l in range(sess.n_layers)]
            sess.view_rows = list(tp["keep"])
            tp["steps"] = sess.make_view_inputs(steps_per_turn, t)
        else:
            tp["steps"] = sess.make_inputs(steps_per_turn, t)
        sess.advance(steps_per_turn)
        plan.append(tp)
    sess.rows = rows0
    return plan


def run_turns(torch, sess, plan, use_graph: bool, view_ws=None):
    """Runs every turn: the turn's append (and, with views, the per-turn
    filter), then its decode steps; returns per-turn event times in ms and
    the total.  Graphs are captured beforehand; their replays are timed."""
    view = view_ws is not None
    turns = []
    for tp in plan:
        def prologue(tp=tp):
            saved = sess.rows
            for l in range(sess.n_layers):
                sess.append_source(l, tp["src"][l])
            if view:
                sess.rows = tp["n_rows"]
                for l in range(sess.n_layers):
                    sess.turn_filter(l, tp["qw"][l], tp["keep"], view_ws)
                sess.rows = saved
        step = sess.view_step if view else sess.step
        if use_graph:
            g_pro = graph_of(torch, prologue)
            g_steps = [graph_of(torch, lambda i=i: step(i)) for i in tp["steps"]]
            turns.append((g_pro.replay, [g.replay for g in g_steps], g_pro, g_steps))
        else:
            turns.append((prologue, [lambda i=i: step(i) for i in tp["steps"]]))
    torch.cuda.synchronize()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in turns]
    torch.cuda.synchronize()
    for t, tr in enumerate(turns):
        ev[t][0].record()
        tr[0]()
        ev[t][1].record()
        for f in tr[1]:
            f()
        ev[t][2].record()
    torch.cuda.synchronize()
    pro = [e[0].elapsed_time(e[1]) for e in ev]
    dec = [e[1].elapsed_time(e[2]) for e in ev]
    total = ev[0][0].elapsed_time(ev[-1][2])
    for tp in plan:
        sess.advance(sess.wl.turn_append + len(tp["steps"]))
    if view:
        sess.view_rows = [k + len(plan[-1]["steps"]) for k in plan[-1]["keep"]]
    return pro, dec, total


def mt_filter_leg(torch, rkv, wl, args, dev, budget: int):
    """RocketKV-MT on the multi-turn workload: per turn, append the turn's
    rows to the full cache, re-run SnapKV++ over the whole history with the
    turn's last w queries into a compacted view (stage 1's share of `budget`
    under the adaptive split), then decode on the view while every new token
    also goes to the full cache.  A session of its own; returns its report."""
    from sparse_kv_cache_hsa_amd.session import Session
    spt = args.steps // wl.turns
    sess = Session(wl, extra_rows=args.warmup + max(0, spt - wl.decode_steps), device=dev)
    for l in range(sess.n_layers):
        sess.prefill_layer(l)
    final = [n + wl.turns * (wl.turn_append + spt) for n in sess.rows]
    most = max(rkv.rkv_split_ratio(n / budget, n, wl.window)[3] if n > budget else n
               for n in final)
    sess.enable_turn_view(most, spt + 1)
    # the last turn's filter sees the longest history
    ws = sess.turn_filter_workspace(max(sess.rows) + wl.turns * wl.turn_append
                                    + (wl.turns - 1) * spt)
    plan = turn_plan(sess, spt, view_budget=budget)
    torch.cuda.synchronize()
    pro, dec, total = run_turns(torch, sess, plan, not args.no_graph, view_ws=ws)
    K = spt * wl.turns
    log(f"[bench] mt-filter: {K} steps over {wl.turns} turns in {total:.2f} ms; per turn "
        f"append+filter {sum(pro) / len(pro):.3f} ms, decode {sum(dec) / len(dec):.3f} ms")
    mode = rkv.decode_mode(sess.g, sess.B, sess.P, sess.view_max_pages, wl.k2, wl.k1,
                           rkv.RKV_BF16 if wl.dtype.itemsize == 2 else rkv.RKV_F32)
    return {"budget": budget, "view_rows_last_turn": plan[-1]["keep"],
            "steps_per_s": round(K / (total * 1e-3), 3), "ms_per_step": round(total / K, 5),
            "append_and_filter_ms_per_turn": [round(x, 4) for x in pro],
            "decode_ms_per_turn": [round(x, 4) for x in dec],
            "decode_us_per_step": round(sum(dec) * 1e3 / K, 3),
            "view_path": FORMS[mode]}


FORMS = {1: "standalone kernels", 2: "fused", 3: "fused split-K"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed decode steps (default 64; multi-turn workloads: every "
                         "turn's steps, spread evenly over the turns)")
    ap.add_argument("--warmup", type=int, default=4)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-graph", action="store_true", help="enqueue steps eagerly")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--mt-filter", type=int, default=0, metavar="BUDGET",
                    help="multi-turn workloads: also time RocketKV-MT's per-turn view at this "
                         "total token budget (reported under mt_filter)")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only copy MIB MiB device to device 3 times (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the decode path has no multi-GPU leg "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_kv_cache_hsa_amd import rkv, workloads
    from sparse_kv_cache_hsa_amd.session import Session

    if args.copy_probe > 0:
        x = torch.ones(args.copy_probe << 20, dtype=torch.uint8, device="cuda:0")
        y = torch.empty_like(x)
        for _ in range(3):
            y.copy_(x)
        torch.cuda.synchronize()
        log(f"[bench] copied {args.copy_probe} MiB device to device 3 times")
        return

    rkv.load_library()
    wl = workloads.ALL[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    turns = wl.turns > 1
    if args.steps is None:
        args.steps = wl.turns * wl.decode_steps if turns else 64
    K, W = args.steps, args.warmup
    if turns and (K % wl.turns or K < wl.turns):
        sys.exit(f"--steps must be a positive multiple of the {wl.turns} turns")
    log(f"[bench] workload {wl.name}: {wl.description}")
    extra = W + (max(0, K // wl.turns - wl.decode_steps) if turns else K)
    sess = Session(wl, extra_rows=extra, device=dev)
    log(f"[bench] keep per sequence {min(sess.keep)}..{max(sess.keep)}, max_pages "
        f"{sess.max_pages}, blocks {sess.num_blocks}")

    # ---- stage 1 (prefill eviction), per layer --------------------------------
    ev_ms = []
    ews = sess.evict_workspace() if wl.evicts else None
    for l in range(sess.n_layers):
        t = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        sess.prefill_layer(l, ws=ews, timer=t)
        torch.cuda.synchronize()
        ev_ms.append(t[0].elapsed_time(t[1]))
    del ews
    torch.cuda.empty_cache()
    log(f"[bench] prefill done: {sum(ev_ms):.1f} ms over {sess.n_layers} layers")

    # ---- decode inputs and graphs ------------------------------------------
    # multi-turn: W warm-up steps on the prefilled cache, then every turn
    # (append of the turn's rows, then its steps) inside the timed region
    n_main = W if turns else W + K
    inputs = sess.make_inputs(n_main)
    torch.cuda.synchronize()
    graphs = []
    if not args.no_graph:
        graphs = [graph_of(torch, lambda i=i: sess.step(i)) for i in inputs]
        torch.cuda.synchronize()
        log(f"[bench] captured {len(graphs)} step graphs")

    def run(s):
        if graphs:
            graphs[s].replay()
        else:
            sess.step(inputs[s])

    for s in range(W):
        run(s)
    torch.cuda.synchronize()
    sess.advance(W)
    turn_report = None
    if turns:
        spt = K // wl.turns
        plan = turn_plan(sess, spt)
        last_inp = plan[-1]["steps"][-1]
        app_ms, dec_ms, ms_total = run_turns(torch, sess, plan, not args.no_graph)
        del plan
        turn_report = {"turns": wl.turns, "steps_per_turn": spt,
                       "append_rows": wl.turn_append,
                       "append_ms_per_turn": [round(x, 4) for x in app_ms],
                       "append_ms_mean": round(sum(app_ms) / len(app_ms), 4),
                       "decode_ms_per_turn": [round(x, 4) for x in dec_ms],
                       "decode_us_per_step": round(sum(dec_ms) * 1e3 / K, 3)}
        log(f"[bench] {wl.turns} turns x ({wl.turn_append}-row append + {spt} steps) in "
            f"{ms_total:.2f} ms; append {turn_report['append_ms_mean']:.3f} ms per turn, decode "
            f"{turn_report['decode_us_per_step']:.1f} us per step")
    else:
        last_inp = inputs[W + K - 1]
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for s in range(W, W + K):
            run(s)
        e1.record()
        torch.cuda.synchronize()
        ms_total = e0.elapsed_time(e1)
        sess.advance(K)
    ms_step = ms_total / K
    log(f"[bench] {K} steps in {ms_total:.2f} ms -> {ms_step * 1e3:.1f} us/step")

    # attended rows of the last step (page_idx of every layer are current)
    rows_last = sess.rows
    per_head_rows = [attended_rows(sess, sess.page_idx[l], rows_last) for l in range(sess.n_layers)]
    attended_seq_layer = sum(per_head_rows) / sess.Hkv       # per (sequence, layer)
    step_b, attend_b0 = step_bytes(sess, rows_last, per_head_rows)
    log(f"[bench] algorithmic bytes per step {step_b / 1e9:.3f} GB, attended rows per step "
        f"(all sequences and layers, per KV head) {attended_seq_layer:.1f}")

    # ---- dominant kernel ----------------------------------------------------
    # Fused path: a step is one decode_kernel launch per layer on this stream,
    # so the timed region itself gives the average launch duration.  Split-K
    # fused path: the same, per layer the split-K decode_kernel and its merge.
    # Standalone path: the attention launches of every layer, captured alone.
    per_layer, _, n_new = last_inp
    mode = rkv.decode_mode(sess.g, sess.B, sess.P, sess.max_pages, wl.k2, wl.k1,
                           rkv.RKV_BF16 if wl.dtype.itemsize == 2 else rkv.RKV_F32)
    if mode in (rkv.RKV_FORM_FUSED, rkv.RKV_FORM_SPLITK):
        kernel = ("decode_kernel" if mode == rkv.RKV_FORM_FUSED
                  else "decode_kernel split-K + attend_merge_kernel")
        launch_us = (turn_report["decode_us_per_step"] if turns else ms_total * 1e3 / K) \
            / sess.n_layers
        bytes_launch = step_b / sess.n_layers
    else:
        kernel = "attend_kernel + attend_merge_kernel"
        for l in range(sess.n_layers):
            rkv.rkv_hsa_select(sess.g, per_layer[l][2], n_new, sess.P, sess.summ[l], wl.k1,
                               wl.k2, sess.page_idx[l], sess.ws)
        torch.cuda.synchronize()
        # back-to-back launches in one graph, so that a replay's own start-up
        # cost is spread over many launches
        reps = max(1, 64 // sess.n_layers)

        def attends():
            for _ in range(reps):
                for l in range(sess.n_layers):
                    rkv.rkv_hsa_attend(sess.g, per_layer[l][2], sess.caches[l], n_new,
                                       sess.page_idx[l], wl.k2, sess.scale, sess.out, sess.ws)
        gph = graph_of(torch, attends)
        bytes_launch = attend_b0
        gph.replay()
        torch.cuda.synchronize()
        k0, k1e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k0.record()
        for _ in range(4):
            gph.replay()
        k1e.record()
        torch.cuda.synchronize()
        launch_us = k0.elapsed_time(k1e) * 1e3 / (4 * reps * sess.n_layers)
    kern_gbs = bytes_launch / (launch_us * 1e-6) / 1e9
    traffic = counted_traffic(kernel, wl.name, rkv.load_library().rkv_build_id().decode())
    log(f"[bench] {kernel}: {launch_us:.2f} us/launch, {bytes_launch / 1e6:.2f} MB/launch -> "
        f"{kern_gbs:.0f} GB/s; counted traffic "
        f"{'n/a' if traffic is None else f'{traffic / 1e6:.2f} MB/launch'}")

    copy_gbs = measured_copy_gbs(dev)
    log(f"[bench] measured device copy (1 GiB, read + write): {copy_gbs:.0f} GB/s")
    read_gbs, gather_gbs = measured_read_gbs(dev)
    log(f"[bench] measured read probe (2 GiB): stream {read_gbs:.0f} GB/s, "
        f"4 KB gather {gather_gbs:.0f} GB/s")

    steps_per_s = 1e3 / ms_step
    result = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if wl.dtype.itemsize == 2 else "f32",
        "data": "synthetic (seeded Gaussian K/V with outlier channels, RoPE'd; no model weights)",
        "attended_tokens_per_s": round(steps_per_s * attended_seq_layer, 1),
        "step_hbm_bytes": step_b,
        "step_hbm_gbs": round(step_b / (ms_step * 1e-3) / 1e9, 1),
        "step_hbm_frac": round(step_b / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "stage1": {"ms_total": round(sum(ev_ms), 3), "ms_per_layer": round(sum(ev_ms) / len(ev_ms), 3),
                   "batch_per_call": sess.B},
        "config": {"workload": wl.name, "layers": sess.n_layers, "batch": sess.B,
                   "q_heads": sess.Hq, "kv_heads": sess.Hkv, "head_dim": sess.d,
                   "page_size": sess.P, "k1": wl.k1, "k2": wl.k2,
                   "prompt_len_min": min(sess.prompt_lens), "prompt_len_max": max(sess.prompt_lens),
                   "kept_rows_min": min(sess.keep), "kept_rows_max": max(sess.keep),
                   "graph": not args.no_graph,
                   "path": FORMS[mode],
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "kernel": kernel, "achieved": round(kern_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kern_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "avg_launch_us": round(launch_us, 3),
                     "measured_copy_gbs": round(copy_gbs, 1),
                     "frac_of_measured_copy": round(kern_gbs / copy_gbs, 4),
                     "measured_read_gbs": round(read_gbs, 1),
                     "frac_of_measured_read": round(kern_gbs / read_gbs, 4),
                     "measured_gather_gbs": round(gather_gbs, 1),
                     "frac_of_measured_gather": round(kern_gbs / gather_gbs, 4),
                     "bytes_per_launch": int(bytes_launch)},
    }
    if turn_report:
        result["config"]["turns"] = wl.turns
        result["config"]["turn_append_rows"] = wl.turn_append
        result["turns"] = turn_report
    if turns and args.mt_filter > 0:
        del graphs, inputs
        torch.cuda.empty_cache()
        result["mt_filter"] = mt_filter_leg(torch, rkv, wl, args, dev, args.mt_filter)
    if not args.no_cpu_baseline:
        nproc, threads = host_threads()
        log(f"[bench] timing the oracle on the host ({threads} of {nproc} CPUs, then 1) ...")
        result["cpu_baseline"] = cpu_baseline(wl, sess, per_layer[0][2], args.cpu_budget)
        log(f"[bench] cpu baseline: {result['cpu_baseline']}")
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
