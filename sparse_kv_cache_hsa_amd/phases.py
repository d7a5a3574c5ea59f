"""Per-phase timing table of the fused decode kernel.

Runs a workload's decode steps as HIP-graph replays (the benchmark's launch
sequence) on the phase-timing build of the library (librkv_timing.so, built
with ``python -m sparse_kv_cache_hsa_amd.build --timing``), whose fused decode
kernel writes a constant-rate clock stamp at every phase boundary of every
block (include/rkv.h, RKV_TRACE_SLOTS).  Prints a markdown table of the
phases' mean durations over the blocks of every layer of the last step, the
per-XCC stream and block times, and the launch spans.

    python -m sparse_kv_cache_hsa_amd.phases [--workload W] [--steps N]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import sys

import numpy as np
import torch

from . import build, rkv, workloads
from .session import Session

STREAM_WAVES = 8
PHASES = [("q + new row", 0, 1), ("channels", 1, 2), ("staging + fold", 2, 3),
          ("page bounds", 3, 24), ("page top-k", 24, 4), ("stream setup", 4, 5)]


def wall_clock_khz(dev: int = 0) -> int:
    hip = ctypes.CDLL("libamdhip64.so")
    v = ctypes.c_int()
    # hipDeviceAttributeWallClockRate (AMD-specific attribute 10017)
    rc = hip.hipDeviceGetAttribute(ctypes.byref(v), 10017, dev)
    if rc != 0 or v.value <= 0:
        raise RuntimeError(f"hipDeviceGetAttribute(WallClockRate) failed: {rc}")
    return v.value


def table(trace: np.ndarray, khz: int) -> dict:
    """trace [layers, blocks, RKV_TRACE_SLOTS] int64 -> phase statistics in us."""
    us = 1e3 / khz
    t = trace.astype(np.float64)
    t0 = t[:, :, 0].min(axis=1, keepdims=True)          # launch start per layer
    rel = (t - t0[..., None]) * us
    rel[:, :, 23] = trace[:, :, 23]                      # XCC id, not a time
    res = {"phases_mean_us": {}, "per_xcc": {}, "launch_span_us": {}}
    for name, a, b in PHASES:
        res["phases_mean_us"][name] = float((rel[:, :, b] - rel[:, :, a]).mean())
    # the decode kernel streams on its first STREAM_WAVES waves; the others
    # stamp their (empty) stream's end at once
    wave_end = rel[:, :, 6:6 + STREAM_WAVES]
    res["phases_mean_us"]["stream, first wave"] = float((wave_end.min(2) - rel[:, :, 5]).mean())
    res["phases_mean_us"]["stream, last wave"] = float((wave_end.max(2) - rel[:, :, 5]).mean())
    res["phases_mean_us"]["merge + outputs"] = float((rel[:, :, 22] - wave_end.max(2)).mean())
    res["phases_mean_us"]["block start offset"] = float(rel[:, :, 0].mean())
    res["phases_mean_us"]["block total"] = float((rel[:, :, 22] - rel[:, :, 0]).mean())
    res["phases_mean_us"]["selection (start to stream)"] = float(
        (rel[:, :, 5] - rel[:, :, 0]).mean())
    span = rel[:, :, 22].max(1)
    res["launch_span_us"] = {"mean": float(span.mean()), "min": float(span.min()),
                             "max": float(span.max())}
    xcc = trace[:, :, 23]
    for x in sorted(set(xcc.ravel().tolist())):
        m = xcc == x
        res["per_xcc"][int(x)] = {
            "blocks": int(m.sum()),
            "stream_last_wave_us": float((wave_end.max(2) - rel[:, :, 5])[m].mean()),
            "block_end_us": float(rel[:, :, 22][m].mean()),
        }
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--workload", default="llama8b-32layer-b32-ctx16k-32k")
    ap.add_argument("--steps", type=int, default=8)
    ap.add_argument("--json", default="")
    args = ap.parse_args()
    lib = rkv.load_library(path=build.LIB_TIMING_PATH)
    wl = workloads.ALL[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    sess = Session(wl, extra_rows=args.steps, device=dev)
    mode = rkv.decode_mode(sess.g, sess.B, sess.P, sess.max_pages, wl.k2, wl.k1,
                           rkv.RKV_BF16 if wl.dtype.itemsize == 2 else rkv.RKV_F32)
    if mode != rkv.RKV_FORM_FUSED:
        sys.exit(f"{wl.name} does not run the one-block-per-unit fused kernel")
    ws = sess.evict_workspace() if wl.evicts else None
    for l in range(sess.n_layers):
        sess.prefill_layer(l, ws=ws)
    del ws
    torch.cuda.synchronize()
    blocks = sess.B * sess.Hkv
    trace = torch.zeros((sess.n_layers, blocks, rkv.RKV_TRACE_SLOTS), dtype=torch.int64,
                        device=dev)
    sess.opts = [rkv.make_opts(trace=trace[l]) for l in range(sess.n_layers)]
    inputs = sess.make_inputs(args.steps)
    graphs = []
    for s in range(args.steps):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            sess.step(inputs[s])
        graphs.append(g)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    for s in range(args.steps - 1):
        graphs[s].replay()
    torch.cuda.synchronize()
    e0.record()
    graphs[-1].replay()
    e1.record()
    torch.cuda.synchronize()
    step_us = e0.elapsed_time(e1) * 1e3
    res = table(trace.cpu().numpy(), wall_clock_khz())
    res["step_us_events"] = step_us
    res["launch_us_events"] = step_us / sess.n_layers
    res["workload"] = wl.name
    res["build_id"] = lib.rkv_build_id().decode()
    print(f"| phase | mean us per block |\n|---|---|")
    for k, v in res["phases_mean_us"].items():
        print(f"| {k} | {v:.2f} |")
    print(f"\nlaunch span from the stamps: mean {res['launch_span_us']['mean']:.2f} us "
          f"(min {res['launch_span_us']['min']:.2f}, max {res['launch_span_us']['max']:.2f}); "
          f"events: {res['launch_us_events']:.2f} us per launch")
    print("\n| XCC | blocks | stream, last wave (us) | block end (us) |\n|---|---|---|---|")
    for x, r in res["per_xcc"].items():
        print(f"| {x} | {r['blocks']} | {r['stream_last_wave_us']:.2f} | {r['block_end_us']:.2f} |")
    if args.json:
        with open(args.json, "w") as f:
            json.dump(res, f, indent=1)


if __name__ == "__main__":
    main()
