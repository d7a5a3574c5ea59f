"""Summaries of rocprofv3 CSV output for the files kept under profiles/.

Three commands:

  stats     kernel time table from a ``--kernel-trace --stats`` run
            (``*_kernel_stats.csv``), restricted to the heaviest kernels.
  counters  HBM traffic per launch of one kernel from two ``--pmc`` runs
            (FETCH_SIZE, WRITE_SIZE; KiB per dispatch), each scaled by what the
            same counter reads for a plain device copy of known size, written
            as JSON together with the library build id, so that a reader can
            tell when the kernel has changed since the counters were taken.
  pmc       the mean per dispatch of every counter of one or more ``--pmc``
            runs, over the dispatches of one kernel, as JSON.
"""
from __future__ import annotations

import argparse
import csv
import json
import re
import sys


def _short(name: str) -> str:
    m = re.search(r"rkv::\(anonymous namespace\)::(\w+)(<[^(]*>)?", name)
    if m:
        return m.group(1) + (m.group(2) or "")
    return name if len(name) <= 60 else name[:57] + "..."


def stats_table(path: str, top: int = 12, match: str = "") -> str:
    rows = [r for r in csv.DictReader(open(path)) if match in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    out = [f"{'kernel':52s} {'calls':>7s} {'avg us':>10s} {'min us':>9s} {'max us':>9s} {'share':>7s}"]
    for r in rows[:top]:
        out.append(f"{_short(r['Name'])[:52]:52s} {int(r['Calls']):7d} "
                   f"{float(r['AverageNs']) / 1e3:10.2f} {float(r['MinNs']) / 1e3:9.2f} "
                   f"{float(r['MaxNs']) / 1e3:9.2f} {float(r['Percentage']):6.2f}%")
    return "\n".join(out)


def _per_dispatch(path: str, counter: str, match) -> list[float]:
    vals = []
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter and match(r):
            vals.append(float(r["Counter_Value"]))
    return vals


def counters(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, copy_bytes, kernel):
    is_kernel = lambda r: kernel in r["Kernel_Name"]
    # The copy probe's own dispatches are the large ones; small blits of the
    # runtime are skipped by size.
    is_copy = lambda r: "copyBuffer" in r["Kernel_Name"] and float(r["Counter_Value"]) > 1024

    def avg(v):
        if not v:
            raise SystemExit("no matching dispatches")
        return sum(v) / len(v)

    f_kib = _per_dispatch(fetch_csv, "FETCH_SIZE", is_kernel)
    w_kib = _per_dispatch(write_csv, "WRITE_SIZE", is_kernel)
    cf = avg(_per_dispatch(copy_fetch_csv, "FETCH_SIZE", is_copy))
    cw = avg(_per_dispatch(copy_write_csv, "WRITE_SIZE", is_copy))
    f_scale = copy_bytes / (cf * 1024.0)
    w_scale = copy_bytes / (cw * 1024.0)
    fetch_b = avg(f_kib) * 1024.0 * f_scale
    write_b = avg(w_kib) * 1024.0 * w_scale
    return {
        "kernel": kernel,
        "dispatches": [len(f_kib), len(w_kib)],
        "fetch_kib_per_dispatch": round(avg(f_kib), 1),
        "write_kib_per_dispatch": round(avg(w_kib), 1),
        "copy_bytes": copy_bytes,
        "copy_fetch_kib": round(cf, 1),
        "copy_write_kib": round(cw, 1),
        "fetch_scale": round(f_scale, 5),
        "write_scale": round(w_scale, 5),
        "fetch_bytes_per_launch": int(fetch_b),
        "write_bytes_per_launch": int(write_b),
        "traffic_bytes_per_launch": int(fetch_b + write_b),
    }


def pmc_means(paths, kernel):
    """{counter: mean value per dispatch} over the dispatches whose kernel
    name contains `kernel`, and the dispatch count of each counter."""
    sums, counts = {}, {}
    for path in paths:
        for r in csv.DictReader(open(path)):
            if kernel not in r["Kernel_Name"]:
                continue
            c = r["Counter_Name"]
            sums[c] = sums.get(c, 0.0) + float(r["Counter_Value"])
            counts[c] = counts.get(c, 0) + 1
    if not sums:
        raise SystemExit("no matching dispatches")
    return ({c: round(sums[c] / counts[c], 3) for c in sorted(sums)},
            {c: counts[c] for c in sorted(counts)})


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--match", default="", help="only kernels whose name contains this")
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--copy-fetch", required=True)
    c.add_argument("--copy-write", required=True)
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--kernel", required=True)
    c.add_argument("--build-id", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--commands", nargs="+", required=True)
    m = sub.add_parser("pmc")
    m.add_argument("csv", nargs="+")
    m.add_argument("--kernel", required=True)
    m.add_argument("--build-id", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--commands", nargs="+", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "stats":
        print(stats_table(a.csv, a.top, a.match))
        return
    if a.cmd == "pmc":
        means, counts = pmc_means(a.csv, a.kernel)
        json.dump({"build_id": a.build_id, "workload": a.workload, "kernel": a.kernel,
                   "mean_per_dispatch": means, "dispatches": counts, "commands": a.commands},
                  sys.stdout, indent=1)
        print()
        return
    res = counters(a.fetch, a.write, a.copy_fetch, a.copy_write, a.copy_bytes, a.kernel)
    res = {"build_id": a.build_id, "workload": a.workload, **res, "commands": a.commands}
    json.dump(res, sys.stdout, indent=1)
    print()


if __name__ == "__main__":
    main()
