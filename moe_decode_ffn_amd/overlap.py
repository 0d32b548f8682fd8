"""Concurrency of the shared-expert branch with the routed branch, from a rocprofv3
kernel trace (one helper for the measurement runs: it reads rocprofv3 output and
launches nothing).

    python -m moe_decode_ffn_amd.overlap summarize --trace DIR [--trace DIR ...]
        --label NAME [--label NAME ...] --command CMD [--command CMD ...] --out FILE

The shared branch is the shared expert's own launches (gate/up with no routed jobs,
k_gate_up<..., false, ...>, and the down step k_down); the routed branch is every
other launch of the layer (router, routing, routed gate/up, down + join, join).  For
each trace the summary gives, per forward: the busy time of each branch (the union of
its kernels' [start, end) intervals), the time both branches run at the same time (the
measure of the intersection of the two unions), the share of the shared branch that
overlaps, and the hardware queues each branch's dispatches went to.
"""
from __future__ import annotations

import argparse
import csv
import glob
import os
import re
import statistics
import sys

SHARED_RE = re.compile(r"moeffn::k_gate_up<[^>]*\bfalse\b|moeffn::k_down<")
ROUTER_RE = re.compile(r"moeffn::k_router")


def read_trace(d: str) -> list[dict]:
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*kernel_trace.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no kernel_trace.csv under {d}")
    rows = [r for r in rows if "moeffn::" in r["Kernel_Name"]]
    rows.sort(key=lambda r: int(r["Start_Timestamp"]))
    return rows


def union(iv: list[tuple[int, int]]) -> list[tuple[int, int]]:
    out: list[list[int]] = []
    for a, b in sorted(iv):
        if out and a <= out[-1][1]:
            out[-1][1] = max(out[-1][1], b)
        else:
            out.append([a, b])
    return [(a, b) for a, b in out]


def measure(iv: list[tuple[int, int]]) -> int:
    return sum(b - a for a, b in iv)


def intersect(x: list[tuple[int, int]], y: list[tuple[int, int]]) -> int:
    i = j = tot = 0
    while i < len(x) and j < len(y):
        a, b = max(x[i][0], y[j][0]), min(x[i][1], y[j][1])
        if a < b:
            tot += b - a
        if x[i][1] < y[j][1]:
            i += 1
        else:
            j += 1
    return tot


def analyse(rows: list[dict]) -> dict:
    shared = [r for r in rows if SHARED_RE.search(r["Kernel_Name"])]
    main = [r for r in rows if not SHARED_RE.search(r["Kernel_Name"])]
    steps = sum(1 for r in main if ROUTER_RE.search(r["Kernel_Name"]))
    iv = lambda rs: [(int(r["Start_Timestamp"]), int(r["End_Timestamp"])) for r in rs]  # noqa: E731
    us, um = union(iv(shared)), union(iv(main))
    both = intersect(us, um)
    span = int(rows[-1]["End_Timestamp"]) - int(rows[0]["Start_Timestamp"])
    per = max(1, steps)
    kern: dict[str, list[float]] = {}
    for r in rows:
        kern.setdefault(r["Kernel_Name"], []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    return {
        "steps": steps,
        "span_us": span / 1e3 / per,
        "shared_busy_us": measure(us) / 1e3 / per,
        "main_busy_us": measure(um) / 1e3 / per,
        "overlap_us": both / 1e3 / per,
        "overlap_frac": both / measure(us) if us else 0.0,
        "queues_shared": sorted({r["Queue_Id"] for r in shared}),
        "queues_main": sorted({r["Queue_Id"] for r in main}),
        "kernels": {k: (len(v), statistics.mean(v)) for k, v in kern.items()},
    }


def one_forward(rows: list[dict]) -> list[str]:
    """The dispatches of one forward near the end of the trace: from the shared branch's
    first launch (or the router's) before the third-last router launch."""
    routers = [i for i, r in enumerate(rows) if ROUTER_RE.search(r["Kernel_Name"])]
    if len(routers) < 3:
        return []
    lo, hi = routers[-3], routers[-2]
    while lo > 0 and SHARED_RE.search(rows[lo - 1]["Kernel_Name"]):
        lo -= 1
    while hi > lo and SHARED_RE.search(rows[hi - 1]["Kernel_Name"]):
        hi -= 1
    t0 = int(rows[lo]["Start_Timestamp"])
    out = []
    for r in rows[lo:hi]:
        name = r["Kernel_Name"].split("(")[0].replace("void ", "")
        out.append(f"q{r['Queue_Id']} {(int(r['Start_Timestamp']) - t0) / 1e3:7.2f} -> "
                   f"{(int(r['End_Timestamp']) - t0) / 1e3:7.2f}  {name}")
    return out


def cmd_summarize(args) -> int:
    lines = ["# Shared-expert branch concurrency (rocprofv3 kernel traces)", "",
             "Per forward, from each dispatch's start and end timestamps: the busy time of the",
             "shared-expert launches (their union), of the routed launches, and of both at once.",
             "Times under the profiler include its per-dispatch overhead; the overlap is what the",
             "trace shows the hardware did.", ""]
    lines += ["| run | forwards | span us | shared busy us | routed busy us | both at once us | shared overlapped | queues shared / routed |",
              "|---|---|---|---|---|---|---|---|"]
    details = []
    for d, label, cmd in zip(args.trace, args.label, args.command):
        rows = read_trace(d)
        a = analyse(rows)
        a["timeline"] = one_forward(rows) if args.timeline else []
        lines.append(f"| {label} | {a['steps']} | {a['span_us']:.2f} | {a['shared_busy_us']:.2f} | "
                     f"{a['main_busy_us']:.2f} | {a['overlap_us']:.2f} | {100 * a['overlap_frac']:.1f}% | "
                     f"{','.join(a['queues_shared']) or '-'} / {','.join(a['queues_main'])} |")
        details.append((label, cmd, a))
    if args.timings:
        # layer_loop's own timing of the same runs without the profiler
        pat = re.compile(r"layer_loop (\S+) .*T=(\d+) mode=(\S+) launch=(\S+) .*: ([0-9.]+) us/forward")
        lines += ["", "Without the profiler (`" + args.timings_command + "`, host clock around the loop):", "",
                  "| workload | launch | aux us | seq us | fused us |", "|---|---|---|---|---|"]
        got: dict = {}
        with open(args.timings) as fh:
            for ln in fh:
                m = pat.search(ln)
                if m:
                    got.setdefault((m.group(1), m.group(4)), {})[m.group(3)] = float(m.group(5))
        for (wl, launch), v in got.items():
            lines.append(f"| {wl} | {launch} | {v.get('aux', 0):.1f} | {v.get('seq', 0):.1f} | {v.get('fused', 0):.1f} |")
    lines += ["", "Commands (from /tmp, one MI355X):", ""]
    for label, cmd, a in details:
        lines += [f"- {label}: `{cmd}`"]
    lines += [""]
    for label, cmd, a in details:
        if a["timeline"] and (not args.timeline_runs or label in args.timeline_runs):
            lines += [f"One forward of {label} (queue, start -> end us from its first dispatch):", ""]
            lines += [f"    {t}" for t in a["timeline"]] + [""]
    if args.kernels:
        for label, cmd, a in details:
            lines += [f"Kernels of {label} (launches, average us):", ""]
            for k, (n, m) in sorted(a["kernels"].items(), key=lambda kv: -kv[1][0] * kv[1][1]):
                lines.append(f"- `{k}`: {n}, {m:.2f}")
            lines += [""]
    lines += args.note
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines[:len(args.trace) + 9]))
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--trace", action="append", required=True)
    s.add_argument("--label", action="append", required=True)
    s.add_argument("--command", action="append", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--timings", default=None, help="layer_loop output of the same runs without the profiler")
    s.add_argument("--timings-command", default="")
    s.add_argument("--timeline", action="store_true", help="list one forward's dispatches per trace")
    s.add_argument("--timeline-runs", action="append", default=[], help="only these labels' timelines")
    s.add_argument("--kernels", action="store_true", help="list every kernel's launches and average time")
    s.add_argument("--note", action="append", default=[], help="a closing line of the summary")
    args = ap.parse_args()
    if not (len(args.trace) == len(args.label) == len(args.command)):
        raise SystemExit("one --label and --command per --trace")
    return cmd_summarize(args)


if __name__ == "__main__":
    sys.exit(main())
