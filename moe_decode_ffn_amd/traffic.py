"""HBM traffic of one kernel from rocprofv3 counters, calibrated on a plain copy.

Two helpers for the measurement runs (they read rocprofv3 output; nothing
here launches a kernel of the layer):

    python -m moe_decode_ffn_amd.traffic copy --mib 1024
        A plain device copy (read N MiB, write N MiB) several times, to be run
        under `rocprofv3 --pmc FETCH_SIZE` and `--pmc WRITE_SIZE`: what the
        counters report for known bytes gives the scale factors.

    python -m moe_decode_ffn_amd.traffic counters --dir DIR [--dir DIR ...] --kernel REGEX \\
        --workload NAME --out FILE [--command CMD ...]
        Per-dispatch means of the shader counters found under the directories (SQ_*),
        with instructions per wave and the share of wave cycles issuing or waiting.

    python -m moe_decode_ffn_amd.traffic kernels --dir DIR --title TEXT --command CMD \\
        --bench-json FILE --out profiles/kernels_<workload>.md
        The per-kernel table of a `rocprofv3 --kernel-trace --stats` run (calls, average,
        minimum and maximum duration), with the kernel source hash and the step time and
        used-expert count bench.py printed under the profiler.

    python -m moe_decode_ffn_amd.traffic summarize --fetch DIR --write DIR \\
        --cal-fetch DIR --cal-write DIR --cal-mib N --kernel REGEX \\
        --workload NAME --shared-mode MODE --kernel-id ID --out profiles/traffic_<workload>.md
        [--extra DIR ...]
        Averages FETCH_SIZE and WRITE_SIZE (KiB per dispatch) over the
        dispatches of the kernel, scales each by the copy's factor, and writes
        a short summary whose fenced `traffic` block bench.py reads
        (hbm_bytes_per_launch, valid only for the kernel sources it names).
        --extra adds the per-dispatch means of any other counters found in
        those directories (hit counts, MFMA busy cycles ...).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def kernel_source_hash() -> str:
    """Hash of the HIP sources (the same definition bench.py uses)."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "moe_decode_ffn_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def read_counters(d: str) -> list[dict]:
    """Rows of every counter_collection.csv under d."""
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit(f"no counter_collection.csv under {d}")
    return rows


def per_dispatch(rows: list[dict], kernel_re: str) -> dict[str, list[float]]:
    """counter name -> list of per-dispatch values for kernels matching kernel_re."""
    pat = re.compile(kernel_re)
    acc: dict[tuple, float] = {}
    for r in rows:
        name = r.get("Kernel_Name", "")
        if not pat.search(name):
            continue
        key = (r["Counter_Name"], r.get("Dispatch_Id", r.get("Correlation_Id", "")))
        acc[key] = acc.get(key, 0.0) + float(r["Counter_Value"])
    out: dict[str, list[float]] = {}
    for (cname, _), v in acc.items():
        out.setdefault(cname, []).append(v)
    return out


def one(rows, kernel_re, counter) -> tuple[float, int]:
    vals = per_dispatch(rows, kernel_re).get(counter)
    if not vals:
        raise SystemExit(f"counter {counter} not found for kernels matching {kernel_re!r}")
    return statistics.mean(vals), len(vals)


def cmd_copy(args) -> int:
    import torch
    n = args.mib * (1 << 20) // 4
    src = torch.randn(n, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(args.reps):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(f"copy: {args.reps} x {args.mib} MiB read + {args.mib} MiB written", flush=True)
    return 0


def cmd_summarize(args) -> int:
    copy_re = "vectorized_elementwise_kernel.*MulFunctor"
    cal_bytes = args.cal_mib * (1 << 20)
    cf, _ = one(read_counters(args.cal_fetch), copy_re, "FETCH_SIZE")
    cw, _ = one(read_counters(args.cal_write), copy_re, "WRITE_SIZE")
    f_fetch = cal_bytes / (cf * 1024.0)
    f_write = cal_bytes / (cw * 1024.0)
    kf, nf = one(read_counters(args.fetch), args.kernel, "FETCH_SIZE")
    kw, nw = one(read_counters(args.write), args.kernel, "WRITE_SIZE")
    fetch_b = kf * 1024.0 * f_fetch
    write_b = kw * 1024.0 * f_write
    extra = {}
    for d in args.extra or []:
        for cname, vals in per_dispatch(read_counters(d), args.kernel).items():
            extra[cname] = statistics.mean(vals)
    lines = [
        f"# HBM traffic: `{args.kernel}`, workload {args.workload}",
        "",
        "Counters per dispatch of the kernel (rocprofv3 --pmc, one counter set per run), each",
        "scaled by what the same counter reads for a plain copy of known size.",
        "",
        "Commands (from the repository root, one MI355X):",
        "",
        "```",
    ]
    lines += [c for c in (args.command or [])]
    lines += [
        "```",
        "",
        "| quantity | value |",
        "|---|---|",
        f"| copy calibration | {args.cal_mib} MiB read + written; FETCH_SIZE {cf:.0f} KiB, WRITE_SIZE {cw:.0f} KiB |",
        f"| scale factors | fetch {f_fetch:.4f}, write {f_write:.4f} |",
        f"| dispatches measured | fetch {nf}, write {nw} |",
        f"| FETCH_SIZE per dispatch | {kf:.0f} KiB -> {fetch_b / 1e6:.3f} MB |",
        f"| WRITE_SIZE per dispatch | {kw:.0f} KiB -> {write_b / 1e6:.3f} MB |",
        f"| HBM bytes per dispatch | {(fetch_b + write_b) / 1e6:.3f} MB |",
    ]
    for cname, v in sorted(extra.items()):
        lines.append(f"| {cname} (mean per dispatch) | {v:.6g} |")
    lines += [
        "",
        "```traffic",
        f"workload: {args.workload}",
        f"shared_mode: {args.shared_mode}",
        f"kernel: {args.kernel}",
        f"kernel_id: {args.kernel_id}",
        f"kernel_source_hash: {kernel_source_hash()}",
        f"hbm_bytes_per_launch: {int(round(fetch_b + write_b))}",
        f"fetch_bytes_per_launch: {int(round(fetch_b))}",
        f"write_bytes_per_launch: {int(round(write_b))}",
        "```",
        "",
    ]
    os.makedirs(os.path.dirname(os.path.abspath(args.out)), exist_ok=True)
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def cmd_counters(args) -> int:
    """Per-dispatch means of the counters found under each --dir for one kernel, and the
    ratios that say what bounds it: VALU instructions and cycles per wave, the share of a
    wave's cycles spent issuing VALU work or waiting."""
    vals: dict[str, float] = {}
    n = 0
    for d in args.dir:
        for cname, v in per_dispatch(read_counters(d), args.kernel).items():
            vals[cname] = statistics.mean(v)
            n = max(n, len(v))
    lines = [f"# Shader counters: `{args.kernel}`, workload {args.workload}", "",
             "Means per dispatch of the kernel (rocprofv3 --pmc, at most 8 SQ counters a run).", "",
             "Commands (from /tmp, one MI355X):", "", "```"] + (args.command or []) + ["```", "",
             "| counter | mean per dispatch |", "|---|---|"]
    for cname, v in sorted(vals.items()):
        lines.append(f"| {cname} | {v:.6g} |")
    w, wc = vals.get("SQ_WAVES"), vals.get("SQ_WAVE_CYCLES")
    ratios = []
    if w:
        for c in ("SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_VMEM_RD", "SQ_INSTS_LDS", "SQ_INSTS_SMEM"):
            if c in vals:
                ratios.append((f"{c} per wave", vals[c] / w))
        ratios.append(("SQ_WAVE_CYCLES per wave", (wc or 0) / w))
    if wc:
        for c in ("SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_ANY", "SQ_ACTIVE_INST_VMEM", "SQ_ACTIVE_INST_LDS",
                  "SQ_ACTIVE_INST_SCA", "SQ_WAIT_ANY", "SQ_WAIT_INST_ANY"):
            if c in vals:
                ratios.append((f"{c} / SQ_WAVE_CYCLES", vals[c] / wc))
    if ratios:
        lines += ["", "| ratio | value |", "|---|---|"] + [f"| {k} | {v:.4g} |" for k, v in ratios]
    lines += ["", f"Dispatches: {n}; kernel source hash `{kernel_source_hash()}`.", ""]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def cmd_kernels(args) -> int:
    """Kernel table of a rocprofv3 --stats run (its kernel_stats.csv)."""
    files = glob.glob(os.path.join(args.dir, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {args.dir}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    rows = [r for r in rows if "moeffn::" in r["Name"]]
    rows.sort(key=lambda r: -float(r["TotalDurationNs"]))
    bench = {}
    if args.bench_json and os.path.exists(args.bench_json):
        with open(args.bench_json) as fh:
            for ln in fh:
                if ln.strip().startswith("{"):
                    bench = __import__("json").loads(ln)
    mode = bench.get("config", {}).get("shared_mode", "?")
    lines = [f"# Kernel trace: {args.title}", "", "Command (run from the repository root on one MI355X):", "",
             "```", args.command, "```", "",
             f"Kernel source hash: `{kernel_source_hash()}`; shared-expert mode: {mode}.",
             "Calls include warm-up, the timed steps and the event-timed pass of bench.py.", "",
             "| kernel | calls | avg us | min us | max us |", "|---|---|---|---|---|"]
    tot = 0.0
    for r in rows:
        name = r["Name"].replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "").replace("moeffn::", "")
        avg = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{name}` | {r['Calls']} | {avg:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
        tot += avg
    lines += ["", f"Sum of per-launch averages: {tot:.2f} us (a kernel launched more than once per step, "
                  "or not every step, counts once here)."]
    if bench:
        lines.append(f"bench.py under the profiler: {bench['ms_per_step'] * 1e3:.2f} us/step, "
                     f"{bench.get('unique_experts_per_step', 0):.1f} used experts per step.")
    lines += ["(The profiler adds dispatch overhead per launch to the step time, and its own signals to",
              "every dispatch, so the HIP-event kernel times bench.py prints under it are inflated; the",
              "durations above are the profiler's own.  Run without the profiler, bench.py times each",
              "kernel with HIP events in its dispatch; those are what its roofline uses.)", ""]
    with open(args.out, "w") as fh:
        fh.write("\n".join(lines))
    print("\n".join(lines))
    return 0


def read_summary(path: str) -> dict | None:
    """The fenced `traffic` block of a summary written by summarize, or None."""
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"```traffic\n(.*?)```", text, re.S)
    if not m:
        return None
    rec = {}
    for line in m.group(1).strip().splitlines():
        k, _, v = line.partition(":")
        v = v.strip()
        rec[k.strip()] = int(v) if v.isdigit() else v
    return rec


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    c = sub.add_parser("copy")
    c.add_argument("--mib", type=int, default=1024)
    c.add_argument("--reps", type=int, default=5)
    s = sub.add_parser("summarize")
    for a in ("--fetch", "--write", "--cal-fetch", "--cal-write", "--kernel", "--workload", "--out"):
        s.add_argument(a, required=True)
    s.add_argument("--cal-mib", type=int, required=True)
    s.add_argument("--shared-mode", required=True, help="aux, seq or fused: the bench mode measured")
    s.add_argument("--kernel-id", required=True,
                   help="the profiling id of the kernel (moe_ffn_kernel_id name, e.g. gate_up, gg_gate_up)")
    s.add_argument("--extra", action="append")
    s.add_argument("--command", action="append", help="a command line to record in the summary")
    kt = sub.add_parser("kernels")
    kt.add_argument("--dir", required=True)
    kt.add_argument("--title", required=True)
    kt.add_argument("--command", required=True)
    kt.add_argument("--bench-json", default=None)
    kt.add_argument("--out", required=True)
    k = sub.add_parser("counters")
    k.add_argument("--dir", action="append", required=True)
    k.add_argument("--kernel", required=True)
    k.add_argument("--workload", required=True)
    k.add_argument("--out", required=True)
    k.add_argument("--command", action="append")
    args = ap.parse_args(argv)
    return {"copy": cmd_copy, "summarize": cmd_summarize, "counters": cmd_counters,
            "kernels": cmd_kernels}[args.cmd](args)


if __name__ == "__main__":
    sys.exit(main())
