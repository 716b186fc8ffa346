"""Summarise rocprofv3 CSV output into the short text files kept in profiles/.

    python rocprof_summary.py stats <run_kernel_stats.csv> \\
        --command "<rocprofv3 command>" --workload qkv_38656 -o profiles/X.md
    python rocprof_summary.py traffic \\
        --fetch <fetch run_counter_collection.csv> --write <write ...csv> \\
        --copy-bytes 536870912 --kernel gemm_i8_kernel --source <kernel .hip> \\
        --command-fetch "..." --command-write "..." -o profiles/Y.md
    python rocprof_summary.py counters <run_counter_collection.csv> ... \\
        --kernel gemm_i8_kernel --command "..." --command "..." -o profiles/Z.md

`traffic` scales each counter by what it reads for the plain device copy of
known size recorded in the same run (FETCH_SIZE and WRITE_SIZE are in KiB per
dispatch), and records the SHA-256 of the kernel source so a reader (and
bench.py) can tell whether the figure still applies to the current kernel.
One call can launch several instantiations of a kernel (the GEMM sends its
last tile-rows to a second launch); every instantiation matching --kernel is
listed, and the per-call figure is the sum of their per-dispatch averages.
"""
from __future__ import annotations

import argparse
import collections
import csv
import hashlib
import json
import sys

COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _short(name: str) -> str:
    name = name.replace("void ", "").replace("convrot::(anonymous namespace)::", "")
    return name.split("(")[0]


def _medians(trace_csv):
    """Median dispatch duration (ns) per kernel name, from the kernel trace."""
    d = collections.defaultdict(list)
    for r in csv.DictReader(open(trace_csv)):
        d[r["Kernel_Name"]].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    return {k: sorted(v)[len(v) // 2] for k, v in d.items()}


def _bench_line(log):
    """The JSON line bench.py printed in the profiled run."""
    for line in reversed(open(log, errors="replace").read().splitlines()):
        if line.startswith('{"metric"'):
            return json.loads(line)
    return None


def stats(args):
    rows = list(csv.DictReader(open(args.csv)))
    med = _medians(args.trace) if args.trace else {}
    out = [f"# Kernel durations -- {args.workload}", "",
           "Command (run from /tmp, repository at $R):", "", "```", args.command, "```", "",
           "| kernel | calls | average (us) | median (us) | min (us) | max (us) | share |",
           "|---|---:|---:|---:|---:|---:|---:|"]
    for r in rows:
        m = med.get(r["Name"])
        out.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} | "
                   f"{'' if m is None else f'{m / 1e3:.1f}'} | "
                   f"{float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                   f"{float(r['Percentage']):.1f}% |")
    out.append("")
    bl = _bench_line(args.bench_log) if args.bench_log else None
    if bl:
        out += ["The averages include the warm-up dispatches; the medians are the steady "
                "state.  The same run's bench.py line timed each stage with HIP events "
                "between the stages (one stage can be several kernels, e.g. a GEMM and "
                "its tail launch):", ""]
        out += [f"- {k['kernel']}: {k['avg_launch_ms'] * 1e3:.1f} us per call"
                for k in bl["kernels"]]
        out.append("")
    text = "\n".join(out)
    _emit(text, args.output)


def _counter(path, counter):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def _pick(agg, needle):
    vals = [v for k, vs in agg.items() if needle in k for v in vs]
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r}")
    return sum(vals) / len(vals), len(vals)


def _per_call(agg, needle):
    """[(instantiation, dispatches, average per dispatch)] for every kernel
    matching `needle`, and the sum of the averages (one call launches each
    instantiation once)."""
    rows = [(_short(k), len(vs), sum(vs) / len(vs)) for k, vs in sorted(agg.items())
            if needle in k]
    if not rows:
        raise SystemExit(f"no dispatch of a kernel matching {needle!r}")
    return rows, sum(r[2] for r in rows)


def traffic(args):
    fetch = _counter(args.fetch, "FETCH_SIZE")
    write = _counter(args.write, "WRITE_SIZE")
    cf, _ = _pick(fetch, COPY_KERNEL)
    cw, _ = _pick(write, COPY_KERNEL)
    frows, kf = _per_call(fetch, args.kernel)
    wrows, kw = _per_call(write, args.kernel)
    sf = args.copy_bytes / (cf * 1024.0)
    sw = args.copy_bytes / (cw * 1024.0)
    rd = kf * 1024.0 * sf
    wr = kw * 1024.0 * sw
    sha = hashlib.sha256(open(args.source, "rb").read()).hexdigest()
    out = [f"# HBM traffic of `{args.kernel}` -- {args.workload}", "",
           "Commands (run from /tmp, repository at $R):", "", "```", args.command_fetch,
           args.command_write, "```", "",
           f"Calibration: the plain device copy `{COPY_KERNEL}` of {args.copy_bytes} bytes reads "
           f"FETCH_SIZE {cf:.0f} KiB and WRITE_SIZE {cw:.0f} KiB per dispatch, so the scale "
           f"factors are {sf:.4f} (fetch) and {sw:.4f} (write).", "",
           "| counter | kernel | dispatches | KiB per dispatch | scaled bytes |",
           "|---|---|---:|---:|---:|",
           *[f"| FETCH_SIZE | `{n}` | {c} | {v:.0f} | {v * 1024.0 * sf:.4g} |" for n, c, v in frows],
           *[f"| WRITE_SIZE | `{n}` | {c} | {v:.0f} | {v * 1024.0 * sw:.4g} |" for n, c, v in wrows],
           "",
           "Per call (the sum over the instantiations above):", "",
           f"traffic_bytes_per_launch: {rd + wr:.6g}",
           f"read_bytes_per_launch: {rd:.6g}",
           f"write_bytes_per_launch: {wr:.6g}",
           f"algorithmic_bytes_per_launch: {args.algorithmic_bytes:.6g}",
           f"kernel_source_sha256: {sha}", ""]
    _emit("\n".join(out), args.output)


def counters(args):
    """Average of every counter per dispatch of each kernel instantiation
    matching --kernel, over one or more counter runs, with the derived figures
    the GEMM analysis uses."""
    vals = collections.defaultdict(lambda: collections.defaultdict(list))
    durs = collections.defaultdict(list)
    for path in args.csv:
        for r in csv.DictReader(open(path)):
            if args.kernel not in r["Kernel_Name"]:
                continue
            name = _short(r["Kernel_Name"])
            vals[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
            durs[name].append(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    if not vals:
        raise SystemExit(f"no dispatch of a kernel matching {args.kernel!r}")
    out = [f"# Counters of `{args.kernel}` -- {args.workload}", "",
           "Commands (run from /tmp, repository at $R):", "", "```", *args.command, "```", ""]
    for name in sorted(vals, key=lambda n: -sum(durs[n]) / len(durs[n])):
        avg = {k: sum(v) / len(v) for k, v in vals[name].items()}
        out += [f"## `{name}`", "", "| counter | dispatches | average per dispatch |",
                "|---|---:|---:|"]
        for k in sorted(avg):
            out.append(f"| {k} | {len(vals[name][k])} | {avg[k]:.6g} |")
        out += ["", "Derived (per dispatch):", ""]
        if "TCC_EA0_RDREQ_sum" in avg:
            out.append(f"- L2 read misses to the fabric: "
                       f"{avg['TCC_EA0_RDREQ_sum'] * 128 / 1e9:.3f} GB (128-byte requests)")
        if "TCC_EA0_WRREQ_sum" in avg:
            out.append(f"- L2 write requests: {avg['TCC_EA0_WRREQ_sum'] * 64 / 1e9:.3f} GB "
                       f"(64-byte)")
        if "TCC_HIT_sum" in avg and "TCC_MISS_sum" in avg:
            h, m = avg["TCC_HIT_sum"], avg["TCC_MISS_sum"]
            out.append(f"- L2 hit rate: {100 * h / (h + m):.1f}%")
        d = sum(durs[name]) / len(durs[name])
        if "GRBM_GUI_ACTIVE" in avg:
            clk = avg["GRBM_GUI_ACTIVE"] / args.xcds / d
            out.append(f"- shader clock: {clk:.3f} GHz (GRBM_GUI_ACTIVE / {args.xcds} XCDs over "
                       f"the dispatch's {d / 1e3:.1f} us under the profiler)")
            if "SQ_VALU_MFMA_BUSY_CYCLES" in avg:
                busy = avg["SQ_VALU_MFMA_BUSY_CYCLES"] / args.simds
                out.append(f"- MFMA busy: {100 * busy / (clk * d):.1f}% of the dispatch's cycles "
                           f"per SIMD ({args.simds} SIMDs)")
        if "SQ_INSTS_VALU_MFMA_MOPS_I8" in avg:
            out.append(f"- INT8 MFMA operations: {avg['SQ_INSTS_VALU_MFMA_MOPS_I8'] * 512:.4g}")
        out.append("")
    _emit("\n".join(out), args.output)


def _emit(text, path):
    if path:
        open(path, "w").write(text)
    else:
        sys.stdout.write(text)


def main():
    p = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    sub = p.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("csv")
    s.add_argument("--command", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--trace", help="run_kernel_trace.csv of the same run (medians)")
    s.add_argument("--bench-log", help="the profiled run's output (its bench.py JSON line)")
    s.add_argument("-o", "--output")
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--source", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--algorithmic-bytes", type=float, default=0.0)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("-o", "--output")
    c = sub.add_parser("counters")
    c.add_argument("csv", nargs="+")
    c.add_argument("--kernel", required=True)
    c.add_argument("--workload", required=True)
    c.add_argument("--command", action="append", required=True)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--simds", type=int, default=1024)
    c.add_argument("-o", "--output")
    a = p.parse_args()
    {"stats": stats, "traffic": traffic, "counters": counters}[a.cmd](a)


if __name__ == "__main__":
    main()
