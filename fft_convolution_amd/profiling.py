"""Summaries of rocprofv3 output for the files under ``profiles/``.

Three subcommands, all reading the CSV output of ``rocprofv3 --output-format csv``:

``stats``   -- per-kernel durations from a ``--kernel-trace --stats`` run:
               python -m fft_convolution_amd.profiling stats DIR --out profiles/X.md --cmd "..."

``counters`` -- the same two counters for every kernel of a run, scaled the
               same way, as a markdown table (kernel, average duration from a
               kernel-trace run, fetch and write MiB per dispatch, TB/s):
               python -m fft_convolution_amd.profiling counters --fetch DIR1 --write DIR2 \
                   --stats DIR3 --copy-bytes B --out profiles/X.md --cmd "..."

``traffic`` -- HBM bytes per launch from two ``--pmc`` runs (FETCH_SIZE, then
               WRITE_SIZE, each in KiB per dispatch) of a command that also runs
               a plain elementwise copy of known size (``bench.py
               --copy-calibration``).  Each counter is scaled by
               known bytes / the counter's reading for that copy:
               python -m fft_convolution_amd.profiling traffic --fetch DIR1 --write DIR2 \\
                   --kernel rows_kernel --copy-bytes B --workload W --out profiles/traffic_W.json

``sq``      -- instruction-level counters per kernel from one ``--pmc`` run of
               SQ_WAVES SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT
               SQ_ACTIVE_INST_LDS SQ_ACTIVE_INST_VALU SQ_WAVE_CYCLES GRBM_GUI_ACTIVE:
               per wave, VALU and LDS instructions and LDS bank-conflict cycles;
               the conflict rate (conflict cycles / LDS active cycles) and VALU
               busy (100 * SQ_ACTIVE_INST_VALU * 4 / SIMDs / (GRBM_GUI_ACTIVE / XCDs):
               1024 SIMDs on MI355X, and GRBM_GUI_ACTIVE reads the sum over its 8
               XCDs -- 3.06e6 cycles for a 176-us kernel, 8 x 382e3 at ~2.2 GHz):
               python -m fft_convolution_amd.profiling sq DIR --stats DIR2 --out profiles/sq_W.md --cmd "..."

The traffic record carries a digest of the kernel sources; ``bench.py``
reports it only while the sources are unchanged.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys


def _find(dirpath: str, suffix: str) -> list[str]:
    hits = sorted(glob.glob(os.path.join(dirpath, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit("no *%s under %s" % (suffix, dirpath))
    return hits


def kernel_stats(dirpath: str) -> list[dict]:
    rows = []
    for path in _find(dirpath, "kernel_stats.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                rows.append({"name": r["Name"], "calls": int(r["Calls"]),
                             "total_ns": float(r["TotalDurationNs"]), "avg_ns": float(r["AverageNs"]),
                             "min_ns": float(r["MinNs"]), "max_ns": float(r["MaxNs"]),
                             "pct": float(r["Percentage"])})
    rows.sort(key=lambda r: -r["total_ns"])
    return rows


def counter_values(dirpath: str, counter: str) -> dict[str, list[float]]:
    """kernel name -> list of per-dispatch values of `counter`."""
    out: dict[str, list[float]] = {}
    for path in _find(dirpath, "counter_collection.csv"):
        with open(path, newline="") as f:
            for r in csv.DictReader(f):
                if r.get("Counter_Name") != counter:
                    continue
                out.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return out


def _pick(values: dict[str, list[float]], needle: str) -> tuple[str, list[float]]:
    names = [k for k in values if needle in k]
    if not names:
        raise SystemExit("no kernel matching %r among %s" % (needle, list(values)))
    name = max(names, key=lambda k: len(values[k]))
    return name, values[name]


def cmd_stats(args):
    rows = kernel_stats(args.dir)
    lines = ["# rocprofv3 kernel summary: %s" % args.title, "",
             "Command:", "", "```", args.cmd, "```", "",
             "| kernel | calls | avg us | min us | max us | % time |", "|---|---|---|---|---|---|"]
    for r in rows:
        name = r["name"].replace("HIP_vector_type<float, 2u>", "float2").replace(
            "HIP_vector_type<double, 2u>", "double2").replace("|", "/")
        if len(name) > 110:
            name = name[:107] + "..."
        lines.append("| `%s` | %d | %.1f | %.1f | %.1f | %.1f |" % (
            name, r["calls"], r["avg_ns"] / 1e3, r["min_ns"] / 1e3, r["max_ns"] / 1e3, r["pct"]))
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def cmd_traffic(args):
    sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    from bench import kernel_sources_digest  # the same digest bench.py checks
    fetch = counter_values(args.fetch, "FETCH_SIZE")
    write = counter_values(args.write, "WRITE_SIZE")
    kname, kf = _pick(fetch, args.kernel)
    _, kw = _pick(write, args.kernel)
    cname, cf = _pick(fetch, args.copy_kernel)
    _, cw = _pick(write, args.copy_kernel)
    kib = 1024.0
    # The copy moves copy_bytes in and copy_bytes out.
    f_fetch = args.copy_bytes / (statistics.median(cf) * kib)
    f_write = args.copy_bytes / (statistics.median(cw) * kib)
    fetch_b = statistics.median(kf) * kib * f_fetch
    write_b = statistics.median(kw) * kib * f_write
    rec = {
        "workload": args.workload,
        "kernel": kname,
        "fetch_kib_per_dispatch_raw": statistics.median(kf),
        "write_kib_per_dispatch_raw": statistics.median(kw),
        "copy_kernel": cname,
        "copy_bytes_each_way": args.copy_bytes,
        "copy_fetch_kib_raw": statistics.median(cf),
        "copy_write_kib_raw": statistics.median(cw),
        "scale_fetch": f_fetch,
        "scale_write": f_write,
        "fetch_bytes_per_launch": fetch_b,
        "write_bytes_per_launch": write_b,
        "traffic_bytes_per_launch": fetch_b + write_b,
        "algorithmic_bytes_per_launch": args.algorithmic_bytes,
        "commands": args.cmd,
        "kernel_sources_sha256": kernel_sources_digest(args.workload),
    }
    with open(args.out, "w") as f:
        json.dump(rec, f, indent=1)
        f.write("\n")
    print(json.dumps(rec, indent=1))


def _scales(fetch, write, copy_kernel, copy_bytes):
    _, cf = _pick(fetch, copy_kernel)
    _, cw = _pick(write, copy_kernel)
    return copy_bytes / (statistics.median(cf) * 1024.0), copy_bytes / (statistics.median(cw) * 1024.0)


def _short(name: str) -> str:
    name = name.replace("HIP_vector_type<float, 2u>", "float2").replace("HIP_vector_type<double, 2u>", "double2")
    cut = name.find("(")
    return (name[:cut] if cut > 0 else name).replace("|", "/")


def cmd_counters(args):
    fetch = counter_values(args.fetch, "FETCH_SIZE")
    write = counter_values(args.write, "WRITE_SIZE")
    f_fetch, f_write = _scales(fetch, write, args.copy_kernel, args.copy_bytes)
    durations = {r["name"]: r["avg_ns"] for r in kernel_stats(args.stats)} if args.stats else {}
    mib = 1024.0 * 1024.0
    lines = ["# HBM traffic per kernel: %s" % args.title, "",
             "Commands (R = repository root):", "", "```"] + list(args.cmd) + ["```", "",
             "FETCH_SIZE and WRITE_SIZE are read per dispatch (KiB) and scaled by the reading of a plain "
             "elementwise copy of %d bytes each way in the same run: fetch x%.4f, write x%.4f."
             % (args.copy_bytes, f_fetch, f_write), "",
             "| kernel | dispatches | avg us | fetch MiB | write MiB | TB/s |", "|---|---|---|---|---|---|"]
    for name in sorted(fetch, key=lambda k: -statistics.median(fetch[k])):
        if args.copy_kernel in name or "copyBuffer" in name:
            continue
        fb = statistics.median(fetch[name]) * 1024.0 * f_fetch
        wb = statistics.median(write.get(name, [0.0])) * 1024.0 * f_write
        us = durations.get(name, 0.0) / 1e3
        tbs = (fb + wb) / (us * 1e-6) / 1e12 if us else 0.0
        lines.append("| `%s` | %d | %.1f | %.1f | %.1f | %.2f |" % (_short(name), len(fetch[name]), us, fb / mib,
                                                                  wb / mib, tbs))
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT", "SQ_ACTIVE_INST_LDS",
               "SQ_ACTIVE_INST_VALU", "SQ_WAVE_CYCLES", "GRBM_GUI_ACTIVE")
MI355X_SIMDS = 256 * 4
MI355X_XCDS = 8


def cmd_sq(args):
    vals = {c: counter_values(args.dir, c) for c in SQ_COUNTERS}
    durations = {r["name"]: r["avg_ns"] for r in kernel_stats(args.stats)} if args.stats else {}
    med = lambda c, k: statistics.median(vals[c][k]) if vals[c].get(k) else float("nan")
    lines = ["# LDS and VALU counters per kernel: %s" % args.title, "",
             "Commands (R = repository root):", "", "```"] + list(args.cmd) + ["```", "",
             "Per wave: instructions and LDS bank-conflict cycles (SQ_LDS_BANK_CONFLICT / SQ_WAVES). "
             "Conflict %% = SQ_LDS_BANK_CONFLICT / SQ_ACTIVE_INST_LDS. VALU busy %% = 100 * "
             "SQ_ACTIVE_INST_VALU * 4 / %d SIMDs / GRBM_GUI_ACTIVE. Medians over dispatches." % MI355X_SIMDS, "",
             "| kernel | dispatches | avg us | waves | VALU inst / wave | LDS inst / wave | "
             "conflict cycles / wave | conflict % | VALU busy % |",
             "|---|---|---|---|---|---|---|---|---|"]
    for k in sorted(vals["SQ_WAVES"], key=lambda k: -med("SQ_WAVES", k)):
        if "copyBuffer" in k or "elementwise" in k:
            continue
        waves = med("SQ_WAVES", k)
        if not waves:
            continue
        lds_act = med("SQ_ACTIVE_INST_LDS", k)
        conf = med("SQ_LDS_BANK_CONFLICT", k)
        gui = med("GRBM_GUI_ACTIVE", k)
        busy = 100.0 * med("SQ_ACTIVE_INST_VALU", k) * 4 / MI355X_SIMDS / (gui / MI355X_XCDS) if gui else float("nan")
        us = next((v for n, v in durations.items() if n == k), 0.0) / 1e3
        lines.append("| `%s` | %d | %.1f | %d | %.0f | %.1f | %.1f | %.1f | %.1f |" % (
            _short(k), len(vals["SQ_WAVES"][k]), us, waves, med("SQ_INSTS_VALU", k) / waves,
            med("SQ_INSTS_LDS", k) / waves, conf / waves, 100.0 * conf / lds_act if lds_act else 0.0, busy))
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--out")
    s.add_argument("--cmd", required=True)
    s.add_argument("--title", default="")
    s.set_defaults(fn=cmd_stats)
    c = sub.add_parser("counters")
    c.add_argument("--fetch", required=True)
    c.add_argument("--write", required=True)
    c.add_argument("--stats")
    c.add_argument("--copy-kernel", default="elementwise")
    c.add_argument("--copy-bytes", type=int, required=True)
    c.add_argument("--title", default="")
    c.add_argument("--out")
    c.add_argument("--cmd", nargs="*", default=[])
    c.set_defaults(fn=cmd_counters)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--copy-kernel", default="elementwise")
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--algorithmic-bytes", type=int, required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--out", required=True)
    t.add_argument("--cmd", nargs="*", default=[])
    t.set_defaults(fn=cmd_traffic)
    q = sub.add_parser("sq")
    q.add_argument("dir")
    q.add_argument("--stats")
    q.add_argument("--title", default="")
    q.add_argument("--out")
    q.add_argument("--cmd", nargs="*", default=[])
    q.set_defaults(fn=cmd_sq)
    args = ap.parse_args(argv)
    args.fn(args)


if __name__ == "__main__":
    main()
