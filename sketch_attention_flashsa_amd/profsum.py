"""Summaries of rocprofv3 CSV output for the streaming kernel.

    python -m sketch_attention_flashsa_amd.profsum stats DIR [--kernel NAME] [--cmd TEXT]
    python -m sketch_attention_flashsa_amd.profsum traffic --fetch DIR --write DIR \\
        --copy-fetch DIR --copy-write DIR --copy-bytes N --kernel NAME --alg-bytes A \\
        [--cmd TEXT] [--json OUT]

``stats`` reads the ``*kernel_stats.csv`` that ``rocprofv3 --kernel-trace
--stats --output-format csv -d DIR`` writes and prints a markdown table of
every kernel (calls, average / min / max duration).

``trace`` reads the ``*kernel_trace.csv`` of the same run and splits one
kernel's dispatches, in dispatch order, into the benchmark's legs: the first
``--warmup`` are warm-up launches, the next ``--timed`` the timed ones, the
rest (if any) later legs; it prints each leg's count, average, median, min
and max duration, so the timed average can be recomputed from the trace.

``counters`` reads one ``--pmc`` run and prints, for every counter it
holds, the per-dispatch value of one kernel (summed over the rows a dispatch
reports, averaged over its dispatches).

``traffic`` reads four ``--pmc`` runs (``*counter_collection.csv``): the
kernel's FETCH_SIZE and WRITE_SIZE runs, and the same two counters for a
plain copy kernel that reads and writes ``copy_bytes`` each.  The counters
are in KiB per dispatch; the copy kernel gives the scale factor from counter
units to bytes (bytes / counter), applied to the kernel's per-dispatch
average.  With ``--json`` it writes the figure that bench.py reports as
``roofline.traffic``, tagged with the hash of the kernel sources the counters
were taken on.
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys


def _rows(pattern_dir: str, suffix: str) -> list[dict]:
    files = sorted(glob.glob(os.path.join(pattern_dir, "**", f"*{suffix}"), recursive=True))
    if not files:
        raise SystemExit(f"no *{suffix} under {pattern_dir}")
    out = []
    for f in files:
        with open(f, newline="") as fh:
            out.extend(csv.DictReader(fh))
    return out


def _pick(row: dict, *names):
    for n in names:
        if n in row:
            return row[n]
    raise KeyError(f"none of {names} in {list(row)}")


def kernel_stats(d: str) -> list[dict]:
    """[{name, calls, avg_us, min_us, max_us, total_ms, pct}] sorted by total time."""
    out = []
    for r in _rows(d, "kernel_stats.csv"):
        out.append({
            "name": _pick(r, "Name", "KERNEL_NAME", "Kernel_Name"),
            "calls": int(_pick(r, "Calls", "CALLS")),
            "avg_us": float(_pick(r, "AverageNs", "AVERAGE_NS")) / 1e3,
            "min_us": float(_pick(r, "MinNs", "MIN_NS")) / 1e3,
            "max_us": float(_pick(r, "MaxNs", "MAX_NS")) / 1e3,
            "total_ms": float(_pick(r, "TotalDurationNs", "TOTAL_DURATION_NS")) / 1e6,
            "pct": float(_pick(r, "Percentage", "PERCENTAGE")),
        })
    out.sort(key=lambda x: -x["total_ms"])
    return out


def counter_avg(d: str, counter: str, kernel: str) -> tuple[float, int]:
    """Average over dispatches of kernel (substring match) of the counter,
    summed over the rows a dispatch reports; returns (average, dispatches)."""
    per = {}
    for r in _rows(d, "counter_collection.csv"):
        if counter != _pick(r, "Counter_Name", "COUNTER_NAME"):
            continue
        if kernel not in _pick(r, "Kernel_Name", "KERNEL_NAME"):
            continue
        k = _pick(r, "Dispatch_Id", "DISPATCH_ID")
        per[k] = per.get(k, 0.0) + float(_pick(r, "Counter_Value", "COUNTER_VALUE"))
    if not per:
        raise SystemExit(f"no {counter} rows for a kernel matching {kernel!r} under {d}")
    return statistics.fmean(per.values()), len(per)


def all_counters(d: str, kernel: str) -> dict:
    """{counter: (per-dispatch average, dispatches)} for kernel (substring match)."""
    per = {}
    for r in _rows(d, "counter_collection.csv"):
        if kernel not in _pick(r, "Kernel_Name", "KERNEL_NAME"):
            continue
        name = _pick(r, "Counter_Name", "COUNTER_NAME")
        k = _pick(r, "Dispatch_Id", "DISPATCH_ID")
        per.setdefault(name, {})
        per[name][k] = per[name].get(k, 0.0) + float(_pick(r, "Counter_Value", "COUNTER_VALUE"))
    if not per:
        raise SystemExit(f"no counters for a kernel matching {kernel!r} under {d}")
    return {n: (statistics.fmean(v.values()), len(v)) for n, v in sorted(per.items())}


def _counters_main(a) -> None:
    res = all_counters(a.dir, a.kernel)
    if a.cmd:
        print(f"Command: `{a.cmd}`\n")
    print(f"| counter ({a.kernel}) | per dispatch | dispatches |")
    print("|---|---:|---:|")
    for n, (v, k) in res.items():
        print(f"| {n} | {v:.6g} | {k} |")


def kernel_durations(d: str, kernel: str) -> list[float]:
    """Durations (us) of every dispatch of kernel (substring match), in
    dispatch order, from the kernel trace."""
    rows = []
    for r in _rows(d, "kernel_trace.csv"):
        if kernel not in _pick(r, "Kernel_Name", "KERNEL_NAME"):
            continue
        start = int(_pick(r, "Start_Timestamp", "START_TIMESTAMP"))
        end = int(_pick(r, "End_Timestamp", "END_TIMESTAMP"))
        rows.append((int(_pick(r, "Dispatch_Id", "DISPATCH_ID")), (end - start) / 1e3))
    if not rows:
        raise SystemExit(f"no dispatch of a kernel matching {kernel!r} under {d}")
    rows.sort()
    return [us for _, us in rows]


def _trace_main(a) -> None:
    us = kernel_durations(a.dir, a.kernel)
    legs = [("warm-up", us[:a.warmup]), ("timed", us[a.warmup:a.warmup + a.timed]),
            ("after the timed steps", us[a.warmup + a.timed:])]
    if a.cmd:
        print(f"Command: `{a.cmd}`\n")
    print(f"Dispatches of `{a.kernel}`: {len(us)}\n")
    print("| leg | launches | avg (us) | median (us) | min (us) | max (us) |")
    print("|---|---:|---:|---:|---:|---:|")
    for name, xs in legs:
        if xs:
            print(f"| {name} | {len(xs)} | {statistics.fmean(xs):.1f} | {statistics.median(xs):.1f} | "
                  f"{min(xs):.1f} | {max(xs):.1f} |")


def _stats_main(a) -> None:
    rows = kernel_stats(a.dir)
    if a.cmd:
        print(f"Command: `{a.cmd}`\n")
    print("| kernel | calls | avg (us) | min (us) | max (us) | total (ms) | % |")
    print("|---|---:|---:|---:|---:|---:|---:|")
    for r in rows:
        name = r["name"] if len(r["name"]) < 120 else r["name"][:117] + "..."
        mark = "**" if a.kernel and a.kernel in r["name"] else ""
        print(f"| {mark}{name}{mark} | {r['calls']} | {r['avg_us']:.1f} | {r['min_us']:.1f} | {r['max_us']:.1f} | "
              f"{r['total_ms']:.3f} | {r['pct']:.1f} |")


def _traffic_main(a) -> None:
    f_k, n_fk = counter_avg(a.fetch, "FETCH_SIZE", a.kernel)
    w_k, n_wk = counter_avg(a.write, "WRITE_SIZE", a.kernel)
    f_c, _ = counter_avg(a.copy_fetch, "FETCH_SIZE", a.copy_kernel)
    w_c, _ = counter_avg(a.copy_write, "WRITE_SIZE", a.copy_kernel)
    scale_f = a.copy_bytes / f_c      # bytes per counter unit, reads
    scale_w = a.copy_bytes / w_c      # bytes per counter unit, writes
    rd, wr = f_k * scale_f, w_k * scale_w
    total = rd + wr
    res = {
        "kernel": a.kernel,
        "fetch_size_per_dispatch": f_k,
        "write_size_per_dispatch": w_k,
        "dispatches": [n_fk, n_wk],
        "copy_kernel": a.copy_kernel,
        "copy_bytes": a.copy_bytes,
        "copy_fetch_size": f_c,
        "copy_write_size": w_c,
        "bytes_per_unit_fetch": scale_f,
        "bytes_per_unit_write": scale_w,
        "hbm_read_bytes_per_launch": rd,
        "hbm_write_bytes_per_launch": wr,
        "hbm_bytes_per_launch": total,
        "algorithmic_bytes_per_launch": a.alg_bytes,
        "traffic_over_algorithmic": total / a.alg_bytes if a.alg_bytes else None,
        "command": a.cmd,
    }
    if a.json:
        from .build import KERNEL_SOURCES, sources_hash
        res["kernel_sources"] = list(KERNEL_SOURCES.get(a.kernel, ()))
        res["kernel_sources_sha256_16"] = sources_hash(KERNEL_SOURCES.get(a.kernel))
        with open(a.json, "w") as fh:
            json.dump(res, fh, indent=1)
            fh.write("\n")
    print(json.dumps(res, indent=1))


def main(argv=None) -> None:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="what", required=True)
    s = sub.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--kernel", default="")
    s.add_argument("--cmd", default="")
    tr = sub.add_parser("trace")
    tr.add_argument("dir")
    tr.add_argument("--kernel", required=True)
    tr.add_argument("--warmup", type=int, required=True)
    tr.add_argument("--timed", type=int, required=True)
    tr.add_argument("--cmd", default="")
    c = sub.add_parser("counters")
    c.add_argument("dir")
    c.add_argument("--kernel", required=True)
    c.add_argument("--cmd", default="")
    t = sub.add_parser("traffic")
    for n in ("fetch", "write", "copy-fetch", "copy-write"):
        t.add_argument(f"--{n}", required=True)
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--copy-kernel", default="neg")
    t.add_argument("--kernel", required=True)
    t.add_argument("--alg-bytes", type=float, default=0.0)
    t.add_argument("--cmd", default="")
    t.add_argument("--json", default="")
    a = ap.parse_args(argv)
    {"stats": _stats_main, "trace": _trace_main, "counters": _counters_main, "traffic": _traffic_main}[a.what](a)


if __name__ == "__main__":
    sys.exit(main())
