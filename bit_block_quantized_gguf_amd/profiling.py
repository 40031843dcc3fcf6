"""Summaries of rocprofv3 output for the committed profile records.

Reads the CSV files rocprofv3 writes (``--kernel-trace --stats`` and
``--pmc``) and prints or writes short summaries: per-kernel dispatch counts
and durations, optionally restricted to one grid size (several launches of
one kernel template with different shapes share a name), and HBM traffic per
dispatch from the FETCH_SIZE / WRITE_SIZE counters, scaled by the reading the
same counter gives for a plain device copy of known size.

    python -m bit_block_quantized_gguf_amd.profiling trace DIR [--kernel SUBSTR] [--grid N]
    python -m bit_block_quantized_gguf_amd.profiling calls DIR --start SUBSTR[|SUBSTR...] [--include SUBSTR]
    python -m bit_block_quantized_gguf_amd.profiling traffic --fetch DIR --write DIR \
        --kernel SUBSTR --grid N --calib-kernel SUBSTR --calib-bytes B \
        --algorithmic-bytes A --source-hash H --out FILE.json
"""
from __future__ import annotations

import argparse
import csv
import glob
import json
import os
import statistics
import sys


def _csv(directory: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(directory, "**", "*" + suffix), recursive=True))
    if not hits:
        raise FileNotFoundError("no *%s under %s" % (suffix, directory))
    return hits[0]


def dispatches(directory: str, kernel: str = "", grid: int | None = None) -> list[dict]:
    """Kernel-trace rows (name, grid size, duration in ns) matching the filters."""
    rows = []
    with open(_csv(directory, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            name = r["Kernel_Name"]
            if kernel and kernel not in name:
                continue
            g = int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0)
            if grid is not None and g != grid:
                continue
            rows.append({"name": name, "grid": g,
                         "ns": int(r["End_Timestamp"]) - int(r["Start_Timestamp"])})
    return rows


def calls(directory: str, start: str, include: str = "") -> list[dict]:
    """Group the dispatches (in time order) into library calls: a call begins
    at a dispatch whose name contains `start` (or any of several substrings
    separated by '|') and takes the following dispatches whose names contain
    `include` (others are skipped).  Returns, per distinct (grids of its
    dispatches, kernel sequence), the number of calls and the median duration
    of each kernel position and of their sum; "grid" is the first
    dispatch's grid."""
    rows = []
    with open(_csv(directory, "kernel_trace.csv")) as f:
        for r in csv.DictReader(f):
            rows.append((int(r["Start_Timestamp"]), r["Kernel_Name"],
                         int(r.get("Grid_Size") or r.get("Grid_Size_X") or 0),
                         int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    rows.sort()
    starts = [x for x in start.split("|") if x]
    groups: dict = {}
    cur = None
    for _, name, grid, ns in rows:
        if any(x in name for x in starts):
            cur = {"grids": [grid], "names": [_short(name)], "ns": [ns]}
            key = None
        elif cur is not None and include and include in name:
            cur["grids"].append(grid)
            cur["names"].append(_short(name))
            cur["ns"].append(ns)
        else:
            continue
        # (re)file the call under its current grids and kernel sequence
        if key is not None:
            groups[key].remove(cur)
        key = (tuple(cur["grids"]), tuple(cur["names"]))
        groups.setdefault(key, []).append(cur)
    out = []
    for (grids, names), cs in groups.items():
        if not cs:
            continue
        med = [statistics.median(c["ns"][i] for c in cs) / 1e3 for i in range(len(names))]
        out.append({"grid": grids[0], "grids": list(grids), "kernels": list(names),
                    "calls": len(cs), "median_us": med,
                    "median_sum_us": statistics.median(sum(c["ns"]) for c in cs) / 1e3})
    return out


def _short(name: str) -> str:
    """Kernel name without the namespace and the parameter list."""
    base = name.replace("(anonymous namespace)::", "").replace("q4k::", "").replace("void ", "")
    return base.split("(")[0]


def kernel_stats(directory: str) -> list[dict]:
    """The rows of rocprofv3's kernel_stats.csv (all kernels)."""
    with open(_csv(directory, "kernel_stats.csv")) as f:
        return list(csv.DictReader(f))


def counter_per_dispatch(directory: str, counter: str, kernel: str,
                         grid: int | None = None) -> tuple[float, int]:
    """Mean value of a PMC counter over the matching dispatches, and their count."""
    vals = []
    with open(_csv(directory, "counter_collection.csv")) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] != counter or kernel not in r["Kernel_Name"]:
                continue
            if grid is not None and int(r["Grid_Size"]) != grid:
                continue
            vals.append(float(r["Counter_Value"]))
    if not vals:
        raise ValueError("no %s samples for kernel %r grid %s" % (counter, kernel, grid))
    return statistics.fmean(vals), len(vals)


def traffic(fetch_dir: str, write_dir: str, kernel: str, grid: int | None, calib_kernel: str,
            calib_bytes: int) -> dict:
    """HBM bytes per dispatch of `kernel`, each counter (KiB) scaled by the
    factor that maps its reading for the calibration copy to the copy's true
    size (calib_bytes read and calib_bytes written)."""
    f_k, nf = counter_per_dispatch(fetch_dir, "FETCH_SIZE", kernel, grid)
    w_k, nw = counter_per_dispatch(write_dir, "WRITE_SIZE", kernel, grid)
    f_c, _ = counter_per_dispatch(fetch_dir, "FETCH_SIZE", calib_kernel)
    w_c, _ = counter_per_dispatch(write_dir, "WRITE_SIZE", calib_kernel)
    f_scale = calib_bytes / (f_c * 1024.0)
    w_scale = calib_bytes / (w_c * 1024.0)
    fetch = f_k * 1024.0 * f_scale
    write = w_k * 1024.0 * w_scale
    return {"fetch_bytes_per_launch": fetch, "write_bytes_per_launch": write,
            "hbm_bytes_per_launch": fetch + write,
            "raw_kib": {"fetch": f_k, "write": w_k, "calib_fetch": f_c, "calib_write": w_c},
            "scale": {"fetch": f_scale, "write": w_scale}, "dispatches": {"fetch": nf, "write": nw}}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(prog="python -m bit_block_quantized_gguf_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("dir")
    t.add_argument("--kernel", default="")
    t.add_argument("--grid", type=int)
    c = sub.add_parser("calls")
    c.add_argument("dir")
    c.add_argument("--start", required=True)
    c.add_argument("--include", default="")
    tr = sub.add_parser("traffic")
    tr.add_argument("--fetch", required=True)
    tr.add_argument("--write", required=True)
    tr.add_argument("--kernel", required=True)
    tr.add_argument("--grid", type=int)
    tr.add_argument("--calib-kernel", required=True)
    tr.add_argument("--calib-bytes", type=int, required=True)
    tr.add_argument("--algorithmic-bytes", type=int, required=True)
    tr.add_argument("--source-hash", required=True)
    tr.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    if a.cmd == "trace":
        for r in kernel_stats(a.dir):
            print("%-90.90s calls %6s  avg %10.1f us" % (r["Name"], r["Calls"],
                                                         float(r["AverageNs"]) / 1e3))
        if a.kernel or a.grid is not None:
            d = dispatches(a.dir, a.kernel, a.grid)
            if d:
                ns = [x["ns"] for x in d]
                print("filter kernel=%r grid=%s: %d dispatches, mean %.2f us, median %.2f us"
                      % (a.kernel, a.grid, len(ns), statistics.fmean(ns) / 1e3,
                         statistics.median(ns) / 1e3))
        return 0
    if a.cmd == "calls":
        for g in calls(a.dir, a.start, a.include):
            print("grids %-24s  calls %4d  %s  sum %.1f us" % (
                "/".join(str(x) for x in g["grids"]), g["calls"],
                "  ".join("%s %.1f us" % (n, u) for n, u in zip(g["kernels"], g["median_us"])),
                g["median_sum_us"]))
        return 0
    res = traffic(a.fetch, a.write, a.kernel, a.grid, a.calib_kernel, a.calib_bytes)
    res.update({"kernel": a.kernel, "grid": a.grid, "algorithmic_bytes_per_launch":
                a.algorithmic_bytes, "traffic_over_algorithmic":
                res["hbm_bytes_per_launch"] / a.algorithmic_bytes,
                "calibration": {"kernel": a.calib_kernel, "bytes_each_way": a.calib_bytes},
                "source_hash": a.source_hash})
    with open(a.out, "w") as f:
        json.dump(res, f, indent=1)
    print(json.dumps(res, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
