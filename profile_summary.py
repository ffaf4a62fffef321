#!/usr/bin/env python3
"""Summarise rocprofv3 CSV output per kernel launch shape.

rocprofv3 --stats averages every dispatch of a kernel symbol, but one GEMM
symbol serves several problem shapes. This groups the dispatches of a
``*_kernel_trace.csv`` by (kernel, grid size) and prints calls, average,
min and max duration in microseconds; with ``--pmc`` it averages the
counter columns of a ``*_counter_collection.csv`` per (kernel, grid).

usage: python profile_summary.py TRACE_CSV [--pmc COUNTER_CSV]
       python profile_summary.py --traffic FETCH_CSV WRITE_CSV KERNEL_SRC OUT_JSON

--traffic turns two counter runs of `bench.py --pmc-gemm` (FETCH_SIZE, then
WRITE_SIZE, in KiB per dispatch) into HBM bytes per GEMM launch. Each counter
is scaled by bytes / counter of the 1 GiB copy kernel in the same run (the
copy reads and writes exactly 2^30 bytes), and the result is written with
the sha256 of the kernel source's code (comments and blank lines dropped)
it was measured on.
"""
from __future__ import annotations

import argparse
import csv
import re
from collections import defaultdict


def short(name: str) -> str:
    """Kernel name with its template arguments, without namespaces and parameters."""
    m = re.search(r"(\w+_kernel)\b", name)
    if not m:
        return name[:60]
    out, i = m.group(1), m.end()
    if i < len(name) and name[i] == "<":
        depth, j = 0, i
        while j < len(name):
            depth += {"<": 1, ">": -1}.get(name[j], 0)
            j += 1
            if depth == 0:
                break
        out += re.sub(r"(\w+::|\(anonymous namespace\)::)", "", name[i:j])
    return out


def trace_summary(path):
    groups = defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            key = (short(row["Kernel_Name"]), int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) *
                   int(row["Grid_Size_Z"]), int(row["Workgroup_Size_X"]))
            dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
            groups[key].append(dur)
    print("| kernel | grid threads | wg | calls | avg us | min us | max us |")
    print("|---|---|---|---|---|---|---|")
    for (k, g, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        print(f"| {k} | {g} | {wg} | {len(d)} | {sum(d) / len(d):.2f} | {min(d):.2f} | {max(d):.2f} |")


def pmc_summary(path):
    groups = defaultdict(lambda: defaultdict(list))
    with open(path) as f:
        rows = list(csv.DictReader(f))
    for row in rows:
        grid = row.get("Grid_Size") or row.get("Grid_Size_X")
        key = (short(row["Kernel_Name"]), grid)
        groups[key][row["Counter_Name"]].append(float(row["Counter_Value"]))
    print("| kernel | grid | counter | dispatches | avg value |")
    print("|---|---|---|---|---|")
    for (k, g), ctrs in groups.items():
        for c, vals in ctrs.items():
            print(f"| {k} | {g} | {c} | {len(vals)} | {sum(vals) / len(vals):.1f} |")


def _per_kernel(path, counter):
    out = defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                out[short(row["Kernel_Name"])].append(float(row["Counter_Value"]))
    return out


def sha_of(path):
    """sha256 (first 16 hex) of a source file's code: // comments and blank
    lines are dropped, so a comment edit does not mark counters as stale."""
    import hashlib
    with open(path) as f:
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in f]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def traffic(fetch_csv, write_csv, kernel_src, out_json):
    import json
    fetch = _per_kernel(fetch_csv, "FETCH_SIZE")
    write = _per_kernel(write_csv, "WRITE_SIZE")
    copy_key = [k for k in fetch if "copyBuffer" in k or "copy" in k.lower()]
    gemm_key = [k for k in fetch if "gemm" in k]
    assert copy_key and gemm_key, (list(fetch), list(write))
    ck, gk = copy_key[0], gemm_key[0]
    copy_bytes = float(1 << 30)
    f_factor = copy_bytes / (sum(fetch[ck]) / len(fetch[ck]) * 1024.0)
    w_factor = copy_bytes / (sum(write[ck]) / len(write[ck]) * 1024.0)
    g_fetch = sum(fetch[gk]) / len(fetch[gk]) * 1024.0 * f_factor
    g_write = sum(write[gk]) / len(write[gk]) * 1024.0 * w_factor
    sha = sha_of(kernel_src)
    rec = {"kernel": gk, "kernel_sha": sha, "bytes_per_launch": round(g_fetch + g_write),
           "read_bytes": round(g_fetch), "write_bytes": round(g_write),
           "fetch_factor": round(f_factor, 4), "write_factor": round(w_factor, 4),
           "calibration": f"{ck}: 1 GiB device copy",
           "algorithmic_bytes": {"A_nibbles": 8192 * 2048, "A_scales": 8192 * 128,
                                 "B_nibbles": 28672 * 2048, "B_scales": 28672 * 128,
                                 "C_fp32": 8192 * 28672 * 4}}
    with open(out_json, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("trace", nargs="?")
    ap.add_argument("--pmc")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL_SRC", "OUT_JSON"))
    a = ap.parse_args()
    if a.trace:
        trace_summary(a.trace)
    if a.pmc:
        pmc_summary(a.pmc)
    if a.traffic:
        traffic(*a.traffic)
