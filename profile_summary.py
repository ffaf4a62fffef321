#!/usr/bin/env python3
"""Summarise rocprofv3 CSV output per kernel launch shape.

rocprofv3 --stats averages every dispatch of a kernel symbol, but one GEMM
symbol serves several problem shapes. This groups the dispatches of a
``*_kernel_trace.csv`` by (kernel, grid size) and prints calls, average,
min and max duration in microseconds; with ``--pmc`` it averages the
counter columns of a ``*_counter_collection.csv`` per (kernel, grid).

usage: python profile_summary.py TRACE_CSV [--pmc COUNTER_CSV]
"""
from __future__ import annotations

import argparse
import csv
import re
from collections import defaultdict


def short(name: str) -> str:
    m = re.search(r"::(\w+_kernel(?:<[^>]*>)?)\(", name)
    return m.group(1) if m else name[:60]


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


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("trace", nargs="?")
    ap.add_argument("--pmc")
    a = ap.parse_args()
    if a.trace:
        trace_summary(a.trace)
    if a.pmc:
        pmc_summary(a.pmc)
