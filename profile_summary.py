#!/usr/bin/env python3
"""Summarise rocprofv3 CSV output per kernel launch shape.

rocprofv3 --stats averages every dispatch of a kernel symbol, but one GEMM
symbol serves several problem shapes. This groups the dispatches of a
``*_kernel_trace.csv`` by (kernel, grid size) and prints calls, average,
min and max duration in microseconds; with ``--pmc`` it averages the
counter columns of a ``*_counter_collection.csv`` per (kernel, grid).

usage: python profile_summary.py TRACE_CSV [--pmc COUNTER_CSV]
       python profile_summary.py --traffic FETCH_CSV WRITE_CSV KERNEL_SRC OUT_JSON
       python profile_summary.py --traffic-md FETCH_CSV WRITE_CSV OUT_MD [--command CMD]
       python profile_summary.py --mfma COUNTER_CSV OUT_MD [--command CMD]

--traffic turns two counter runs of `bench.py --pmc-gemm` (FETCH_SIZE, then
WRITE_SIZE, in KiB per dispatch) into HBM bytes per GEMM launch. Each counter
is scaled by bytes / counter of the 1 GiB copy kernel in the same run (the
copy reads and writes exactly 2^30 bytes), and the result is written with
the sha256 of the kernel source's code (comments and blank lines dropped)
it was measured on. --traffic-md writes the same calibrated bytes for every
kernel of the run (GEMM and quantizers) as a markdown table, and --mfma
turns a GRBM_GUI_ACTIVE / SQ_VALU_MFMA_BUSY_CYCLES / TA_TA_BUSY_sum run into
MFMA utilisation and effective clock per GEMM launch.
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


# The persistent GEMM launches one work-group per CU for every shape, so its
# grid does not identify the product; the quantizer launch just before it
# does. Keys are grid sizes in threads: the two-operand launch of each
# product (512 threads per work-group: A and B groups together), and the B
# operand's own launch for runs that quantize the operands one by one.
PRODUCT_OF_B_GRID = {(2048 + 1536) * 512: "qkv fprop (8192,6144,4096)",
                     (2048 + 7168) * 512: "gate+up fprop (8192,28672,4096)",
                     (2048 + 896) * 512: "down dgrad (8192,14336,4096)",
                     (512 + 1792) * 512: "down wgrad (4096,14336,8192)",
                     786432: "qkv fprop (8192,6144,4096)",
                     3670016: "gate+up fprop (8192,28672,4096)",
                     458752: "down dgrad (8192,14336,4096)",
                     917504: "down wgrad (4096,14336,8192)"}


def trace_summary(path, window=None):
    groups = defaultdict(list)
    with open(path) as f:
        rows = sorted(csv.DictReader(f), key=lambda r: int(r["Start_Timestamp"]))
    prev = None
    for row in rows:
        name = short(row["Kernel_Name"])
        grid = int(row["Grid_Size_X"]) * int(row["Grid_Size_Y"]) * int(row["Grid_Size_Z"])
        key = (name, grid, int(row["Workgroup_Size_X"]))
        if name.startswith("gemm_dma_kernel") and prev is not None:
            key = (f"{name} [{PRODUCT_OF_B_GRID.get(prev[1], 'after ' + prev[0])}]", grid, key[2])
        dur = (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3
        groups[key].append(dur)
        if name.startswith("quant"):
            prev = (name, grid)
    print("| kernel | grid threads | wg | calls | avg us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|")
    for (k, g, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
        med = sorted(d)[len(d) // 2]
        print(f"| {k} | {g} | {wg} | {len(d)} | {sum(d) / len(d):.2f} | {med:.2f} | {min(d):.2f} | "
              f"{max(d):.2f} |")
    if window:
        # bench.py's first GPU work is W warm-up steps, then K steps with an
        # event around every launch: dispatches W .. W + K - 1 of each
        # step kernel (in time order) are the ones its per-kernel means use
        w, k = window
        print()
        print(f"Step launches only (dispatches {w} .. {w + k - 1} of each kernel and product, "
              f"the bench's per-kernel pass):")
        print()
        print("| kernel | calls | avg us | median us | min us | max us |")
        print("|---|---|---|---|---|---|")
        for (name, g, wg), d in sorted(groups.items(), key=lambda kv: -sum(kv[1])):
            if not (name.startswith("gemm_dma_kernel") and name.endswith("]") and ", 0>" in name
                    or name.startswith("quant_pair_kernel")):
                continue
            sel = d[w:w + k]
            if len(sel) < k:
                continue
            med = sorted(sel)[len(sel) // 2]
            print(f"| {name} (grid {g}) | {len(sel)} | {sum(sel) / len(sel):.2f} | {med:.2f} | "
                  f"{min(sel):.2f} | {max(sel):.2f} |")


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


def _per_launch(path, counter):
    """Counter values per (kernel, grid size) launch shape."""
    out = defaultdict(list)
    with open(path) as f:
        for row in csv.DictReader(f):
            if row["Counter_Name"] == counter:
                grid = int(row.get("Grid_Size") or row.get("Grid_Size_X"))
                out[(short(row["Kernel_Name"]), grid)].append(float(row["Counter_Value"]))
    return out


# Algorithmic bytes of the launch shapes that bench.py --pmc-gemm runs: the
# quantizers (2 B read + 0.5 B nibbles + 1/32 B scale per element) and the
# gate+up GEMM (packed operands + fp32 C).
QUANT_PER_ELEMENT = 2 + 0.5 + 1 / 32
GEMM_BYTES = 8192 * 2048 + 8192 * 128 + 28672 * 2048 + 28672 * 128 + 8192 * 28672 * 4


def traffic_table(fetch_csv, write_csv, out_md, command):
    """Markdown table: HBM-side read/write bytes per launch of every kernel
    in a --pmc-gemm run, calibrated on the 1 GiB copy."""
    fetch = _per_launch(fetch_csv, "FETCH_SIZE")
    write = _per_launch(write_csv, "WRITE_SIZE")
    ck = [k for k in fetch if "copyBuffer" in k[0] and k in write]
    ck = max(ck, key=lambda k: sum(fetch[k]) / len(fetch[k]))
    f_factor = float(1 << 30) / (sum(fetch[ck]) / len(fetch[ck]) * 1024.0)
    w_factor = float(1 << 30) / (sum(write[ck]) / len(write[ck]) * 1024.0)
    lines = ["| kernel | grid | dispatches | read MB | write MB | total MB | algorithmic MB |",
             "|---|---|---|---|---|---|---|"]
    for key in fetch:
        if key not in write or key == ck:
            continue
        rd = sum(fetch[key]) / len(fetch[key]) * 1024.0 * f_factor
        wr = sum(write[key]) / len(write[key]) * 1024.0 * w_factor
        alg = GEMM_BYTES if "gemm" in key[0] else None
        if key[0].startswith("quant_row"):             # one thread per 32-element block
            alg = key[1] * 32 * QUANT_PER_ELEMENT
        elif key[0].startswith("quant_col_staged"):   # one thread per 4 x 32 patch
            alg = key[1] * 128 * QUANT_PER_ELEMENT
        lines.append(f"| {key[0]} | {key[1]} | {len(fetch[key])} | {rd / 1e6:.1f} | {wr / 1e6:.1f} | "
                     f"{(rd + wr) / 1e6:.1f} | {alg / 1e6 if alg else float('nan'):.1f} |")
    text = ("# HBM-side traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE)\n\n"
            f"Calibration: {ck[0]} copying 1 GiB; FETCH_SIZE x {f_factor:.3f}, WRITE_SIZE x "
            f"{w_factor:.3f} give its 2^30 read and written bytes. FETCH_SIZE and WRITE_SIZE "
            "count L2-to-fabric bytes (HBM or the Infinity Cache in front of it).\n\n"
            f"Command (from /tmp, TMPDIR=/tmp, repository at $R):\n\n    {command}\n\n"
            + "\n".join(lines) + "\n")
    with open(out_md, "w") as f:
        f.write(text)
    print(text)


def mfma_table(csv_path, out_md, command, xcds=8, simds=1024):
    """MFMA utilisation and effective clock per GEMM launch shape from a run
    with GRBM_GUI_ACTIVE and SQ_VALU_MFMA_BUSY_CYCLES (GRBM_GUI_ACTIVE is
    summed over the XCDs; SQ_VALU_MFMA_BUSY_CYCLES over every SIMD)."""
    per = defaultdict(lambda: defaultdict(float))
    meta = {}
    with open(csv_path) as f:
        for row in csv.DictReader(f):
            d = int(row["Dispatch_Id"])
            per[d][row["Counter_Name"]] += float(row["Counter_Value"])
            meta[d] = (short(row["Kernel_Name"]), int(row.get("Grid_Size") or row.get("Grid_Size_X")),
                       (int(row["End_Timestamp"]) - int(row["Start_Timestamp"])) / 1e3)
    lines = ["| kernel | grid | dispatch | us | clock GHz | MFMA busy % | TA busy % |",
             "|---|---|---|---|---|---|---|"]
    for d in sorted(per):
        k, g, us = meta[d]
        c = per[d]
        gui = c.get("GRBM_GUI_ACTIVE", 0.0) / xcds
        if not gui or "SQ_VALU_MFMA_BUSY_CYCLES" not in c or "gemm" not in k:
            continue
        mf = 100.0 * c["SQ_VALU_MFMA_BUSY_CYCLES"] / (gui * simds)
        ta = 100.0 * c.get("TA_TA_BUSY_sum", float("nan")) / (gui * simds / 4)
        lines.append(f"| {k} | {g} | {d} | {us:.1f} | {gui / us / 1e3:.2f} | {mf:.1f} | {ta:.1f} |")
    text = ("# MFMA utilisation of the GEMM launches (rocprofv3 counters)\n\n"
            "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 XCDs x 1024 SIMDs); "
            "TA busy = TA_TA_BUSY summed over CUs / (GRBM_GUI_ACTIVE / 8 x 256 CUs); clock = "
            "GRBM_GUI_ACTIVE / 8 / kernel duration.\n\n"
            f"Command (from /tmp, TMPDIR=/tmp, repository at $R):\n\n    {command}\n\n"
            + "\n".join(lines) + "\n")
    with open(out_md, "w") as f:
        f.write(text)
    print(text)


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
    ap.add_argument("--step-window", nargs=2, type=int, metavar=("W", "K"),
                    help="also list dispatches W .. W+K-1 of each step kernel")
    ap.add_argument("--pmc")
    ap.add_argument("--traffic", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "KERNEL_SRC", "OUT_JSON"))
    ap.add_argument("--traffic-md", nargs=3, metavar=("FETCH_CSV", "WRITE_CSV", "OUT_MD"))
    ap.add_argument("--mfma", nargs=2, metavar=("COUNTER_CSV", "OUT_MD"))
    ap.add_argument("--command", default="", help="command line recorded in the markdown")
    a = ap.parse_args()
    if a.trace:
        trace_summary(a.trace, a.step_window)
    if a.pmc:
        pmc_summary(a.pmc)
    if a.traffic:
        traffic(*a.traffic)
    if a.traffic_md:
        traffic_table(*a.traffic_md, a.command)
    if a.mfma:
        mfma_table(*a.mfma, a.command)
