#!/usr/bin/env python3
"""Benchmark of the H16 + MXFP4 quantize + MXFP4 GEMM hot path on one MI355X.

One step = the four linear-layer products of a Llama-3.1-8B block at 8192
tokens, each as the two launches its fused entry point issues (both
operands rotated and quantized in one launch, then the MXFP4 GEMM) through
the C ABI, on one stream:

  qkv fprop         Y  = X W^T      GEMM (M, N, K) = (8192, 6144, 4096)
  gate+up fprop     Y  = X W^T      (8192, 28672, 4096)
  down-proj dgrad   dX = dY W       (8192, 14336, 4096)   W quantized 32x1
  down-proj wgrad   dW = dY^T X     (4096, 14336, 8192)   both 32x1 along T

H16 rotation along each reduction axis, OCP-floor scales, fp32 output.
Inputs are seeded synthetic tensors (synthetic.make) already resident in
HBM when the timed region starts. The timed region is K steps launched
back to back with nothing else on the stream; `value` is the step's total
2MNK over its wall time. A second pass of K steps brackets every launch
with HIP events on the launch stream, giving per-kernel average durations
(the roofline figure). The fused entry points, and the step captured in a
HIP graph and replayed, are timed as well (same kernels), right after the
timed region, as cross-checks.

Also measured: the quantizer-only workload (8192 x 4096, Student-t x
log-normal) for every axis and scale rule with H16, plus H0/H32 row-wise,
cycling six buffer sets (> 400 MB) so the 256 MB last-level cache cannot
hold the data, in GB/s of algorithmic bytes (2 B read + 0.5 B nibbles +
1/32 B scale per element): 10 warm-up launches, then 50 launches each
bracketed by events (median, min) and 50 launched back to back between two
events (mean, the headline GB/s); a 1 GiB device-to-device copy gives the
achievable-HBM reference. The quantization error of every product against
the exact product of its bf16 operands (fp64, on a row sample) is reported
for H0/H16/H32 x both scale rules.

The CPU baseline is the oracle (numpy, fp64 GEMM) timed on this host on a
bounded sample of the same step.

Prints ONE JSON line.
"""
from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "H16+MXFP4 quant+GEMM TFLOP/s (Llama-8B Fprop/Dgrad/Wgrad); quantizer GB/s"
HBM_PEAK_GBS = 8000.0
MXFP4_PEAK_TFLOPS = 10100.0

# name, workload, op, (T, N, K), source tensors (P, Q)
PRODUCTS = [
    ("qkv_fprop", "qkv", "fprop", (8192, 6144, 4096), ("X", "W")),
    ("gateup_fprop", "mlp", "fprop", (8192, 28672, 4096), ("X", "W_gu")),
    ("down_dgrad", "mlp", "dgrad", (8192, 4096, 14336), ("dY", "W_down")),
    ("down_wgrad", "wgrad", "wgrad", (8192, 4096, 14336), ("dY", "X")),
]
DOMINANT = "gateup_fprop"


def plan(op, T, N, K):
    """(A source shape, A axis), (B source shape, B axis), GEMM (M, N, K)."""
    if op == "fprop":
        return ((T, K), 0), ((N, K), 0), (T, N, K)
    if op == "dgrad":
        return ((T, N), 0), ((N, K), 1), (T, K, N)
    return ((T, N), 1), ((T, K), 1), (N, K, T)


def quant_bytes(rows, cols, axis):
    n = rows * cols
    return 2 * n + n // 2 + (n // 1024 if axis == 2 else n // 32)


def sha_of(path):
    """sha256 (first 16 hex) of a source file's code: // comments and blank
    lines are dropped, so a comment edit does not mark counters as stale."""
    with open(path) as f:
        lines = [re.sub(r"//.*", "", ln).rstrip() for ln in f]
    code = "\n".join(ln for ln in lines if ln.strip())
    return hashlib.sha256(code.encode()).hexdigest()[:16]


def load_traffic(kernel_src):
    """HBM bytes per launch of the dominant GEMM from the committed counter
    summary, if it was taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", "gemm_gateup_fprop_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_sha") != sha_of(kernel_src):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(work, budget_rows=8192, budget_cols=16384):
    """Oracle on a bounded sample of the step: for each product, a
    budget_rows x budget_cols tile of the output at full reduction length
    (quantize the matching source slices, dequantize, fp64 GEMM + sum|a||b|)."""
    import numpy as np
    import oracle as O
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_info
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas = None
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    flops = qbytes = tq = 0.0
    t0 = time.perf_counter()
    for name, wl, op, (T, N, K), (pn, qn) in PRODUCTS:
        P, Q = work[wl][pn], work[wl][qn]
        (_, _), (_, _), (GM, GN, GK) = plan(op, T, N, K)
        m, n = min(budget_rows, GM), min(budget_cols, GN)
        tq0 = time.perf_counter()
        def q(src, axis):
            return O.quantize_chunked(np.ascontiguousarray(src), axis, 16, 0, chunk=64,
                                      threads=cores)
        if op == "fprop":
            qa, qb = q(P[:m], O.AXIS_ROW), q(Q[:n], O.AXIS_ROW)
        elif op == "dgrad":
            qa, qb = q(P[:m], O.AXIS_ROW), q(Q[:, :n], O.AXIS_COL)
        else:
            qa, qb = q(P[:, :m], O.AXIS_COL), q(Q[:, :n], O.AXIS_COL)
        tq += time.perf_counter() - tq0
        qbytes += (m + n) * GK * (2 + 0.5 + 1 / 32)
        O.gemm_ref(O.dequantize(*qa), O.dequantize(*qb))
        flops += 2.0 * m * n * GK
    dt = time.perf_counter() - t0
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu_model": model, "blas_threads": blas,
            "seconds": round(dt, 3),
            "quantize_GB/s": round(qbytes / tq / 1e9, 3),
            "gemm_GFLOP/s": round(flops / (dt - tq) / 1e9, 1),
            "sample": f"{budget_rows}x{budget_cols} output tile of each of the 4 products at full "
                      f"reduction length: oracle rotate+quantize of the matching source slices "
                      f"({cores} threads over 64-row or 64-column slabs), dequantize, fp64 GEMM "
                      f"and sum|a||b| (numpy; BLAS threads = {blas})"}


def gemm_error(mx, an, asc, bn, bsc, p, ref, rows, stream):
    """Error statistics of mxfp4_gemm(A, B) (first `rows` output rows)
    against the fp64 reference `ref`."""
    import numpy as np
    mx.mxfp4_gemm(an, asc, bn, bsc, p["GM"], p["GN"], p["GK"], p["C"], mx.OUT_F32, stream)
    c = p["C"][:rows].double()
    d = c - ref
    nd, nr = float((d * d).sum()), float((ref * ref).sum())
    return {"mse": float((d * d).mean()),
            "cosine": float((c * ref).sum() / (c.norm() * ref.norm())),
            "rel_fro": (nd / nr) ** 0.5,
            "snr_db": 10.0 * np.log10(nr / nd)}


def error_report(mx, torch, prods, stream, dev, rows=128):
    """Quantization error of each product's fused entry point against the
    exact product of its original bf16 operands (fp64 on the GPU, first
    `rows` output rows), for H in {0, 16, 32} x {ocp_floor, ceil}: MSE,
    cosine, relative Frobenius error and SNR in dB."""
    import numpy as np
    out = {}
    for p in prods:
        fn = {"fprop": mx.mxfp4_fprop, "dgrad": mx.mxfp4_dgrad, "wgrad": mx.mxfp4_wgrad}[p["op"]]
        P64, Q64 = p["P"], p["Q"]
        if p["op"] == "fprop":
            ref = P64[:rows].double() @ Q64.double().t()
        elif p["op"] == "dgrad":
            ref = P64[:rows].double() @ Q64.double()
        else:
            ref = P64[:, :rows].double().t() @ Q64.double()
        rec = {}
        for h in (0, 16, 32):
            for m in (0, 1):
                fn(p["P"], p["Q"], p["T"], p["N"], p["K"], h, m, p["ws"], p["C"], mx.OUT_F32,
                   stream)
                c = p["C"][:rows].double()
                d = c - ref
                nd, nr = float((d * d).sum()), float((ref * ref).sum())
                rec[f"h{h}_{['ocp_floor', 'ceil'][m]}"] = {
                    "mse": float((d * d).mean()),
                    "cosine": float((c * ref).sum() / (c.norm() * ref.norm())),
                    "rel_fro": (nd / nr) ** 0.5,
                    "snr_db": 10.0 * np.log10(nr / nd)}
        if p["op"] == "fprop":
            # outlier fallback on the weight: Y = [X | X] . [W1 | W2]^T over 2K
            for m in (0, 1):
                an, asc = mx.quantize(p["P"], mx.AXIS_ROW, 16, m, stream)
                bn, bsc = mx.quantize_of(p["Q"], mx.AXIS_ROW, 16, m, stream)
                a2n = torch.cat([an, an], 1).contiguous()
                a2s = torch.cat([asc, asc], 1).contiguous()
                mx.mxfp4_gemm(a2n, a2s, bn, bsc, p["GM"], p["GN"], 2 * p["GK"], p["C"],
                              mx.OUT_F32, stream)
                c = p["C"][:rows].double()
                d = c - ref
                nd, nr = float((d * d).sum()), float((ref * ref).sum())
                rec[f"of_w_h16_{['ocp_floor', 'ceil'][m]}"] = {
                    "mse": float((d * d).mean()),
                    "cosine": float((c * ref).sum() / (c.norm() * ref.norm())),
                    "rel_fro": (nd / nr) ** 0.5,
                    "snr_db": 10.0 * np.log10(nr / nd)}
                del an, asc, bn, bsc, a2n, a2s
            # comparison arms ([P1]: random Hadamard and stochastic rounding
            # diverge in training): the same signs on both operands along K;
            # independent random integers for the two operands
            import synthetic
            signs = torch.from_numpy(synthetic.random_signs(p["K"], 61)).to(dev)
            for m in (0, 1):
                an, asc = mx.quantize_rs(p["P"], signs, mx.AXIS_ROW, 16, m, stream)
                bn, bsc = mx.quantize_rs(p["Q"], signs, mx.AXIS_ROW, 16, m, stream)
                rec[f"rs_h16_{['ocp_floor', 'ceil'][m]}"] = gemm_error(
                    mx, an, asc, bn, bsc, p, ref, rows, stream)
                del an, asc, bn, bsc
                ra = torch.from_numpy(synthetic.random_u32(tuple(p["P"].shape), 62).view(np.int32)).to(dev)
                rb = torch.from_numpy(synthetic.random_u32(tuple(p["Q"].shape), 63).view(np.int32)).to(dev)
                an, asc = mx.quantize_sr(p["P"], ra, mx.AXIS_ROW, 16, m, stream)
                bn, bsc = mx.quantize_sr(p["Q"], rb, mx.AXIS_ROW, 16, m, stream)
                rec[f"sr_h16_{['ocp_floor', 'ceil'][m]}"] = gemm_error(
                    mx, an, asc, bn, bsc, p, ref, rows, stream)
                del an, asc, bn, bsc, ra, rb
                # macro-block scaling ([P3] MBS: prescale, quantize, postscale)
                # on both operands, multiplied by the MBS GEMM
                qa = mx.quantize_mbs(p["P"], mx.AXIS_ROW, 16, m, stream)
                qb = mx.quantize_mbs(p["Q"], mx.AXIS_ROW, 16, m, stream)
                args = (*qa, *qb, p["GM"], p["GN"], p["GK"], p["C"], mx.OUT_F32, stream)
                mx.mxfp4_gemm_mbs(*args)
                c = p["C"][:rows].double()
                d = c - ref
                nd, nr = float((d * d).sum()), float((ref * ref).sum())
                key = f"mbs_h16_{['ocp_floor', 'ceil'][m]}"
                rec[key] = {"mse": float((d * d).mean()),
                            "cosine": float((c * ref).sum() / (c.norm() * ref.norm())),
                            "rel_fro": (nd / nr) ** 0.5,
                            "snr_db": 10.0 * np.log10(nr / nd)}
                if m == 1:
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    for _ in range(10):
                        mx.mxfp4_gemm_mbs(*args)
                    e1.record(stream)
                    e1.synchronize()
                    us = e0.elapsed_time(e1) / 10 * 1e3
                    rec["mbs_gemm_us"] = round(us, 2)
                    rec["mbs_gemm_TFLOPs"] = round(
                        2.0 * p["GM"] * p["GN"] * p["GK"] / (us * 1e-6) / 1e12, 1)
                del qa, qb, args
        out[p["name"]] = rec
        del ref
    torch.cuda.synchronize()
    return out


def error_decomposition(mx, torch, synthetic, np, prods, stream, dev):
    """GPU three-way error decomposition (mxfp4_error_stats) of the quantizer
    workload (row and column blocks, H0/H16/H32 x both scale rules) and of
    every product operand as its fused entry quantizes it (H16, both rules):
    cos(e_scale, e_grid), deadzone fraction and the shares of ||e||^2.
    Also times the statistics kernel on the 8192 x 4096 tensor."""
    def summary(d):
        e2 = d["sum_e2"]
        return {"cos_scale_grid": round(d["cos_scale_grid"], 4),
                "deadzone_fraction": round(d["deadzone_fraction"], 4),
                "scale_share": round(d["sum_e_scale2"] / e2, 4) if e2 else None,
                "dz_share": round(d["sum_e_dz2"] / e2, 4) if e2 else None,
                "grid_share": round(d["sum_e_grid2"] / e2, 4) if e2 else None,
                "rel_err": round((e2 / d["sum_x2"]) ** 0.5, 5) if d["sum_x2"] else None}
    ws = torch.empty(mx.ERROR_STATS_WS_BYTES, dtype=torch.uint8, device=dev)
    A = synthetic.make("quant")["A"]
    a = torch.from_numpy(A.view(np.int16)).to(dev).view(torch.bfloat16)
    out = {"quant_8192x4096": {}}
    for ax in (0, 1):
        for h in (0, 16, 32):
            for m in (0, 1):
                d = mx.error_stats(a, ax, h, m, stream, ws)
                out["quant_8192x4096"][f"{['row', 'col'][ax]}_h{h}_{['ocp_floor', 'ceil'][m]}"] = summary(d)
    for p in prods:
        for which, t, shape, ax in (("A", p["P"], p["sa"], p["axa"]), ("B", p["Q"], p["sb"], p["axb"])):
            for m in (0, 1):
                d = mx.error_stats(t.view(shape[0], shape[1]), ax, 16, m, stream, ws)
                out.setdefault(p["name"], {})[f"{which}_h16_{['ocp_floor', 'ceil'][m]}"] = summary(d)
    o = torch.empty(mx.ERROR_STATS_COUNT, dtype=torch.float64, device=dev)
    R, C = A.shape
    for _ in range(3):
        mx.mxfp4_error_stats(a, R, C, 0, 16, 0, ws, o, stream)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(20):
        mx.mxfp4_error_stats(a, R, C, 0, 16, 0, ws, o, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / 20 * 1e3
    out["kernel_row_h16_us"] = round(us, 2)
    out["kernel_row_h16_GB/s"] = round(2.0 * R * C / (us * 1e-6) / 1e9, 1)
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    # 30 warm-up steps (~40 ms): the first ~30 ms of sustained load after the
    # host-side setup run at lower clocks (measured: 1.32 ms/step for the first
    # steps against 1.22 ms once warm), and the timed steps should see the
    # steady state.
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantizer", action="store_true")
    ap.add_argument("--quant-iters", type=int, default=50)
    ap.add_argument("--no-error-report", action="store_true")
    ap.add_argument("--pmc-gemm", action="store_true",
                    help="counter-collection mode: run only the gate+up GEMM (3 launches), the "
                         "row and column H16 quantizers on the 8192x4096 workload (3 launches "
                         "each) and a 1 GiB device-to-device copy (3 launches, the calibration "
                         "kernel)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the path has no multi-GPU component)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import mxfp4_quantized_gemm_amd as mx
    import synthetic

    mx.load_library()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    if args.pmc_gemm:
        mlp = synthetic.make("mlp")
        x = torch.from_numpy(mlp["X"].view(np.int16)).to(dev).view(torch.bfloat16)
        w = torch.from_numpy(mlp["W_gu"].view(np.int16)).to(dev).view(torch.bfloat16)
        an, asc = mx.quantize(x, mx.AXIS_ROW, 16, 0)
        bn, bsc = mx.quantize(w, mx.AXIS_ROW, 16, 0)
        c = torch.empty((8192, 28672), dtype=torch.float32, device=dev)
        for _ in range(3):
            mx.mxfp4_gemm(an, asc, bn, bsc, 8192, 28672, 4096, c, mx.OUT_F32, stream)
        del c
        q = torch.from_numpy(synthetic.make("quant")["A"].view(np.int16)).to(dev).view(torch.bfloat16)
        for axis in (mx.AXIS_ROW, mx.AXIS_COL):
            for _ in range(3):
                mx.quantize(q, axis, 16, 0)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("pmc-gemm done: 3 gate+up GEMMs, 3 row + 3 column quantizations, 3 copies of 1 GiB")
        return

    # ---------------------------------------------------------------- inputs
    t0 = time.perf_counter()
    work = {wl: synthetic.make(wl) for wl in ("qkv", "mlp", "wgrad")}
    log(f"inputs generated in {time.perf_counter() - t0:.1f}s")
    dev_t = {}
    for wl, d in work.items():
        for k, v in d.items():
            dev_t[(wl, k)] = torch.from_numpy(v.view(np.int16)).to(dev).view(torch.bfloat16)

    prods = []
    for name, wl, op, (T, N, K), (pn, qn) in PRODUCTS:
        (sa, axa), (sb, axb), (GM, GN, GK) = plan(op, T, N, K)
        na, sca = mx.packed_shapes(sa[0], sa[1], axa)
        nb, scb = mx.packed_shapes(sb[0], sb[1], axb)
        opcode = {"fprop": mx.OP_FPROP, "dgrad": mx.OP_DGRAD, "wgrad": mx.OP_WGRAD}[op]
        prods.append(dict(
            name=name, op=op, T=T, N=N, K=K, opcode=opcode, GM=GM, GN=GN, GK=GK,
            P=dev_t[(wl, pn)], Q=dev_t[(wl, qn)], sa=sa, axa=axa, sb=sb, axb=axb,
            an=torch.empty(na, dtype=torch.uint8, device=dev),
            asc=torch.empty(sca, dtype=torch.uint8, device=dev),
            bn=torch.empty(nb, dtype=torch.uint8, device=dev),
            bsc=torch.empty(scb, dtype=torch.uint8, device=dev),
            C=torch.empty((GM, GN), dtype=torch.float32, device=dev),
            ws=torch.empty(mx.mxfp4_workspace_bytes(opcode, T, N, K), dtype=torch.uint8,
                           device=dev),
        ))

    def launches(p, mode=0, st=None, h=16):
        # both operands in one launch (mxfp4_quantize_pair), then the GEMM:
        # the launches mxfp4_fprop / dgrad / wgrad issue
        st = stream if st is None else st
        return [
            lambda: mx.mxfp4_quantize_pair(p["P"], p["sa"][0], p["sa"][1], p["axa"], p["an"],
                                           p["asc"], p["Q"], p["sb"][0], p["sb"][1], p["axb"],
                                           p["bn"], p["bsc"], h, mode, st),
            lambda: mx.mxfp4_gemm(p["an"], p["asc"], p["bn"], p["bsc"], p["GM"], p["GN"], p["GK"],
                                  p["C"], mx.OUT_F32, st),
        ]

    seq = [(p, j, fn) for p in prods for j, fn in enumerate(launches(p))]

    K_ = args.steps
    total_flops = sum(2.0 * p["GM"] * p["GN"] * p["GK"] for p in prods)
    # warm-up before the per-kernel pass (the timed region below has its own)
    for _ in range(args.warmup):
        for _, _, fn in seq:
            fn()
    torch.cuda.synchronize()

    # ------------------------------------- per-kernel pass (events per launch)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(K_)]
    for s in range(K_):
        ev[s][0].record(stream)
        for i, (_, _, fn) in enumerate(seq):
            fn()
            ev[s][i + 1].record(stream)
    torch.cuda.synchronize()
    D = np.array([[ev[s][i].elapsed_time(ev[s][i + 1]) for i in range(len(seq))]
                  for s in range(K_)])
    kernel_ms = D.mean(axis=0)
    kernel_med, kernel_min = np.median(D, axis=0), D.min(axis=0)

    per_product = {}
    kernels = []
    for idx, (p, j, _) in enumerate(seq):
        name = p["name"]
        rec = per_product.setdefault(name, {"GEMM_MNK": [p["GM"], p["GN"], p["GK"]]})
        if j == 0:
            b = (quant_bytes(p["sa"][0], p["sa"][1], p["axa"]) +
                 quant_bytes(p["sb"][0], p["sb"][1], p["axb"]))
            gbs = b / (kernel_ms[idx] * 1e-3) / 1e9
            rec["quant_AB_us"] = round(kernel_ms[idx] * 1e3, 2)
            rec["quant_AB_GBs"] = round(gbs, 1)
            kernels.append({"kernel": f"{name}.quant_AB",
                            "axes": [["row", "col"][p["axa"]], ["row", "col"][p["axb"]]],
                            "us": round(kernel_ms[idx] * 1e3, 2),
                            "us_median": round(kernel_med[idx] * 1e3, 2),
                            "us_min": round(kernel_min[idx] * 1e3, 2), "GB/s": round(gbs, 1),
                            "frac_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        else:
            f = 2.0 * p["GM"] * p["GN"] * p["GK"]
            tf = f / (kernel_ms[idx] * 1e-3) / 1e12
            rec["gemm_us"] = round(kernel_ms[idx] * 1e3, 2)
            rec["gemm_TFLOPs"] = round(tf, 1)
            tot = kernel_ms[idx - 1] + kernel_ms[idx]
            rec["fused_TFLOPs"] = round(f / (tot * 1e-3) / 1e12, 1)
            kernels.append({"kernel": f"{name}.gemm", "us": round(kernel_ms[idx] * 1e3, 2),
                            "us_median": round(kernel_med[idx] * 1e3, 2),
                            "us_min": round(kernel_min[idx] * 1e3, 2),
                            "TFLOP/s": round(tf, 1), "frac_mfma": round(tf / MXFP4_PEAK_TFLOPS, 4)})
    # fused entry points, same work (timed after the headline step, below)
    def fused_step():
        for p in prods:
            fn = {"fprop": mx.mxfp4_fprop, "dgrad": mx.mxfp4_dgrad, "wgrad": mx.mxfp4_wgrad}[p["op"]]
            fn(p["P"], p["Q"], p["T"], p["N"], p["K"], 16, 0, p["ws"], p["C"], mx.OUT_F32, stream)

    # the same GEMMs with bf16 output (C written in bf16, RNE), K launches each
    for p in prods:
        cb = torch.empty((p["GM"], p["GN"]), dtype=torch.bfloat16, device=dev)
        g = lambda: mx.mxfp4_gemm(p["an"], p["asc"], p["bn"], p["bsc"], p["GM"], p["GN"], p["GK"],
                                  cb, mx.OUT_BF16, stream)
        for _ in range(3):
            g()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(K_):
            g()
        e1.record(stream)
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / K_ * 1e3
        rec = per_product[p["name"]]
        rec["gemm_bf16_out_us"] = round(us, 2)
        rec["gemm_bf16_out_TFLOPs"] = round(2.0 * p["GM"] * p["GN"] * p["GK"] / (us * 1e-6) / 1e12, 1)
        del cb

    # the step with H0 and H32 instead of H16 (the comparison arms of the
    # rotation), K steps with an event around every launch as in the pass
    # above: each product's two-operand quantize launch in its place in the
    # step, and the fused TFLOP/s with that step's GEMM time
    for h in (0, 32):
        seq_h = [fn for p in prods for fn in launches(p, 0, None, h)]
        for fn in seq_h:
            fn()
        evh = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq_h) + 1)]
               for _ in range(K_)]
        for s_ in range(K_):
            evh[s_][0].record(stream)
            for i, fn in enumerate(seq_h):
                fn()
                evh[s_][i + 1].record(stream)
        torch.cuda.synchronize()
        Dh = np.array([[evh[s_][i].elapsed_time(evh[s_][i + 1]) for i in range(len(seq_h))]
                       for s_ in range(K_)]).mean(axis=0) * 1e3
        for k, p in enumerate(prods):
            rec = per_product[p["name"]]
            b = (quant_bytes(p["sa"][0], p["sa"][1], p["axa"]) +
                 quant_bytes(p["sb"][0], p["sb"][1], p["axb"]))
            qu, gu = Dh[2 * k], Dh[2 * k + 1]
            rec[f"quant_AB_h{h}_us"] = round(qu, 2)
            rec[f"quant_AB_h{h}_GBs"] = round(b / (qu * 1e-6) / 1e9, 1)
            rec[f"fused_h{h}_TFLOPs"] = round(2.0 * p["GM"] * p["GN"] * p["GK"] /
                                              ((qu + gu) * 1e-6) / 1e12, 1)

    # -------------------------------------------------- quantizer workload
    quant = None
    if not args.no_quantizer:
        A = synthetic.make("quant")["A"]
        nsets = 6
        srcs = [torch.from_numpy(A.view(np.int16)).to(dev).view(torch.bfloat16)]
        for i in range(1, nsets):
            srcs.append(srcs[0].clone())
        R, Cc = A.shape
        quant = {}
        arms = [(ax, 16, m) for ax in (0, 1, 2) for m in (0, 1)] + [(0, 0, 0), (0, 32, 0), (1, 0, 0),
                                                                   (1, 32, 0)]
        its = args.quant_iters
        for ax, h, m in arms:
            ns_, ss_ = mx.packed_shapes(R, Cc, ax)
            outs = [(torch.empty(ns_, dtype=torch.uint8, device=dev),
                     torch.empty(ss_, dtype=torch.uint8, device=dev)) for _ in range(nsets)]

            def q(i):
                k = i % nsets
                mx.mxfp4_quantize(srcs[k], R, Cc, ax, h, m, outs[k][0], outs[k][1], stream)
            for i in range(10):
                q(i)
            torch.cuda.synchronize()
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(its + 1)]
            evs[0].record(stream)
            for i in range(its):
                q(i)
                evs[i + 1].record(stream)
            torch.cuda.synchronize()
            d = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(its)])
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(its):
                q(i)
            e1.record(stream)
            torch.cuda.synchronize()
            mean_ms = e0.elapsed_time(e1) / its
            b = quant_bytes(R, Cc, ax)
            key = f"{['row', 'col', '2d'][ax]}_h{h}_{['ocp_floor', 'ceil'][m]}"
            quant[key] = {"us": round(mean_ms * 1e3, 2),
                          "GB/s": round(b / (mean_ms * 1e-3) / 1e9, 1),
                          "us_event_median": round(float(np.median(d)) * 1e3, 2),
                          "us_event_min": round(float(d.min()) * 1e3, 2),
                          "GB/s_event_median": round(b / (np.median(d) * 1e-3) / 1e9, 1)}
            quant[key]["frac_hbm"] = round(quant[key]["GB/s"] / HBM_PEAK_GBS, 4)
            del outs
        # dual orientation: one read, row-wise + column-wise transposed outputs
        for m in (0, 1):
            (rn_, rs_), (cn_, cs_) = mx.packed_shapes(R, Cc, 0), mx.packed_shapes(R, Cc, 1)
            outs = [[torch.empty(sh, dtype=torch.uint8, device=dev) for sh in (rn_, rs_, cn_, cs_)]
                    for _ in range(nsets)]

            def qd(i):
                k = i % nsets
                mx.mxfp4_quantize_dual(srcs[k], R, Cc, 16, m, *outs[k], stream=stream)
            for i in range(10):
                qd(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(its):
                qd(i)
            e1.record(stream)
            torch.cuda.synchronize()
            mean_ms = e0.elapsed_time(e1) / its
            b = R * Cc * (2 + 2 * (0.5 + 1 / 32))
            key = f"dual_h16_{['ocp_floor', 'ceil'][m]}"
            quant[key] = {"us": round(mean_ms * 1e3, 2), "GB/s": round(b / (mean_ms * 1e-3) / 1e9, 1),
                          "frac_hbm": round(b / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            if f"row_h16_{['ocp_floor', 'ceil'][m]}" in quant:
                quant[key]["speedup_vs_row_plus_col"] = round(
                    (quant[f"row_h16_{['ocp_floor', 'ceil'][m]}"]["us"] +
                     quant[f"col_h16_{['ocp_floor', 'ceil'][m]}"]["us"]) / (mean_ms * 1e3), 3)
            del outs
        # outlier fallback: q1 and the half-residual q2 in one pass (2x the output)
        for ax, m in ((0, 0), (0, 1), (1, 0)):
            Ro, Ko = (R, Cc) if ax == 0 else (Cc, R)
            outs = [(torch.empty((Ro, Ko), dtype=torch.uint8, device=dev),
                     torch.empty((Ro, 2 * Ko // 32), dtype=torch.uint8, device=dev))
                    for _ in range(nsets)]

            def qo(i):
                k = i % nsets
                mx.mxfp4_quantize_of(srcs[k], R, Cc, ax, 16, m, outs[k][0], outs[k][1], stream)
            for i in range(10):
                qo(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(its):
                qo(i)
            e1.record(stream)
            torch.cuda.synchronize()
            mean_ms = e0.elapsed_time(e1) / its
            b = R * Cc * (2 + 2 * (0.5 + 1 / 32))
            quant[f"of_{['row', 'col'][ax]}_h16_{['ocp_floor', 'ceil'][m]}"] = {
                "us": round(mean_ms * 1e3, 2), "GB/s": round(b / (mean_ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del outs
        # macro-block scaling: prescaled operand + one mantissa byte per 128
        for ax in (0, 1):
            ns_, ss_ = mx.packed_shapes(R, Cc, ax)
            ms_ = (R, Cc // 128) if ax == 0 else (Cc, R // 128)
            outs = [[torch.empty(sh, dtype=torch.uint8, device=dev) for sh in (ns_, ss_, ms_)]
                    for _ in range(nsets)]

            def qm(i):
                k = i % nsets
                mx.mxfp4_quantize_mbs(srcs[k], R, Cc, ax, 16, 1, *outs[k], stream=stream)
            for i in range(10):
                qm(i)
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            for i in range(its):
                qm(i)
            e1.record(stream)
            torch.cuda.synchronize()
            mean_ms = e0.elapsed_time(e1) / its
            b = R * Cc * (2 + 0.5 + 1 / 32 + 1 / 128)
            quant[f"mbs_{['row', 'col'][ax]}_h16_ceil"] = {
                "us": round(mean_ms * 1e3, 2), "GB/s": round(b / (mean_ms * 1e-3) / 1e9, 1),
                "frac_hbm": round(b / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del outs
        # comparison arms: random-sign H16 (signs along the blocked axis) and
        # stochastic rounding (one 32-bit random integer per element, read too)
        for ax in (0, 1):
            ns_, ss_ = mx.packed_shapes(R, Cc, ax)
            outs = [(torch.empty(ns_, dtype=torch.uint8, device=dev),
                     torch.empty(ss_, dtype=torch.uint8, device=dev)) for _ in range(nsets)]
            signs = torch.from_numpy(synthetic.random_signs(Cc if ax == 0 else R, 51)).to(dev)
            rnd = [torch.from_numpy(synthetic.random_u32((R, Cc), 52 + k).view(np.int32)).to(dev)
                   for k in range(2)]
            for arm in ("rs", "sr"):
                def qa(i):
                    k = i % nsets
                    if arm == "rs":
                        mx.mxfp4_quantize_rs(srcs[k], R, Cc, ax, 16, 0, signs, outs[k][0],
                                             outs[k][1], stream)
                    else:
                        mx.mxfp4_quantize_sr(srcs[k], R, Cc, ax, 16, 0, rnd[i % 2], outs[k][0],
                                             outs[k][1], stream)
                for i in range(10):
                    qa(i)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in range(its):
                    qa(i)
                e1.record(stream)
                torch.cuda.synchronize()
                mean_ms = e0.elapsed_time(e1) / its
                b = quant_bytes(R, Cc, ax) + (4 * R * Cc if arm == "sr" else 0)
                quant[f"{arm}_{['row', 'col'][ax]}_h16_ocp_floor"] = {
                    "us": round(mean_ms * 1e3, 2), "GB/s": round(b / (mean_ms * 1e-3) / 1e9, 1),
                    "frac_hbm": round(b / (mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
            del outs, rnd, signs
        if "row_h16_ocp_floor" in quant and "row_h32_ocp_floor" in quant:
            quant["h16_over_h32_row"] = round(quant["row_h16_ocp_floor"]["GB/s"] /
                                              quant["row_h32_ocp_floor"]["GB/s"], 3)
        # achievable-HBM reference: 1 GiB device-to-device copy (read + write)
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            dst.copy_(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(10):
            dst.copy_(src)
        e1.record(stream)
        torch.cuda.synchronize()
        quant["hbm_copy_GB/s"] = round(2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
        del src, dst
        log("quantizer arms done")

    # ------------------------------------------------------- error report
    errs = decomp = None
    if not args.no_error_report:
        errs = error_report(mx, torch, prods, stream, dev)
        decomp = error_decomposition(mx, torch, synthetic, np, prods, stream, dev)
        log("error report done")

    # ---------------------------------------------------------- timed region
    # After the other GPU sections (they bring the GPU to its sustained
    # clocks): W untimed warm-up steps, then exactly K steps between two
    # synchronizations.
    for _ in range(args.warmup):
        for _, _, fn in seq:
            fn()
    torch.cuda.synchronize()
    e_t0, e_t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t_start = time.perf_counter()
    e_t0.record(stream)
    for s in range(K_):
        for _, _, fn in seq:
            fn()
    e_t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_start
    ms_per_step = wall * 1e3 / K_
    event_ms_per_step = e_t0.elapsed_time(e_t1) / K_
    value = total_flops / (ms_per_step * 1e-3) / 1e12
    log(f"step {ms_per_step:.3f} ms, {value:.1f} TFLOP/s")

    # the same step with ceiling-rounded scales (the rule that keeps the
    # heavy-tailed Wgrad operand from clipping; same kernels otherwise)
    seq_ceil = [fn for p in prods for fn in launches(p, 1)]
    for fn in seq_ceil:
        fn()
    torch.cuda.synchronize()
    t_c = time.perf_counter()
    for s in range(K_):
        for fn in seq_ceil:
            fn()
    torch.cuda.synchronize()
    ceil_ms_per_step = (time.perf_counter() - t_c) * 1e3 / K_

    # the same step through the fused entry points (mxfp4_fprop / dgrad /
    # wgrad, workspace-resident operands): a cross-check of the launch
    # sequence above, timed the same way while the GPU is at the same clocks
    fused_step()
    torch.cuda.synchronize()
    t_f = time.perf_counter()
    for _ in range(K_):
        fused_step()
    torch.cuda.synchronize()
    fused_ms = (time.perf_counter() - t_f) * 1e3 / K_

    # the same step captured once in a HIP graph (the library allocates and
    # synchronizes nothing, so its launches are capturable) and replayed K
    # times: a cross-check that host launch overhead is not in the headline
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side), torch.cuda.graph(graph, stream=side):
        for p in prods:
            for fn in launches(p, 0, side):
                fn()
    stream.wait_stream(side)
    graph.replay()
    torch.cuda.synchronize()
    t_g = time.perf_counter()
    for _ in range(K_):
        graph.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t_g) * 1e3 / K_
    del graph

    # -------------------------------------------------------------- roofline
    dom = [k for k in kernels if k["kernel"] == f"{DOMINANT}.gemm"][0]
    dp = [p for p in prods if p["name"] == DOMINANT][0]
    gemm_src = os.path.join(ROOT, "mxfp4_quantized_gemm_amd", "csrc", "gemm.hip")
    roofline = {"kernel": f"mxfp4 GEMM {DOMINANT} (M,N,K)=({dp['GM']},{dp['GN']},{dp['GK']})",
                "bound": "mfma", "achieved": dom["TFLOP/s"], "peak": MXFP4_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(dom["TFLOP/s"] / MXFP4_PEAK_TFLOPS, 4),
                "traffic": load_traffic(gemm_src)}

    cpu = None if args.no_cpu_baseline else cpu_baseline(work)
    if cpu:
        log(f"cpu baseline {cpu['value']:.4f} TFLOP/s in {cpu['seconds']} s")

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K_, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "mxfp4",
        "data": "synthetic",
        "config": {"workload": "llama3.1-8b linear products at 8192 tokens: qkv fprop "
                               "(T,N,K)=(8192,6144,4096), mlp gate+up fprop (8192,28672,4096), "
                               "down-proj dgrad (8192,4096,14336), down-proj wgrad "
                               "(8192,4096,14336); H16 along each reduction axis, 1x32 row / "
                               "32x1 col blocks, ocp_floor scales, fp32 out",
                   "hadamard": 16, "scale_mode": "ocp_floor", "out_dtype": "f32",
                   "parallelism": "single-gpu"},
        # the long reports first, so that the end of the line (what a log
        # tail keeps) holds the per-kernel times, quantizer rates, roofline
        # and CPU baseline
        "error_report": errs,
        "error_decomposition": decomp,
        "products": per_product,
        "event_ms_per_step": round(event_ms_per_step, 4),
        "fused_entry_ms_per_step": round(fused_ms, 4),
        "graph_replay_ms_per_step": round(graph_ms, 4),
        "ceil_scales_ms_per_step": round(ceil_ms_per_step, 4),
        "ceil_scales_TFLOP/s": round(total_flops / (ceil_ms_per_step * 1e-3) / 1e12, 2),
        "kernels": kernels,
        "quantizer": quant,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
