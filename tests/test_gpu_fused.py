"""GPU parity of the fused linear-layer products (mxfp4_fprop / dgrad / wgrad
through the C ABI) against the oracle.

Each product quantizes both operands into the caller's workspace and runs
the GEMM. The tests check (1) the packed operands left in the workspace,
bit-exactly, and (2) the output against the oracle's fp64 GEMM of the
oracle's dequantized operands (|C - C_ref| <= 1e-5 sum|a||b|, plus 2^-8
|C_ref| for bf16 output). Small ragged shapes are checked in full; the four
Llama-3.1-8B products at full size are checked on sampled output rows and
columns for every rotation, rule and output type, with the sampled operand
rows quantized by the oracle from the matching source slices; with
H16 and OCP floor scales all four are also checked on every output element
and every operand byte.
"""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

OPS = {"fprop": 0, "dgrad": 1, "wgrad": 2}


def r256(x):
    return (x + 255) // 256 * 256


def operand_layout(op, T, N, K):
    """(rows, kbytes) of the A and B packed operands, and GEMM (M, N, K)."""
    if op == "fprop":
        return (T, K), (N, K), (T, N, K)
    if op == "dgrad":
        return (T, N), (K, N), (T, K, N)
    return (N, T), (K, T), (N, K, T)


def run_fused(op, P, Q, T, N, K, h, mode, out_dtype=0):
    """Returns (C, (A nib, A sc), (B nib, B sc)) read back from the GPU."""
    import torch
    import mxfp4_quantized_gemm_amd as mx
    p, q = to_dev_bf16(P), to_dev_bf16(Q)
    ws = torch.empty(mx.mxfp4_workspace_bytes(OPS[op], T, N, K), dtype=torch.uint8, device="cuda")
    (ra, ka), (rb, kb), (GM, GN, GK) = operand_layout(op, T, N, K)
    out = torch.empty((GM, GN), dtype=torch.float32 if out_dtype == 0 else torch.bfloat16,
                      device="cuda")
    fn = {"fprop": mx.mxfp4_fprop, "dgrad": mx.mxfp4_dgrad, "wgrad": mx.mxfp4_wgrad}[op]
    fn(p, q, T, N, K, h, mode, ws, out, out_dtype)
    torch.cuda.synchronize()
    w = ws.cpu().numpy()
    o = 0
    a_nib = w[o:o + ra * ka // 2].reshape(ra, ka // 2); o += r256(ra * ka // 2)
    a_sc = w[o:o + ra * ka // 32].reshape(ra, ka // 32); o += r256(ra * ka // 32)
    b_nib = w[o:o + rb * kb // 2].reshape(rb, kb // 2); o += r256(rb * kb // 2)
    b_sc = w[o:o + rb * kb // 32].reshape(rb, kb // 32)
    return out.float().cpu().numpy().astype(np.float64), (a_nib, a_sc), (b_nib, b_sc)


def check_output(C, qa, qb, out_bf16, what):
    Cr, S = O.gemm_ref(O.dequantize(*qa), O.dequantize(*qb))
    tol = O.gemm_tolerance(S, Cr, out_bf16)
    bad = ~(np.abs(C - Cr) <= tol)
    assert np.all(C[S == 0] == 0), what
    if bad.any():
        i, j = np.argwhere(bad)[0]
        pytest.fail(f"{what}: {bad.sum()} out of tolerance, C[{i},{j}]={C[i, j]!r} "
                    f"ref={Cr[i, j]!r} S={S[i, j]!r}")


def small_operands(op, T, N, K, seed):
    rng = np.random.default_rng(seed)
    def heavy(r, c):
        return synthetic.f64_to_bf16_bits(rng.standard_t(4, size=(r, c)) *
                                          rng.lognormal(0, 1, size=(1, c)))
    if op == "fprop":
        return heavy(T, K), heavy(N, K)
    if op == "dgrad":
        return heavy(T, N), heavy(N, K)
    return heavy(T, N), heavy(T, K)


SMALL = [(128, 256, 256), (96, 64, 160), (64, 96, 32), (160, 200, 288), (32, 33, 64)]


@pytest.mark.parametrize("op", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_fused_small(op, h, mode):
    for i, (T, N, K) in enumerate(SMALL):
        if op == "fprop" and K % 32 or op == "dgrad" and N % 32 or op == "wgrad" and T % 32:
            continue
        P, Q = small_operands(op, T, N, K, 31 * i + h + mode)
        C, ga, gb = run_fused(op, P, Q, T, N, K, h, mode)
        qa, qb = O.product_operands(op, P, Q, h, mode)
        what = f"{op} h={h} mode={mode} T,N,K={(T, N, K)}"
        assert np.array_equal(ga[0], qa[0]) and np.array_equal(ga[1], qa[1]), what + " A bytes"
        assert np.array_equal(gb[0], qb[0]) and np.array_equal(gb[1], qb[1]), what + " B bytes"
        check_output(C, qa, qb, False, what)


def test_tiny_fprop_workload_fp32_and_bf16():
    """The tiny Fprop workload (X 128x256 with 5 outlier channels x40,
    W 256x256), H16, 1x32, OCP floor: every output element."""
    w = synthetic.make("tiny")
    qa, qb = O.product_operands("fprop", w["X"], w["W"], 16, 0)
    for out_dtype in (0, 1):
        C, ga, gb = run_fused("fprop", w["X"], w["W"], 128, 256, 256, 16, 0, out_dtype)
        assert np.array_equal(ga[0], qa[0]) and np.array_equal(ga[1], qa[1])
        assert np.array_equal(gb[0], qb[0]) and np.array_equal(gb[1], qb[1])
        check_output(C, qa, qb, out_dtype == 1, f"tiny fprop out={out_dtype}")


# --------------------------------------------------------------- full size
def sampled_check(op, P, Q, T, N, K, h, mode, out_dtype, nsample=192, seed=0):
    C, ga, gb = run_fused(op, P, Q, T, N, K, h, mode, out_dtype)
    (GM, GN, GK) = operand_layout(op, T, N, K)[2]
    rng = np.random.default_rng(seed)
    I = np.sort(rng.choice(GM, min(nsample, GM), replace=False))
    J = np.sort(rng.choice(GN, min(nsample, GN), replace=False))
    I[0], J[-1] = 0, GN - 1  # include the first row and the last column
    # oracle operands for the sampled GEMM rows only
    if op == "fprop":
        qa = O.quantize(P[I], O.AXIS_ROW, h, mode)
        qb = O.quantize(Q[J], O.AXIS_ROW, h, mode)
    elif op == "dgrad":
        qa = O.quantize(P[I], O.AXIS_ROW, h, mode)
        qb = O.quantize(np.ascontiguousarray(Q[:, J]), O.AXIS_COL, h, mode)
    else:
        qa = O.quantize(np.ascontiguousarray(P[:, I]), O.AXIS_COL, h, mode)
        qb = O.quantize(np.ascontiguousarray(Q[:, J]), O.AXIS_COL, h, mode)
    what = f"{op} full T,N,K={(T, N, K)} h={h} mode={mode}"
    assert np.array_equal(ga[0][I], qa[0]) and np.array_equal(ga[1][I], qa[1]), what + " A bytes"
    assert np.array_equal(gb[0][J], qb[0]) and np.array_equal(gb[1][J], qb[1]), what + " B bytes"
    check_output(C[np.ix_(I, J)], qa, qb, out_dtype == 1, what)
    assert np.all(np.isfinite(C)), what + " non-finite outputs"


@pytest.fixture(scope="module")
def qkv():
    return synthetic.make("qkv")


@pytest.fixture(scope="module")
def mlp():
    return synthetic.make("mlp")


@pytest.fixture(scope="module")
def down_wgrad():
    return synthetic.make("wgrad")


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_qkv_fprop_full(qkv, out_dtype):
    sampled_check("fprop", qkv["X"], qkv["W"], 8192, 6144, 4096, 16, 0, out_dtype)


@pytest.mark.parametrize("out_dtype", [0, 1])
def test_mlp_gate_up_fprop_full(mlp, out_dtype):
    sampled_check("fprop", mlp["X"], mlp["W_gu"], 8192, 28672, 4096, 16, 0, out_dtype)


@pytest.mark.parametrize("h,mode,out_dtype", [(16, 0, 0), (16, 1, 1), (32, 0, 0), (0, 1, 0)])
def test_mlp_down_dgrad_full(mlp, h, mode, out_dtype):
    sampled_check("dgrad", mlp["dY"], mlp["W_down"], 8192, 4096, 14336, h, mode, out_dtype)


@pytest.mark.parametrize("h", [16, 32, 0])
def test_down_wgrad_full(down_wgrad, h):
    sampled_check("wgrad", down_wgrad["dY"], down_wgrad["X"], 8192, 4096, 14336, h, 0, 0)


def test_down_wgrad_full_ceil(down_wgrad):
    sampled_check("wgrad", down_wgrad["dY"], down_wgrad["X"], 8192, 4096, 14336, 16, 1, 0)


def test_down_wgrad_full_bf16_out(down_wgrad):
    sampled_check("wgrad", down_wgrad["dY"], down_wgrad["X"], 8192, 4096, 14336, 16, 1, 1)


def full_check(op, P, Q, T, N, K, h, mode, out_dtype):
    """Every byte of both packed operands against the oracle's quantizer and
    every output element against the oracle's fp64 product."""
    import os
    C, ga, gb = run_fused(op, P, Q, T, N, K, h, mode, out_dtype)
    threads = max(1, len(os.sched_getaffinity(0)))
    axa, axb = {"fprop": (0, 0), "dgrad": (0, 1), "wgrad": (1, 1)}[op]
    qa = O.quantize_chunked(P, axa, h, mode, chunk=64, threads=threads)
    qb = O.quantize_chunked(Q, axb, h, mode, chunk=64, threads=threads)
    what = f"{op} T,N,K={(T, N, K)} h={h} mode={mode} every element"
    for g, w, name in ((ga, qa, "A"), (gb, qb, "B")):
        assert np.array_equal(g[0], w[0]), f"{what}: {name} nibbles"
        assert np.array_equal(g[1], w[1]), f"{what}: {name} scales"
    check_output(C, qa, qb, out_dtype == 1, what)


def test_qkv_fprop_every_element(qkv):
    """The QKV Fprop at full size (8192 x 6144 outputs, K = 4096): all 50 M
    outputs and all operand bytes."""
    full_check("fprop", qkv["X"], qkv["W"], 8192, 6144, 4096, 16, 0, 0)


def test_down_wgrad_every_element(down_wgrad):
    """The down-projection Wgrad at full size (4096 x 14336 outputs, the
    8192-token reduction, both operands column-wise): all 59 M outputs and
    all operand bytes."""
    full_check("wgrad", down_wgrad["dY"], down_wgrad["X"], 8192, 4096, 14336, 16, 0, 0)


def test_down_dgrad_every_element(mlp):
    """The down-projection Dgrad at full size (8192 x 14336 outputs, K = 4096
    along N, W quantized column-wise): all 117 M outputs and all operand
    bytes."""
    full_check("dgrad", mlp["dY"], mlp["W_down"], 8192, 4096, 14336, 16, 0, 0)


def test_gate_up_fprop_every_element(mlp):
    """The MLP gate+up Fprop at full size (8192 x 28672 outputs, K = 4096):
    all 235 M outputs and all operand bytes."""
    full_check("fprop", mlp["X"], mlp["W_gu"], 8192, 28672, 4096, 16, 0, 0)
