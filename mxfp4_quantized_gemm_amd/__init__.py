"""Python binding of libmxfp4 (MI355X / gfx950 H16 + MXFP4 quantize + GEMM).

Thin ctypes marshalling over the C ABI declared in ``include/mxfp4.h``: the
functions below carry the C names, take torch tensors (device memory) and
the current HIP stream, check shapes and dtypes, and call the library.
Every step of the computation runs in the library's HIP kernels; there is no
fallback. If ``libmxfp4.so`` has not been built, every call raises.

Layouts (see the header): bf16 sources are row-major; a packed MXFP4
operand is ``nibbles`` (uint8, two E2M1 codes per byte, element 2j in the
low nibble) plus ``e8m0`` (uint8, one scale byte per 32-element block).
"""
from __future__ import annotations

import ctypes
import os

AXIS_ROW, AXIS_COL, AXIS_2D32 = 0, 1, 2
SCALE_OCP_FLOOR, SCALE_CEIL = 0, 1
OUT_F32, OUT_BF16 = 0, 1
OP_FPROP, OP_DGRAD, OP_WGRAD = 0, 1, 2
ERROR_STATS_COUNT = 10
ERROR_STATS_WS_BYTES = 1024 * ERROR_STATS_COUNT * 8
ERROR_STATS_FIELDS = ("sum_e_scale2", "sum_e_dz2", "sum_e_grid2", "dot_scale_grid",
                      "dot_scale_dz", "sum_e2", "sum_x2", "n_deadzone", "n_elements",
                      "n_nonfinite_blocks")

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmxfp4.so")

EXPORTS = (
    "mxfp4_quantize", "mxfp4_quantize_pair", "mxfp4_quantize_dual", "mxfp4_quantize_of", "mxfp4_quantize_mbs",
    "mxfp4_quantize_rs", "mxfp4_quantize_sr", "mxfp4_error_stats",
    "mxfp4_error_stats_noalloc", "mxfp4_gemm", "mxfp4_gemm_mbs", "mxfp4_fprop", "mxfp4_dgrad", "mxfp4_wgrad",
    "mxfp4_workspace_bytes", "mxfp4_status_string",
)

_LIB = None


class MXFP4Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)} ({status})")


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libmxfp4.so (once) and declare the C signatures."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is missing: build it with `python -m mxfp4_quantized_gemm_amd.build`")
    lib = ctypes.CDLL(path)
    p, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_size_t
    lib.mxfp4_quantize.argtypes = [p, i64, i64, i32, i32, i32, p, p, p]
    lib.mxfp4_quantize.restype = i32
    lib.mxfp4_quantize_pair.argtypes = [p, i64, i64, i32, p, p, p, i64, i64, i32, p, p, i32, i32, p]
    lib.mxfp4_quantize_pair.restype = i32
    lib.mxfp4_quantize_dual.argtypes = [p, i64, i64, i32, i32, p, p, p, p, p]
    lib.mxfp4_quantize_dual.restype = i32
    lib.mxfp4_quantize_of.argtypes = [p, i64, i64, i32, i32, i32, p, p, p]
    lib.mxfp4_quantize_of.restype = i32
    lib.mxfp4_quantize_mbs.argtypes = [p, i64, i64, i32, i32, i32, p, p, p, p]
    lib.mxfp4_quantize_mbs.restype = i32
    lib.mxfp4_quantize_rs.argtypes = [p, i64, i64, i32, i32, i32, p, p, p, p]
    lib.mxfp4_quantize_rs.restype = i32
    lib.mxfp4_quantize_sr.argtypes = [p, i64, i64, i32, i32, i32, p, p, p, p]
    lib.mxfp4_quantize_sr.restype = i32
    lib.mxfp4_error_stats.argtypes = [p, i64, i64, i32, i32, i32, p, sz, p, p]
    lib.mxfp4_error_stats.restype = i32
    lib.mxfp4_error_stats_noalloc.argtypes = [p, i64, i64, i32, i32, i32, p, p]
    lib.mxfp4_error_stats_noalloc.restype = i32
    lib.mxfp4_gemm.argtypes = [p, p, p, p, i64, i64, i64, p, i32, p]
    lib.mxfp4_gemm.restype = i32
    lib.mxfp4_gemm_mbs.argtypes = [p, p, p, p, p, p, i64, i64, i64, p, i32, p]
    lib.mxfp4_gemm_mbs.restype = i32
    for name in ("mxfp4_fprop", "mxfp4_dgrad", "mxfp4_wgrad"):
        fn = getattr(lib, name)
        fn.argtypes = [p, p, i64, i64, i64, i32, i32, p, sz, p, i32, p]
        fn.restype = i32
    lib.mxfp4_workspace_bytes.argtypes = [i32, i64, i64, i64]
    lib.mxfp4_workspace_bytes.restype = sz
    lib.mxfp4_status_string.argtypes = [i32]
    lib.mxfp4_status_string.restype = ctypes.c_char_p
    _LIB = lib
    return lib


def status_string(status: int) -> str:
    return load_library().mxfp4_status_string(int(status)).decode()


def _check(status: int, where: str) -> None:
    if status != 0:
        raise MXFP4Error(status, where)


def _stream(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _need(t, dtype, numel, name):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must live in GPU memory")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() < numel:
        raise ValueError(f"{name} holds {t.numel()} elements, needs {numel}")


# ----------------------------------------------------------------- C calls
def mxfp4_quantize(src, rows, cols, axis, hadamard, scale_mode, out_nibbles, out_e8m0,
                   stream=None):
    """Rotate + quantize ``src`` (bf16 [rows][cols]) into caller buffers."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    nib, nsc = packed_sizes(rows, cols, axis)
    _need(out_nibbles, torch.uint8, nib, "out_nibbles")
    _need(out_e8m0, torch.uint8, nsc, "out_e8m0")
    _check(load_library().mxfp4_quantize(_ptr(src), rows, cols, axis, hadamard, scale_mode,
                                         _ptr(out_nibbles), _ptr(out_e8m0), _stream(stream)),
           "mxfp4_quantize")


def mxfp4_quantize_pair(src_a, rows_a, cols_a, axis_a, nibbles_a, e8m0_a, src_b, rows_b, cols_b,
                        axis_b, nibbles_b, e8m0_b, hadamard, scale_mode, stream=None):
    """Both operands of a product (each as mxfp4_quantize) in one launch
    where the shapes allow it."""
    import torch
    for src, rows, cols, axis, nb, sc, w in ((src_a, rows_a, cols_a, axis_a, nibbles_a, e8m0_a, "a"),
                                             (src_b, rows_b, cols_b, axis_b, nibbles_b, e8m0_b, "b")):
        _need(src, torch.bfloat16, rows * cols, "src_" + w)
        n, ns = packed_sizes(rows, cols, axis)
        _need(nb, torch.uint8, n, "nibbles_" + w)
        _need(sc, torch.uint8, ns, "e8m0_" + w)
    _check(load_library().mxfp4_quantize_pair(
        _ptr(src_a), rows_a, cols_a, axis_a, _ptr(nibbles_a), _ptr(e8m0_a), _ptr(src_b), rows_b,
        cols_b, axis_b, _ptr(nibbles_b), _ptr(e8m0_b), hadamard, scale_mode, _stream(stream)),
        "mxfp4_quantize_pair")


def mxfp4_quantize_dual(src, rows, cols, hadamard, scale_mode, row_nibbles, row_e8m0,
                        col_nibbles, col_e8m0, stream=None):
    """One read of ``src`` (bf16 [rows][cols]); row-wise and column-wise
    transposed packed operands into caller buffers."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(row_nibbles, torch.uint8, rows * cols // 2, "row_nibbles")
    _need(row_e8m0, torch.uint8, rows * cols // 32, "row_e8m0")
    _need(col_nibbles, torch.uint8, rows * cols // 2, "col_nibbles")
    _need(col_e8m0, torch.uint8, rows * cols // 32, "col_e8m0")
    _check(load_library().mxfp4_quantize_dual(
        _ptr(src), rows, cols, hadamard, scale_mode, _ptr(row_nibbles), _ptr(row_e8m0),
        _ptr(col_nibbles), _ptr(col_e8m0), _stream(stream)), "mxfp4_quantize_dual")


def mxfp4_quantize_of(src, rows, cols, axis, hadamard, scale_mode, out_nibbles, out_e8m0,
                      stream=None):
    """Outlier-fallback operand (twice as deep as mxfp4_quantize's)."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(out_nibbles, torch.uint8, rows * cols, "out_nibbles")
    _need(out_e8m0, torch.uint8, rows * cols // 16, "out_e8m0")
    _check(load_library().mxfp4_quantize_of(_ptr(src), rows, cols, axis, hadamard, scale_mode,
                                            _ptr(out_nibbles), _ptr(out_e8m0), _stream(stream)),
           "mxfp4_quantize_of")


def mxfp4_quantize_rs(src, rows, cols, axis, hadamard, scale_mode, signs, out_nibbles, out_e8m0,
                      stream=None):
    """Random-sign Hadamard comparison arm: signs is a uint8 tensor with one
    byte per index of the blocked axis (bit 0 set = flip)."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(signs, torch.uint8, cols if axis == AXIS_ROW else rows, "signs")
    _need(out_nibbles, torch.uint8, rows * cols // 2, "out_nibbles")
    _need(out_e8m0, torch.uint8, rows * cols // 32, "out_e8m0")
    _check(load_library().mxfp4_quantize_rs(_ptr(src), rows, cols, axis, hadamard, scale_mode,
                                            _ptr(signs), _ptr(out_nibbles), _ptr(out_e8m0),
                                            _stream(stream)), "mxfp4_quantize_rs")


def mxfp4_quantize_sr(src, rows, cols, axis, hadamard, scale_mode, rand_u32, out_nibbles,
                      out_e8m0, stream=None):
    """Stochastic-rounding comparison arm: rand_u32 holds one 32-bit integer
    per source element ([rows][cols], any 4-byte dtype, e.g. torch.int32)."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(rand_u32, torch.uint32 if rand_u32.dtype == torch.uint32 else torch.int32, rows * cols,
          "rand_u32")
    _need(out_nibbles, torch.uint8, rows * cols // 2, "out_nibbles")
    _need(out_e8m0, torch.uint8, rows * cols // 32, "out_e8m0")
    _check(load_library().mxfp4_quantize_sr(_ptr(src), rows, cols, axis, hadamard, scale_mode,
                                            _ptr(rand_u32), _ptr(out_nibbles), _ptr(out_e8m0),
                                            _stream(stream)), "mxfp4_quantize_sr")


def mxfp4_quantize_mbs(src, rows, cols, axis, hadamard, scale_mode, out_nibbles, out_e8m0,
                       out_mbs, stream=None):
    """Macro-block-scaled operand: nibbles and E8M0 of the prescaled values
    plus one mantissa byte per 128 elements."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(out_nibbles, torch.uint8, rows * cols // 2, "out_nibbles")
    _need(out_e8m0, torch.uint8, rows * cols // 32, "out_e8m0")
    _need(out_mbs, torch.uint8, rows * cols // 128, "out_mbs")
    _check(load_library().mxfp4_quantize_mbs(_ptr(src), rows, cols, axis, hadamard, scale_mode,
                                             _ptr(out_nibbles), _ptr(out_e8m0), _ptr(out_mbs),
                                             _stream(stream)), "mxfp4_quantize_mbs")


def mxfp4_error_stats(src, rows, cols, axis, hadamard, scale_mode, ws, out_stats, stream=None):
    """Error-decomposition sums of the quantized ``src`` into ``out_stats``
    (float64, 10 values; see the header for their order)."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(ws, torch.uint8, ERROR_STATS_WS_BYTES, "ws")
    _need(out_stats, torch.float64, ERROR_STATS_COUNT, "out_stats")
    _check(load_library().mxfp4_error_stats(_ptr(src), rows, cols, axis, hadamard, scale_mode,
                                            _ptr(ws), ws.numel(), _ptr(out_stats),
                                            _stream(stream)), "mxfp4_error_stats")


def mxfp4_error_stats_noalloc(src, rows, cols, axis, hadamard, scale_mode, out_stats,
                              stream=None):
    """mxfp4_error_stats with the library's static partial-sum array
    instead of a workspace (allocates nothing)."""
    import torch
    _need(src, torch.bfloat16, rows * cols, "src")
    _need(out_stats, torch.float64, ERROR_STATS_COUNT, "out_stats")
    _check(load_library().mxfp4_error_stats_noalloc(_ptr(src), rows, cols, axis, hadamard,
                                                    scale_mode, _ptr(out_stats),
                                                    _stream(stream)),
           "mxfp4_error_stats_noalloc")


def mxfp4_gemm(Aq, As, Bq, Bs, M, N, K, C, out_dtype=OUT_F32, stream=None):
    """C[M][N] = deq(A) deq(B)^T from packed K-contiguous operands."""
    import torch
    _need(Aq, torch.uint8, M * K // 2, "Aq")
    _need(As, torch.uint8, M * K // 32, "As")
    _need(Bq, torch.uint8, N * K // 2, "Bq")
    _need(Bs, torch.uint8, N * K // 32, "Bs")
    _need(C, torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, M * N, "C")
    _check(load_library().mxfp4_gemm(_ptr(Aq), _ptr(As), _ptr(Bq), _ptr(Bs), M, N, K, _ptr(C),
                                     out_dtype, _stream(stream)), "mxfp4_gemm")


def mxfp4_gemm_mbs(Aq, As, Am, Bq, Bs, Bm, M, N, K, C, out_dtype=OUT_F32, stream=None):
    """C[M][N] = (deq(A) / cA) (deq(B) / cB)^T from two MBS operands."""
    import torch
    _need(Aq, torch.uint8, M * K // 2, "Aq")
    _need(As, torch.uint8, M * K // 32, "As")
    _need(Am, torch.uint8, M * K // 128, "Am")
    _need(Bq, torch.uint8, N * K // 2, "Bq")
    _need(Bs, torch.uint8, N * K // 32, "Bs")
    _need(Bm, torch.uint8, N * K // 128, "Bm")
    _need(C, torch.float32 if out_dtype == OUT_F32 else torch.bfloat16, M * N, "C")
    _check(load_library().mxfp4_gemm_mbs(_ptr(Aq), _ptr(As), _ptr(Am), _ptr(Bq), _ptr(Bs),
                                         _ptr(Bm), M, N, K, _ptr(C), out_dtype,
                                         _stream(stream)), "mxfp4_gemm_mbs")


def _fused(name, op, P, Q, T, N, K, hadamard, scale_mode, ws, out, out_dtype, stream, pshape,
           qshape, oshape):
    import torch
    _need(P, torch.bfloat16, pshape[0] * pshape[1], "first operand")
    _need(Q, torch.bfloat16, qshape[0] * qshape[1], "second operand")
    _need(out, torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
          oshape[0] * oshape[1], "output")
    need = mxfp4_workspace_bytes(op, T, N, K)
    _need(ws, torch.uint8, need, "workspace")
    _check(getattr(load_library(), name)(_ptr(P), _ptr(Q), T, N, K, hadamard, scale_mode,
                                         _ptr(ws), ws.numel(), _ptr(out), out_dtype,
                                         _stream(stream)), name)


def mxfp4_fprop(X, W, T, N, K, hadamard, scale_mode, ws, Y, out_dtype=OUT_F32, stream=None):
    """Y[T][N] = X[T][K] W[N][K]^T (both operands rotated along K)."""
    _fused("mxfp4_fprop", OP_FPROP, X, W, T, N, K, hadamard, scale_mode, ws, Y, out_dtype,
           stream, (T, K), (N, K), (T, N))


def mxfp4_dgrad(dY, W, T, N, K, hadamard, scale_mode, ws, dX, out_dtype=OUT_F32, stream=None):
    """dX[T][K] = dY[T][N] W[N][K] (both rotated along N)."""
    _fused("mxfp4_dgrad", OP_DGRAD, dY, W, T, N, K, hadamard, scale_mode, ws, dX, out_dtype,
           stream, (T, N), (N, K), (T, K))


def mxfp4_wgrad(dY, X, T, N, K, hadamard, scale_mode, ws, dW, out_dtype=OUT_F32, stream=None):
    """dW[N][K] = dY[T][N]^T X[T][K] (both rotated along T)."""
    _fused("mxfp4_wgrad", OP_WGRAD, dY, X, T, N, K, hadamard, scale_mode, ws, dW, out_dtype,
           stream, (T, N), (T, K), (N, K))


def mxfp4_workspace_bytes(op, T, N, K) -> int:
    return int(load_library().mxfp4_workspace_bytes(op, T, N, K))


def mxfp4_status_string(status: int) -> str:
    return status_string(status)


# ------------------------------------------------------ allocating helpers
def packed_sizes(rows, cols, axis):
    """(nibble bytes, scale bytes) of ``mxfp4_quantize``'s outputs."""
    if axis == AXIS_2D32:
        return rows * cols // 2, (rows // 32) * (cols // 32)
    return rows * cols // 2, rows * cols // 32


def packed_shapes(rows, cols, axis):
    """Shapes of (nibbles, e8m0) for a bf16 [rows][cols] source."""
    if axis == AXIS_COL:
        return (cols, rows // 2), (cols, rows // 32)
    if axis == AXIS_2D32:
        return (rows, cols // 2), (rows // 32, cols // 32)
    return (rows, cols // 2), (rows, cols // 32)


def quantize(src, axis=AXIS_ROW, hadamard=16, scale_mode=SCALE_OCP_FLOOR, stream=None):
    """Allocate outputs and quantize; returns (nibbles, e8m0) uint8 tensors."""
    import torch
    rows, cols = src.shape
    ns, ss = packed_shapes(rows, cols, axis)
    nib = torch.empty(ns, dtype=torch.uint8, device=src.device)
    sc = torch.empty(ss, dtype=torch.uint8, device=src.device)
    mxfp4_quantize(src, rows, cols, axis, hadamard, scale_mode, nib, sc, stream)
    return nib, sc


def quantize_dual(src, hadamard=16, scale_mode=SCALE_OCP_FLOOR, stream=None):
    """Allocate outputs and quantize both orientations with one read; returns
    ((row_nibbles, row_e8m0), (col_nibbles, col_e8m0))."""
    import torch
    rows, cols = src.shape
    (rn, rs), (cn, cs) = packed_shapes(rows, cols, AXIS_ROW), packed_shapes(rows, cols, AXIS_COL)
    out = [torch.empty(sh, dtype=torch.uint8, device=src.device) for sh in (rn, rs, cn, cs)]
    mxfp4_quantize_dual(src, rows, cols, hadamard, scale_mode, *out, stream=stream)
    return (out[0], out[1]), (out[2], out[3])


def quantize_of(src, axis=AXIS_ROW, hadamard=16, scale_mode=SCALE_OCP_FLOOR, stream=None):
    """Allocate and compute the OF operand; returns (nibbles [R][Kb],
    e8m0 [R][2 Kb / 32]) with R, Kb = rows, cols (ROW) or cols, rows (COL)."""
    import torch
    rows, cols = src.shape
    R, Kb = (rows, cols) if axis == AXIS_ROW else (cols, rows)
    nib = torch.empty((R, Kb), dtype=torch.uint8, device=src.device)
    sc = torch.empty((R, 2 * Kb // 32), dtype=torch.uint8, device=src.device)
    mxfp4_quantize_of(src, rows, cols, axis, hadamard, scale_mode, nib, sc, stream)
    return nib, sc


def quantize_rs(src, signs, axis=AXIS_ROW, hadamard=16, scale_mode=SCALE_OCP_FLOOR, stream=None):
    """Allocate and compute the random-sign Hadamard operand (nibbles, e8m0)."""
    import torch
    rows, cols = src.shape
    ns, ss = packed_shapes(rows, cols, axis)
    nib = torch.empty(ns, dtype=torch.uint8, device=src.device)
    sc = torch.empty(ss, dtype=torch.uint8, device=src.device)
    mxfp4_quantize_rs(src, rows, cols, axis, hadamard, scale_mode, signs, nib, sc, stream)
    return nib, sc


def quantize_sr(src, rand_u32, axis=AXIS_ROW, hadamard=16, scale_mode=SCALE_OCP_FLOOR,
                stream=None):
    """Allocate and compute the stochastic-rounding operand (nibbles, e8m0)."""
    import torch
    rows, cols = src.shape
    ns, ss = packed_shapes(rows, cols, axis)
    nib = torch.empty(ns, dtype=torch.uint8, device=src.device)
    sc = torch.empty(ss, dtype=torch.uint8, device=src.device)
    mxfp4_quantize_sr(src, rows, cols, axis, hadamard, scale_mode, rand_u32, nib, sc, stream)
    return nib, sc


def quantize_mbs(src, axis=AXIS_ROW, hadamard=16, scale_mode=SCALE_CEIL, stream=None):
    """Allocate and compute the MBS operand; returns (nibbles, e8m0, mbs)."""
    import torch
    rows, cols = src.shape
    ns, ss = packed_shapes(rows, cols, axis)
    ms = (rows, cols // 128) if axis == AXIS_ROW else (cols, rows // 128)
    out = [torch.empty(sh, dtype=torch.uint8, device=src.device) for sh in (ns, ss, ms)]
    mxfp4_quantize_mbs(src, rows, cols, axis, hadamard, scale_mode, *out, stream=stream)
    return tuple(out)


def error_stats(src, axis=AXIS_ROW, hadamard=16, scale_mode=SCALE_OCP_FLOOR, stream=None,
                ws=None):
    """Run mxfp4_error_stats; returns a dict of the ten sums plus the derived
    cosine(e_scale, e_grid) and deadzone fraction (synchronizes)."""
    import torch
    rows, cols = src.shape
    if ws is None:
        ws = torch.empty(ERROR_STATS_WS_BYTES, dtype=torch.uint8, device=src.device)
    out = torch.empty(ERROR_STATS_COUNT, dtype=torch.float64, device=src.device)
    mxfp4_error_stats(src, rows, cols, axis, hadamard, scale_mode, ws, out, stream)
    v = out.cpu().tolist()
    d = dict(zip(ERROR_STATS_FIELDS, v))
    den = (d["sum_e_scale2"] * d["sum_e_grid2"]) ** 0.5
    d["cos_scale_grid"] = d["dot_scale_grid"] / den if den > 0 else float("nan")
    d["deadzone_fraction"] = d["n_deadzone"] / d["n_elements"] if d["n_elements"] else float("nan")
    return d


def gemm(Aq, As, Bq, Bs, out_dtype=OUT_F32, stream=None):
    """Allocate C and run the MXFP4 GEMM on packed operands."""
    import torch
    M, kh = Aq.shape
    N = Bq.shape[0]
    C = torch.empty((M, N), dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                    device=Aq.device)
    mxfp4_gemm(Aq, As, Bq, Bs, M, N, 2 * kh, C, out_dtype, stream)
    return C


def linear(op, P, Q, hadamard=16, scale_mode=SCALE_OCP_FLOOR, out_dtype=OUT_F32, ws=None,
           stream=None):
    """One fused product ('fprop', 'dgrad' or 'wgrad'); allocates the output."""
    import torch
    if op == "fprop":
        T, K = P.shape
        N = Q.shape[0]
        oshape, fn, code = (T, N), mxfp4_fprop, OP_FPROP
    elif op == "dgrad":
        T, N = P.shape
        K = Q.shape[1]
        oshape, fn, code = (T, K), mxfp4_dgrad, OP_DGRAD
    elif op == "wgrad":
        T, N = P.shape
        K = Q.shape[1]
        oshape, fn, code = (N, K), mxfp4_wgrad, OP_WGRAD
    else:
        raise ValueError(op)
    if ws is None:
        ws = torch.empty(mxfp4_workspace_bytes(code, T, N, K), dtype=torch.uint8, device=P.device)
    out = torch.empty(oshape, dtype=torch.float32 if out_dtype == OUT_F32 else torch.bfloat16,
                      device=P.device)
    fn(P, Q, T, N, K, hadamard, scale_mode, ws, out, out_dtype, stream)
    return out
