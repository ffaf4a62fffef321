"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, its enums match the binding, and argument validation
returns the documented status before any HIP call (no kernel is launched
by any call in this file)."""
import ctypes
import os
import re

import pytest

import mxfp4_quantized_gemm_amd as mx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mxfp4.h")


def header_text():
    with open(HEADER) as f:
        return f.read()


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(mx.LIB_PATH):
        pytest.fail("libmxfp4.so is not built (run __graft_entry__.build())")
    return mx.load_library()


def test_header_declares_the_bound_functions():
    decl = set(re.findall(r"\b(mxfp4_[a-z_0-9]+)\s*\(", re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)))
    assert decl == set(mx.EXPORTS)


def test_library_exports_every_declared_symbol(lib):
    text = re.sub(r"/\*.*?\*/", "", header_text(), flags=re.S)
    for name in set(re.findall(r"\b(mxfp4_[a-z_0-9]+)\s*\(", text)):
        assert hasattr(lib, name), name
        assert ctypes.cast(getattr(lib, name), ctypes.c_void_p).value


def test_enums_match_binding():
    text = header_text()
    def val(name):
        m = re.search(rf"\b{name}\s*=\s*(\d+)", text)
        assert m, name
        return int(m.group(1))
    assert val("MXFP4_AXIS_ROW") == mx.AXIS_ROW
    assert val("MXFP4_AXIS_COL") == mx.AXIS_COL
    assert val("MXFP4_AXIS_2D32") == mx.AXIS_2D32
    assert val("MXFP4_SCALE_OCP_FLOOR") == mx.SCALE_OCP_FLOOR
    assert val("MXFP4_SCALE_CEIL") == mx.SCALE_CEIL
    assert val("MXFP4_OUT_F32") == mx.OUT_F32 and val("MXFP4_OUT_BF16") == mx.OUT_BF16
    assert val("MXFP4_OP_FPROP") == mx.OP_FPROP and val("MXFP4_OP_WGRAD") == mx.OP_WGRAD


def test_status_strings(lib):
    names = ["MXFP4_OK", "MXFP4_ERR_NULL", "MXFP4_ERR_SHAPE", "MXFP4_ERR_MODE",
             "MXFP4_ERR_WORKSPACE", "MXFP4_ERR_HIP", "MXFP4_ERR_ALIGN"]
    for code, name in enumerate(names):
        assert lib.mxfp4_status_string(code).decode() == name
    assert lib.mxfp4_status_string(99).decode() == "MXFP4_ERR_UNKNOWN"
    assert lib.mxfp4_status_string(-1).decode() == "MXFP4_ERR_UNKNOWN"


def test_workspace_bytes(lib):
    r = lambda x: (x + 255) // 256 * 256
    T, N, K = 8192, 6144, 4096
    want = r(T * K // 2) + r(T * K // 32) + r(N * K // 2) + r(N * K // 32)
    assert lib.mxfp4_workspace_bytes(mx.OP_FPROP, T, N, K) == want
    T, N, K = 8192, 4096, 14336
    want = r(T * N // 2) + r(T * N // 32) + r(K * N // 2) + r(K * N // 32)
    assert lib.mxfp4_workspace_bytes(mx.OP_DGRAD, T, N, K) == want
    want = r(N * T // 2) + r(N * T // 32) + r(K * T // 2) + r(K * T // 32)
    assert lib.mxfp4_workspace_bytes(mx.OP_WGRAD, T, N, K) == want
    assert lib.mxfp4_workspace_bytes(mx.OP_FPROP, 10, 10, 33) == 0  # K % 32
    assert lib.mxfp4_workspace_bytes(mx.OP_DGRAD, 10, 33, 10) == 0  # N % 32
    assert lib.mxfp4_workspace_bytes(mx.OP_WGRAD, 33, 10, 10) == 0  # T % 32
    assert lib.mxfp4_workspace_bytes(7, 32, 32, 32) == 0
    assert lib.mxfp4_workspace_bytes(mx.OP_FPROP, 0, 32, 32) == 0


FAKE = ctypes.c_void_p(0x10000)   # aligned non-null address; never dereferenced
FAKE_ODD = ctypes.c_void_p(0x10008)
NULL = ctypes.c_void_p(0)


def q(lib, src=FAKE, rows=64, cols=64, axis=0, h=16, mode=0, nib=FAKE, sc=FAKE):
    return lib.mxfp4_quantize(src, rows, cols, axis, h, mode, nib, sc, NULL)


def test_quantize_validation(lib):
    assert q(lib, axis=3) == 3
    assert q(lib, axis=-1) == 3
    assert q(lib, h=8) == 3
    assert q(lib, mode=2) == 3
    assert q(lib, cols=48) == 2                # row axis: cols % 32
    assert q(lib, axis=1, rows=48) == 2        # col axis: rows % 32
    assert q(lib, axis=2, rows=48) == 2        # 2D: both % 32
    assert q(lib, axis=2, cols=40) == 2
    assert q(lib, rows=-32) == 2
    assert q(lib, src=NULL) == 1
    assert q(lib, nib=NULL) == 1
    assert q(lib, sc=NULL) == 1
    assert q(lib, src=FAKE_ODD) == 6
    assert q(lib, nib=FAKE_ODD) == 6
    # empty inputs are valid and launch nothing, even with NULL buffers
    assert q(lib, rows=0, src=NULL, nib=NULL, sc=NULL) == 0
    assert q(lib, cols=0, src=NULL, nib=NULL, sc=NULL) == 0
    assert q(lib, axis=1, cols=0, src=NULL, nib=NULL, sc=NULL) == 0


def qd(lib, src=FAKE, rows=64, cols=64, h=16, mode=0, rn=FAKE, rs=FAKE, cn=FAKE, cs=FAKE):
    return lib.mxfp4_quantize_dual(src, rows, cols, h, mode, rn, rs, cn, cs, NULL)


def test_quantize_dual_validation(lib):
    assert qd(lib, h=8) == 3
    assert qd(lib, mode=5) == 3
    assert qd(lib, cols=48) == 2               # row orientation: cols % 32
    assert qd(lib, rows=48) == 2               # column orientation: rows % 32
    assert qd(lib, rows=-32) == 2
    for kw in ("src", "rn", "rs", "cn", "cs"):
        assert qd(lib, **{kw: NULL}) == 1, kw
    assert qd(lib, src=FAKE_ODD) == 6
    assert qd(lib, rn=FAKE_ODD) == 6
    assert qd(lib, cn=FAKE_ODD) == 6
    assert qd(lib, rows=0, src=NULL, rn=NULL, rs=NULL, cn=NULL, cs=NULL) == 0
    assert qd(lib, cols=0, src=NULL, rn=NULL, rs=NULL, cn=NULL, cs=NULL) == 0


def test_quantize_of_validation(lib):
    call = lambda **kw: lib.mxfp4_quantize_of(kw.get("src", FAKE), kw.get("rows", 64),
                                              kw.get("cols", 64), kw.get("axis", 0),
                                              kw.get("h", 16), kw.get("mode", 0),
                                              kw.get("nib", FAKE), kw.get("sc", FAKE), NULL)
    assert call(axis=2) == 3
    assert call(h=4) == 3
    assert call(mode=3) == 3
    assert call(cols=40) == 2
    assert call(axis=1, rows=40) == 2
    assert call(nib=NULL) == 1
    assert call(src=FAKE_ODD) == 6
    assert call(rows=0, src=NULL, nib=NULL, sc=NULL) == 0


def test_quantize_rs_and_sr_validation(lib):
    for fn in (lib.mxfp4_quantize_rs, lib.mxfp4_quantize_sr):
        call = lambda **kw: fn(kw.get("src", FAKE), kw.get("rows", 64), kw.get("cols", 64),
                               kw.get("axis", 0), kw.get("h", 16), kw.get("mode", 0),
                               kw.get("aux", FAKE), kw.get("nib", FAKE), kw.get("sc", FAKE), NULL)
        assert call(axis=2) == 3
        assert call(h=8) == 3
        assert call(mode=2) == 3
        assert call(cols=40) == 2
        assert call(axis=1, rows=40) == 2
        assert call(aux=NULL) == 1
        assert call(nib=NULL) == 1
        assert call(src=FAKE_ODD) == 6
        assert call(rows=0, src=NULL, aux=NULL, nib=NULL, sc=NULL) == 0
    # row-axis signs are read 16 bytes at a time; random integers always are
    assert lib.mxfp4_quantize_rs(FAKE, 64, 64, 0, 16, 0, FAKE_ODD, FAKE, FAKE, NULL) == 6
    assert lib.mxfp4_quantize_sr(FAKE, 64, 64, 1, 16, 0, FAKE_ODD, FAKE, FAKE, NULL) == 6


def test_quantize_mbs_validation(lib):
    call = lambda **kw: lib.mxfp4_quantize_mbs(kw.get("src", FAKE), kw.get("rows", 128),
                                               kw.get("cols", 128), kw.get("axis", 0),
                                               kw.get("h", 16), kw.get("mode", 1),
                                               kw.get("nib", FAKE), kw.get("sc", FAKE),
                                               kw.get("mbs", FAKE), NULL)
    assert call(axis=2) == 3
    assert call(cols=96) == 2                  # row axis: cols % 128
    assert call(axis=1, rows=96) == 2          # col axis: rows % 128
    assert call(mbs=NULL) == 1
    assert call(nib=NULL) == 1
    assert call(src=FAKE_ODD) == 6
    assert call(rows=0, src=NULL, nib=NULL, sc=NULL, mbs=NULL) == 0


def es(lib, src=FAKE, rows=64, cols=64, axis=0, h=16, mode=0, ws=FAKE, wsb=None, out=FAKE):
    wsb = mx.ERROR_STATS_WS_BYTES if wsb is None else wsb
    return lib.mxfp4_error_stats(src, rows, cols, axis, h, mode, ws, wsb, out, NULL)


def test_error_stats_validation(lib):
    assert "MXFP4_ERROR_STATS_WS_BYTES (1024 * MXFP4_ERROR_STATS_COUNT * 8)" in header_text()
    assert "MXFP4_ERROR_STATS_COUNT 10" in header_text() and mx.ERROR_STATS_COUNT == 10
    assert es(lib, axis=2) == 3                # 2D blocks have no per-block decomposition here
    assert es(lib, h=8) == 3
    assert es(lib, mode=2) == 3
    assert es(lib, cols=48) == 2
    assert es(lib, axis=1, rows=48) == 2
    assert es(lib, src=NULL) == 1
    assert es(lib, ws=NULL) == 1
    assert es(lib, out=NULL) == 1
    assert es(lib, wsb=mx.ERROR_STATS_WS_BYTES - 1) == 4
    assert es(lib, src=FAKE_ODD) == 6
    assert es(lib, out=ctypes.c_void_p(0x10004)) == 6


def test_error_stats_noalloc_validation(lib):
    call = lambda **kw: lib.mxfp4_error_stats_noalloc(
        kw.get("src", FAKE), kw.get("rows", 64), kw.get("cols", 64), kw.get("axis", 0),
        kw.get("h", 16), kw.get("mode", 0), kw.get("out", FAKE), NULL)
    assert call(axis=2) == 3
    assert call(h=8) == 3
    assert call(mode=2) == 3
    assert call(cols=48) == 2
    assert call(axis=1, rows=48) == 2
    assert call(src=NULL) == 1
    assert call(out=NULL) == 1
    assert call(src=FAKE_ODD) == 6
    assert call(out=ctypes.c_void_p(0x10004)) == 6


def qp(lib, a=(FAKE, 64, 64, 0, FAKE, FAKE), b=(FAKE, 64, 64, 1, FAKE, FAKE), h=16, mode=0):
    return lib.mxfp4_quantize_pair(*a, *b, h, mode, NULL)


def test_quantize_pair_validation(lib):
    """Each operand is validated as by mxfp4_quantize, operand A's errors
    first; 2D blocks are not a pair axis."""
    A, B = (FAKE, 64, 64, 0, FAKE, FAKE), (FAKE, 64, 64, 1, FAKE, FAKE)
    with_ = lambda t, i, v: tuple(v if k == i else x for k, x in enumerate(t))
    assert qp(lib, a=with_(A, 3, 2)) == 3
    assert qp(lib, b=with_(B, 3, 2)) == 3
    assert qp(lib, h=8) == 3
    assert qp(lib, mode=2) == 3
    assert qp(lib, a=with_(A, 2, 48)) == 2            # A row axis: cols % 32
    assert qp(lib, b=with_(B, 1, 48)) == 2            # B column axis: rows % 32
    assert qp(lib, a=with_(A, 0, NULL)) == 1
    assert qp(lib, b=with_(B, 4, NULL)) == 1
    assert qp(lib, b=with_(B, 0, FAKE_ODD)) == 6
    # A's error is reported when both operands are invalid
    assert qp(lib, a=with_(A, 2, 48), b=with_(B, 0, NULL)) == 2
    assert qp(lib, a=with_(A, 0, NULL), b=with_(B, 1, 48)) == 1
    # two empty operands are valid and launch nothing, even with NULL buffers
    assert qp(lib, a=(NULL, 0, 64, 0, NULL, NULL), b=(NULL, 64, 0, 1, NULL, NULL)) == 0


def test_gemm_mbs_validation(lib):
    call = lambda **kw: lib.mxfp4_gemm_mbs(
        kw.get("A", FAKE), kw.get("As", FAKE), kw.get("Am", FAKE), kw.get("B", FAKE),
        kw.get("Bs", FAKE), kw.get("Bm", FAKE), kw.get("M", 64), kw.get("N", 64),
        kw.get("K", 128), kw.get("C", FAKE), kw.get("out", 0), NULL)
    assert call(out=2) == 3
    assert call(M=0) == 2
    assert call(K=96) == 2                     # K % 128 (one 8-bit mantissa per 128 k)
    assert call(K=48) == 2
    assert call(A=NULL) == 1
    assert call(Am=NULL) == 1
    assert call(Bm=NULL) == 1
    assert call(C=ctypes.c_void_p(0x10002)) == 6


def g(lib, M=64, N=64, K=64, out=0, A=FAKE, As=FAKE, B=FAKE, Bs=FAKE, C=FAKE):
    return lib.mxfp4_gemm(A, As, B, Bs, M, N, K, C, out, NULL)


def test_gemm_validation(lib):
    assert g(lib, out=2) == 3
    assert g(lib, M=0) == 2
    assert g(lib, N=0) == 2
    assert g(lib, K=0) == 2
    assert g(lib, K=48) == 2
    assert g(lib, K=16) == 2
    assert g(lib, A=NULL) == 1
    assert g(lib, Bs=NULL) == 1
    assert g(lib, C=NULL) == 1
    assert g(lib, A=FAKE_ODD) == 6
    assert g(lib, C=ctypes.c_void_p(0x10002)) == 6             # fp32 C needs 4 B alignment
    assert g(lib, C=ctypes.c_void_p(0x10001), out=1) == 6      # bf16 C needs 2 B alignment


@pytest.mark.parametrize("name", ["mxfp4_fprop", "mxfp4_dgrad", "mxfp4_wgrad"])
def test_fused_validation(lib, name):
    fn = getattr(lib, name)
    T, N, K = 64, 64, 64
    op = {"mxfp4_fprop": 0, "mxfp4_dgrad": 1, "mxfp4_wgrad": 2}[name]
    need = lib.mxfp4_workspace_bytes(op, T, N, K)
    assert need > 0
    call = lambda **kw: fn(kw.get("P", FAKE), kw.get("Q", FAKE), kw.get("T", T), kw.get("N", N),
                           kw.get("K", K), kw.get("h", 16), kw.get("mode", 0),
                           kw.get("ws", FAKE), kw.get("wsb", need), kw.get("out", FAKE),
                           kw.get("od", 0), NULL)
    assert call(h=4) == 3
    assert call(mode=5) == 3
    assert call(od=9) == 3
    assert call(T=0) == 2
    bad_axis = {"mxfp4_fprop": "K", "mxfp4_dgrad": "N", "mxfp4_wgrad": "T"}[name]
    assert call(**{bad_axis: 40}) == 2
    assert call(P=NULL) == 1
    assert call(ws=NULL) == 1
    assert call(out=NULL) == 1
    assert call(wsb=need - 1) == 4
    assert call(P=FAKE_ODD) == 6
    assert call(ws=ctypes.c_void_p(0x10010)) == 6   # workspace must be 256 B aligned


def test_linear_wrapper_validates_and_never_computes_on_the_cpu():
    """MXFP4Linear checks its sizes, and a CPU tensor is rejected by the
    binding before any call (there is no CPU path)."""
    import torch
    from mxfp4_quantized_gemm_amd.linear import MXFP4Linear
    with pytest.raises(ValueError):
        MXFP4Linear(48, 64)
    layer = MXFP4Linear(64, 32)
    with pytest.raises(ValueError):
        layer(torch.zeros(16, 64, dtype=torch.bfloat16))      # 16 rows: not a multiple of 32
    with pytest.raises(ValueError, match="GPU memory"):
        layer(torch.zeros(32, 64, dtype=torch.bfloat16))


def test_binding_fails_loudly_without_library(tmp_path):
    saved = mx._LIB
    try:
        mx._LIB = None
        with pytest.raises(RuntimeError, match="missing"):
            mx.load_library(str(tmp_path / "missing.so"))
    finally:
        mx._LIB = saved


def test_product_path_does_not_import_oracle():
    """The package and its sources never reference the oracle."""
    pkg = os.path.dirname(mx.__file__)
    for dirpath, _, files in os.walk(pkg):
        for fn in files:
            if fn.endswith((".py", ".hip", ".cpp", ".h")):
                with open(os.path.join(dirpath, fn)) as f:
                    text = f.read()
                assert not re.search(r"\boracle\b", text), fn


def test_bench_refuses_more_than_one_gpu():
    """The bench measures one GPU: --gpus 2 exits (status 2) with a message,
    before touching a device."""
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
