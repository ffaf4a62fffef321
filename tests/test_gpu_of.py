"""GPU parity of the outlier-fallback operand (mxfp4_quantize_of) with the
oracle's quantize_of: bit-exact nibbles and E8M0 bytes, and the MXFP4 GEMM
of depth 2K on it (against the other operand repeated along K) within the
GEMM tolerance |C - C_ref| <= 1e-5 sum|a||b| of the oracle's fp64 product.
Calls go through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16
from tests.test_gpu_quant import edge_matrix, heavy

pytestmark = pytest.mark.gpu


def run_of(bits, axis, h, mode):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    nib, sc = mx.quantize_of(to_dev_bf16(bits), axis, h, mode)
    torch.cuda.synchronize()
    return nib.cpu().numpy(), sc.cpu().numpy()


def assert_of_same(bits, axis, h, mode, what):
    gn, gs = run_of(bits, axis, h, mode)
    on, os_ = O.quantize_of(bits, axis, h, mode)
    assert gn.shape == on.shape and gs.shape == os_.shape, what
    bs, bn = np.argwhere(gs != os_), np.argwhere(gn != on)
    assert bs.size == 0, f"{what}: {len(bs)} scale bytes differ, first {bs[:4].tolist()}"
    assert bn.size == 0, f"{what}: {len(bn)} nibble bytes differ, first {bn[:4].tolist()}"


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_small_shapes_bit_exact(axis, h, mode):
    # column axis: the staged kernel for rows % 128 == 0 and cols % 4 == 0
    # ((256, 512), (384, 100), (128, 260)), the per-column kernel otherwise
    shapes = [(32, 32), (64, 96), (96, 320), (256, 512), (33 * 32, 64)]
    if axis == 1:
        shapes += [(384, 100), (128, 260)]
    for i, (r, c) in enumerate(shapes):
        assert_of_same(heavy(r, c, 9100 + 7 * i + axis), axis, h, mode,
                       f"axis={axis} h={h} mode={mode} shape={(r, c)}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("mode", [0, 1])
def test_edge_values_bit_exact(axis, mode):
    mats = [edge_matrix(128, 256, seed=17)]
    if axis == 1:  # special blocks down the columns as well
        mats.append(np.ascontiguousarray(edge_matrix(256, 128, seed=18).T))
    for k, bits in enumerate(mats):
        for h in (0, 16, 32):
            assert_of_same(bits, axis, h, mode, f"edge {k} axis={axis} h={h}")


@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_workload_full_size(axis):
    A = synthetic.make("quant")["A"]
    assert_of_same(A, axis, 16, 1, f"full axis={axis} ceil")


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_on_the_of_operand(mode):
    """Fprop with the weight in OF form: Y = [X | X] . [W1 | W2]^T over 2K."""
    import torch
    import mxfp4_quantized_gemm_amd as mx
    T, N, K = 192, 160, 512
    xb = heavy(T, K, 51)
    wb = heavy(N, K, 52)
    x, w = to_dev_bf16(xb), to_dev_bf16(wb)
    an, asc = mx.quantize(x, mx.AXIS_ROW, 16, mode)
    bn, bsc = mx.quantize_of(w, mx.AXIS_ROW, 16, mode)
    a2n, a2s = torch.cat([an, an], 1).contiguous(), torch.cat([asc, asc], 1).contiguous()
    C = mx.gemm(a2n, a2s, bn, bsc, mx.OUT_F32)
    torch.cuda.synchronize()
    oa = O.quantize(xb, O.AXIS_ROW, 16, mode)
    ob = O.quantize_of(wb, O.AXIS_ROW, 16, mode)
    da = O.dequantize(*oa)
    C_ref, S = O.gemm_ref(np.concatenate([da, da], 1), O.dequantize(*ob))
    c = C.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(c - C_ref) <= O.gemm_tolerance(S, C_ref, False))
    # the OF product is closer to the unquantized rotated product than the plain one
    exact = O.rotated_unquantized_product("fprop", xb, wb, 16)
    plain, _ = O.gemm_ref(da, O.dequantize(*O.quantize(wb, O.AXIS_ROW, 16, mode)))
    assert np.sum((C_ref - exact) ** 2) < np.sum((plain - exact) ** 2)
