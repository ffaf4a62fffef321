"""MXFP4Linear (the autograd wrapper over mxfp4_fprop / dgrad / wgrad):
forward and both gradients equal the fused entry points' outputs bit for
bit, and the forward output meets the GEMM bar against the oracle."""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16
from tests.test_gpu_quant import heavy

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("modes", [(0, 0, 0), (0, 0, 1), (1, 1, 1)])
@pytest.mark.parametrize("h", [16, 32, 0])
def test_linear_matches_fused_entry_points(h, modes):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    from mxfp4_quantized_gemm_amd.linear import MXFP4Linear
    T, N, K = 256, 384, 512
    layer = MXFP4Linear(K, N, hadamard=h, modes=modes, device="cuda")
    wb = heavy(N, K, 61 + h)
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(wb))
    xb, gb = heavy(T, K, 62 + h), heavy(T, N, 63 + h)
    x = to_dev_bf16(xb).requires_grad_(True)
    dy = to_dev_bf16(gb)
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    W = layer.weight.detach()

    def direct(fn, op, P, Q, shape, mode):
        ws = torch.empty(mx.mxfp4_workspace_bytes(op, T, N, K), dtype=torch.uint8, device="cuda")
        out = torch.empty(shape, dtype=torch.bfloat16, device="cuda")
        fn(P, Q, T, N, K, h, mode, ws, out, mx.OUT_BF16)
        return out
    want_y = direct(mx.mxfp4_fprop, mx.OP_FPROP, x.detach(), W, (T, N), modes[0])
    want_dx = direct(mx.mxfp4_dgrad, mx.OP_DGRAD, dy, W, (T, K), modes[1])
    want_dw = direct(mx.mxfp4_wgrad, mx.OP_WGRAD, dy, x.detach(), (N, K), modes[2])
    torch.cuda.synchronize()
    assert np.array_equal(_bits(y.detach()), _bits(want_y))
    assert np.array_equal(_bits(x.grad), _bits(want_dx))
    assert np.array_equal(_bits(layer.weight.grad), _bits(want_dw))
    # the forward output against the oracle's product of its own operands
    qa, qb = O.product_operands("fprop", xb, wb, h, modes[0])
    Cr, S = O.gemm_ref(O.dequantize(*qa), O.dequantize(*qb))
    got = y.detach().float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - Cr) <= O.gemm_tolerance(S, Cr, True))


def test_linear_on_the_tiny_fprop_workload_3d_input():
    """[2, 64, 256] input (flattened to 128 rows) on the tiny Fprop workload."""
    import torch
    from mxfp4_quantized_gemm_amd.linear import MXFP4Linear
    w = synthetic.make("tiny")
    layer = MXFP4Linear(256, 256, device="cuda")
    with torch.no_grad():
        layer.weight.copy_(to_dev_bf16(w["W"]))
    x = to_dev_bf16(w["X"]).reshape(2, 64, 256)
    y = layer(x)
    assert y.shape == (2, 64, 256) and y.dtype == torch.bfloat16
    qa, qb = O.product_operands("fprop", w["X"], w["W"], 16, 0)
    Cr, S = O.gemm_ref(O.dequantize(*qa), O.dequantize(*qb))
    got = y.detach().reshape(128, 256).float().cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - Cr) <= O.gemm_tolerance(S, Cr, True))
