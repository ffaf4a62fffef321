"""GPU parity of the macro-block-scaled operand (mxfp4_quantize_mbs) with the
oracle's quantize_mbs: bit-exact nibbles, E8M0 bytes and mantissa bytes
(the mantissa is an fp64 decision on both sides, from the same fp32 amax).
Calls go through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16
from tests.test_gpu_quant import edge_matrix, heavy

pytestmark = pytest.mark.gpu

SHAPES = {0: [(1, 128), (3, 256), (64, 640), (257, 128)],
          1: [(128, 1), (256, 7), (384, 100), (128, 300)]}


def assert_mbs_same(bits, axis, h, mode, what):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    got = [t.cpu().numpy() for t in mx.quantize_mbs(to_dev_bf16(bits), axis, h, mode)]
    torch.cuda.synchronize()
    want = O.quantize_mbs(bits, axis, h, mode)
    for g, w, name in zip(got, want, ("nibbles", "scales", "mantissas")):
        assert g.shape == w.shape, f"{what} {name}"
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{what}: {len(bad)} {name} differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_small_shapes_bit_exact(axis, h, mode):
    for i, (r, c) in enumerate(SHAPES[axis]):
        assert_mbs_same(heavy(r, c, 9500 + 5 * i + axis), axis, h, mode,
                        f"axis={axis} h={h} mode={mode} shape={(r, c)}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("mode", [0, 1])
def test_edge_values_bit_exact(axis, mode):
    mats = [edge_matrix(128, 256, seed=23)]
    if axis == 1:  # special blocks down the columns as well
        mats.append(np.ascontiguousarray(edge_matrix(256, 128, seed=24).T))
    for k, bits in enumerate(mats):
        for h in (0, 16, 32):
            assert_mbs_same(bits, axis, h, mode, f"edge {k} axis={axis} h={h}")


@pytest.mark.parametrize("axis", [0, 1])
def test_quantizer_workload_full_size(axis):
    assert_mbs_same(synthetic.make("quant")["A"], axis, 16, 1, f"full axis={axis}")
