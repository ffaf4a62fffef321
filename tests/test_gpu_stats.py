"""GPU parity of mxfp4_error_stats (the three-way MXFP4 error decomposition
summed over a tensor) against the CPU oracle's error_stats.

The per-element terms are the same fp64 operations on both sides (the codes
come from the bit-exact quantizer path, Q* and the deadzone test are fp64
divisions and compares in both), so only the order of the fp64 sums
differs: sums agree to 1e-9 relative (cross terms to 1e-9 of the matching
norm product), counts exactly. Calls go through the C ABI.
"""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16
from tests.test_gpu_quant import edge_matrix, heavy

pytestmark = pytest.mark.gpu

SUMS = ("sum_e_scale2", "sum_e_dz2", "sum_e_grid2", "sum_e2", "sum_x2")
COUNTS = ("n_deadzone", "n_elements", "n_nonfinite_blocks")


def gpu_stats(bits, axis, h, mode):
    import mxfp4_quantized_gemm_amd as mx
    return mx.error_stats(to_dev_bf16(bits), axis, h, mode)


def assert_stats_close(got, want, what):
    for k in COUNTS:
        assert got[k] == want[k], f"{what}: {k} {got[k]} != {want[k]}"
    for k in SUMS:
        assert got[k] == pytest.approx(want[k], rel=1e-9, abs=0), f"{what}: {k}"
    scale_grid = np.sqrt(want["sum_e_scale2"] * want["sum_e_grid2"])
    scale_dz = np.sqrt(want["sum_e_scale2"] * want["sum_e_dz2"])
    assert abs(got["dot_scale_grid"] - want["dot_scale_grid"]) <= 1e-9 * scale_grid, what
    assert abs(got["dot_scale_dz"] - want["dot_scale_dz"]) <= 1e-9 * scale_dz, what


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_small_shapes(axis, h, mode):
    for i, (r, c) in enumerate([(32, 32), (64, 96), (96, 320), (256, 512)]):
        bits = heavy(r, c, 7000 + 13 * i + axis)
        assert_stats_close(gpu_stats(bits, axis, h, mode), O.error_stats(bits, axis, h, mode),
                           f"axis={axis} h={h} mode={mode} shape={(r, c)}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("mode", [0, 1])
def test_edge_values_and_nonfinite_blocks(axis, mode):
    bits = edge_matrix(128, 256, seed=3)
    want = O.error_stats(bits, axis, 16, mode)
    assert want["n_nonfinite_blocks"] > 0
    assert_stats_close(gpu_stats(bits, axis, 16, mode), want, f"edge axis={axis} mode={mode}")


def test_ceil_mode_orthogonality_and_identity_on_gpu():
    """[P3] Property 1 on the GPU's own sums: <e_DZ, e_scale> is exactly 0
    under the ceiling scale, and the MSE identity holds to fp64 rounding."""
    bits = heavy(512, 1024, 11)
    st = gpu_stats(bits, 0, 16, 1)
    assert st["dot_scale_dz"] == 0.0
    rhs = st["sum_e_scale2"] + st["sum_e_dz2"] + st["sum_e_grid2"] + 2 * st["dot_scale_grid"]
    assert st["sum_e2"] == pytest.approx(rhs, rel=1e-10)
    assert st["cos_scale_grid"] < 0


def test_deterministic_and_empty():
    import torch
    import mxfp4_quantized_gemm_amd as mx
    bits = heavy(256, 512, 5)
    a = gpu_stats(bits, 1, 16, 0)
    b = gpu_stats(bits, 1, 16, 0)
    assert all(a[k] == b[k] for k in O.STAT_FIELDS)
    x = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(mx.ERROR_STATS_WS_BYTES, dtype=torch.uint8, device="cuda")
    out = torch.full((10,), 7.0, dtype=torch.float64, device="cuda")
    mx.mxfp4_error_stats(x, 0, 64, 0, 16, 0, ws, out)
    assert out.cpu().tolist() == [0.0] * 10


@pytest.mark.parametrize("axis,mode", [(0, 0), (1, 1)])
def test_quantizer_workload_full_size(axis, mode):
    """8192 x 4096 Student-t x log-normal tensor, H16."""
    A = synthetic.make("quant")["A"]
    assert_stats_close(gpu_stats(A, axis, 16, mode), O.error_stats_chunked(A, axis, 16, mode),
                       f"full axis={axis} mode={mode}")
