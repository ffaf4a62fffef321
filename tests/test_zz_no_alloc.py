"""mxfp4_error_stats_noalloc (partial sums in the library's static device
array, no workspace) against mxfp4_error_stats (caller workspace) through
the C ABI: two calls in a row, the second on a smaller input, each equal to
the workspace entry point's sums bit for bit (same kernels, fixed-order
reduction) and within the oracle's bar."""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import to_dev_bf16
from tests.test_gpu_quant import heavy
from tests.test_gpu_stats import assert_stats_close

pytestmark = pytest.mark.gpu


def _both(bits, axis, h, mode):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    rows, cols = bits.shape
    x = to_dev_bf16(bits)
    ws = torch.empty(mx.ERROR_STATS_WS_BYTES, dtype=torch.uint8, device="cuda")
    want = torch.full((mx.ERROR_STATS_COUNT,), float("nan"), dtype=torch.float64, device="cuda")
    got = torch.full((mx.ERROR_STATS_COUNT,), float("nan"), dtype=torch.float64, device="cuda")
    mx.mxfp4_error_stats(x, rows, cols, axis, h, mode, ws, want)
    mx.mxfp4_error_stats_noalloc(x, rows, cols, axis, h, mode, got)
    torch.cuda.synchronize()
    return got.cpu().numpy(), want.cpu().numpy()


@pytest.mark.parametrize("axis", [0, 1])
def test_noalloc_matches_workspace_entry_point_twice(axis):
    import mxfp4_quantized_gemm_amd as mx
    # first call: 1024 work-groups of partials (the array's maximum); the
    # second, smaller call reads only the partials it writes
    for shape, seed, h, mode in (((2048, 4096), 5, 16, 0), ((96, 320), 6, 32, 1)):
        bits = heavy(*shape, seed + axis)
        got, want = _both(bits, axis, h, mode)
        assert np.array_equal(got.view(np.uint64), want.view(np.uint64)), (shape, got, want)
        d = dict(zip(mx.ERROR_STATS_FIELDS, got.tolist()))
        assert_stats_close(d, O.error_stats(bits, axis, h, mode), f"noalloc {shape} axis={axis}")
