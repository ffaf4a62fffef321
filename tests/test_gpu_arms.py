"""GPU parity of the comparison arms (mxfp4_quantize_rs: random-sign
Hadamard; mxfp4_quantize_sr: stochastic rounding) with the oracle's
quantize_rs / quantize_sr: every nibble and E8M0 byte equal. The random
signs and random integers come from the seeded generators in ``synthetic``
and are passed to both sides. Calls go through the C ABI."""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16, to_dev_u8
from tests.test_gpu_quant import edge_matrix, heavy

pytestmark = pytest.mark.gpu

# row: one thread per block; col: the staged kernel (rows % 128 == 0,
# cols % 4 == 0) and the scalar kernel otherwise
SHAPES = {0: [(1, 32), (3, 96), (257, 160), (64, 4128)],
          1: [(32, 1), (64, 7), (128, 100), (256, 520), (96, 64), (384, 4)]}


def to_dev_u32(arr):
    import torch
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.uint32).view(np.int32)).to("cuda")


def gpu_rs(bits, axis, h, mode, signs):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    nib, sc = mx.quantize_rs(to_dev_bf16(bits), to_dev_u8(signs), axis, h, mode)
    torch.cuda.synchronize()
    return nib.cpu().numpy(), sc.cpu().numpy()


def gpu_sr(bits, axis, h, mode, rnd):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    nib, sc = mx.quantize_sr(to_dev_bf16(bits), to_dev_u32(rnd), axis, h, mode)
    torch.cuda.synchronize()
    return nib.cpu().numpy(), sc.cpu().numpy()


def assert_same(got, want, what):
    for g, w, name in zip(got, want, ("nibbles", "scales")):
        assert g.shape == w.shape, f"{what} {name}"
        bad = np.argwhere(g != w)
        assert bad.size == 0, f"{what}: {len(bad)} {name} bytes differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_random_signs_small_shapes(axis, h, mode):
    for i, (r, c) in enumerate(SHAPES[axis]):
        bits = heavy(r, c, 3100 + 7 * i + axis)
        signs = synthetic.random_signs(c if axis == 0 else r, 3200 + i)
        assert_same(gpu_rs(bits, axis, h, mode, signs), O.quantize_rs(bits, axis, h, mode, signs),
                    f"rs axis={axis} h={h} mode={mode} shape={(r, c)}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_stochastic_rounding_small_shapes(axis, h, mode):
    for i, (r, c) in enumerate(SHAPES[axis]):
        bits = heavy(r, c, 3300 + 7 * i + axis)
        rnd = synthetic.random_u32((r, c), 3400 + i)
        assert_same(gpu_sr(bits, axis, h, mode, rnd), O.quantize_sr(bits, axis, h, mode, rnd),
                    f"sr axis={axis} h={h} mode={mode} shape={(r, c)}")


@pytest.mark.parametrize("axis", [0, 1])
@pytest.mark.parametrize("mode", [0, 1])
def test_arms_edge_values(axis, mode):
    mats = [edge_matrix(128, 256, seed=31)]
    if axis == 1:
        mats.append(np.ascontiguousarray(edge_matrix(256, 128, seed=32).T))
    for k, bits in enumerate(mats):
        r, c = bits.shape
        signs = synthetic.random_signs(c if axis == 0 else r, 33 + k)
        for h in (0, 16, 32):
            assert_same(gpu_rs(bits, axis, h, mode, signs), O.quantize_rs(bits, axis, h, mode, signs),
                        f"rs edge {k} axis={axis} h={h}")
        # the extreme integers 0 and 2^32 - 1 and the exact thresholds
        rnd = synthetic.random_u32(bits.shape, 34 + k)
        rnd[::3] = 0
        rnd[1::3] = 0xFFFFFFFF
        for h in (0, 16, 32):
            assert_same(gpu_sr(bits, axis, h, mode, rnd), O.quantize_sr(bits, axis, h, mode, rnd),
                        f"sr edge {k} axis={axis} h={h}")


def test_sr_exact_thresholds_on_gpu():
    """0.375 in a block of amax 4 rounds up for u < 0.75 * 2^32, 5.0 and -3.5
    for u < 2^31 (both scale rules give 2^0 here)."""
    row = np.zeros((1, 32))
    row[0, :4] = (4.0, 0.375, 5.0, -3.5)
    bits = synthetic.f64_to_bf16_bits(row)
    for r1 in (3221225471, 3221225472):
        for r2 in (2 ** 31 - 1, 2 ** 31):
            rnd = np.full((1, 32), 0xFFFFFFFF, np.uint32)
            rnd[0, 1], rnd[0, 2], rnd[0, 3] = r1, r2, r2
            for mode in (0, 1):
                assert_same(gpu_sr(bits, 0, 0, mode, rnd), O.quantize_sr(bits, 0, 0, mode, rnd),
                            f"thresholds {r1} {r2} mode={mode}")


@pytest.fixture(scope="module")
def quant_workload():
    return synthetic.make("quant")["A"]


@pytest.mark.parametrize("axis", [0, 1])
def test_arms_workload_full_size(quant_workload, axis):
    """8192 x 4096 Student-t workload, H16: every byte of both arms."""
    a = quant_workload
    n = a.shape[1] if axis == 0 else a.shape[0]
    signs = synthetic.random_signs(n, 41)
    assert_same(gpu_rs(a, axis, 16, 1, signs), O.quantize_rs(a, axis, 16, 1, signs),
                f"rs full axis={axis}")
    rnd = synthetic.random_u32(a.shape, 42)
    assert_same(gpu_sr(a, axis, 16, 0, rnd), O.quantize_sr(a, axis, 16, 0, rnd),
                f"sr full axis={axis}")


@pytest.mark.parametrize("axis", [0, 1])
def test_sr_scaled_values_below_fp32_range_on_gpu(axis):
    """Blocks whose large first element puts E at 8..27 while the other
    rotation group holds bf16 subnormals: the scaled values fall below
    2^-149, where an fp32 multiply rounds to 0 but the exact p is positive,
    so u = 0 must round them up to 0.5. Random u elsewhere, both rules,
    H0/H16/H32 (H32 mixes the groups, which the oracle follows as well)."""
    rng = np.random.default_rng(77)
    R = 64
    bits = np.zeros((R, 64), np.uint16)
    for r in range(R):
        bits[r, 0] = synthetic.f64_to_bf16_bits(np.array([2.0 ** (10 + r % 20)]))[0]
        bits[r, 16:32] = rng.integers(1, 0x80, 16) | (rng.integers(0, 2, 16) << 15)
        bits[r, 32] = bits[r, 0]
        bits[r, 48:64] = rng.integers(1, 0x80, 16)
    if axis == 1:
        bits = np.ascontiguousarray(bits.T)
    for mode in (0, 1):
        for h in (0, 16, 32):
            rnd = synthetic.random_u32(bits.shape, 78)
            rnd[rng.random(bits.shape) < 0.5] = 0
            assert_same(gpu_sr(bits, axis, h, mode, rnd), O.quantize_sr(bits, axis, h, mode, rnd),
                        f"sr underflow axis={axis} h={h} mode={mode}")
            want = O.quantize_sr(bits, axis, h, mode, np.zeros(bits.shape, np.uint32))
            assert_same(gpu_sr(bits, axis, h, mode, np.zeros(bits.shape, np.uint32)), want,
                        f"sr underflow u=0 axis={axis} h={h} mode={mode}")
