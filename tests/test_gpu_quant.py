"""GPU parity of the rotate+quantize kernels against the CPU oracle.

The bar is bit-exact equality of every nibble byte and every E8M0 byte, for
every axis (1x32 row, 32x1 column-transposed, 32x32 2D) x rotation (none,
H16, H32) x scale rule (OCP floor, ceil), at small ragged shapes, at edge
values, and at the full 8192 x 4096 quantizer workload. All calls go through
the C ABI (mxfp4_quantize) via the ctypes binding.
"""
import numpy as np
import pytest

import oracle as O
import synthetic
from tests.gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu

AXES = {"row": 0, "col": 1, "2d": 2}


def run_gpu(bits, axis, h, mode):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    x = to_dev_bf16(bits)
    nib, sc = mx.quantize(x, axis, h, mode)
    torch.cuda.synchronize()
    return nib.cpu().numpy(), sc.cpu().numpy()


def assert_same(bits, axis, h, mode, what=""):
    gn, gs = run_gpu(bits, axis, h, mode)
    on, os_ = O.quantize_chunked(bits, axis, h, mode)
    assert gs.shape == os_.shape and gn.shape == on.shape, what
    bad_s = np.argwhere(gs != os_)
    bad_n = np.argwhere(gn != on)
    assert bad_s.size == 0, f"{what}: {len(bad_s)} scale bytes differ, first {bad_s[:4].tolist()}"
    assert bad_n.size == 0, f"{what}: {len(bad_n)} nibble bytes differ, first {bad_n[:4].tolist()}"


def heavy(rows, cols, seed):
    rng = np.random.default_rng(seed)
    a = rng.standard_t(3, size=(rows, cols)) * rng.lognormal(0, 1, size=(1, cols))
    return synthetic.f64_to_bf16_bits(a)


SHAPES = {
    0: [(1, 32), (3, 96), (257, 160), (64, 4128), (256, 256), (96, 8192)],
    1: [(32, 1), (64, 7), (32, 100), (96, 520), (128, 1544), (160, 8), (256, 300), (384, 4),
        (128, 260)],
    2: [(32, 32), (64, 96), (96, 320), (32, 4096), (64, 512), (96, 256)],
}


@pytest.mark.parametrize("axis", [0, 1, 2])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_small_shapes_bit_exact(axis, h, mode):
    for i, (r, c) in enumerate(SHAPES[axis]):
        bits = heavy(r, c, 1000 + 7 * i + axis)
        assert_same(bits, axis, h, mode, f"axis={axis} h={h} mode={mode} shape={(r, c)}")


def edge_matrix(rows=64, cols=128, seed=5):
    """Blocks of special values: zeros, negative zeros, bf16 subnormals,
    exact E2M1 ties at several scales, huge values whose rotation overflows,
    NaN, Inf, and a tiny-amax block that hits the E clamp."""
    rng = np.random.default_rng(seed)
    a = rng.normal(size=(rows, cols)).astype(np.float32)
    bits = synthetic.f64_to_bf16_bits(a)
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], np.float32)
    for r in range(rows):
        kind = r % 8
        seg = slice(32 * (r % (cols // 32)), 32 * (r % (cols // 32)) + 32)
        if kind == 0:
            bits[r, seg] = 0
        elif kind == 1:
            bits[r, seg] = 0x8000
            bits[r, seg.start + 3] = 0x0001            # smallest subnormal
        elif kind == 2:
            bits[r, seg] = rng.integers(1, 0x80, 32)  # positive subnormals only
        elif kind == 3:
            vals = np.tile(np.concatenate([ties, -ties]), 2) * np.float32(2.0 ** (r % 5 - 2))
            bits[r, seg] = synthetic.f64_to_bf16_bits(vals)
        elif kind == 4:
            bits[r, seg] = 0x7F70                     # ~3.2e38: sums overflow to inf
        elif kind == 5:
            bits[r, seg.start + 7] = 0x7FC0           # NaN
        elif kind == 6:
            bits[r, seg.start + 9] = 0xFF80           # -Inf
        else:
            bits[r, seg] = rng.integers(0x0080, 0x0180, 32)  # around 2^-126
    return bits


@pytest.mark.parametrize("axis", [0, 1, 2])
@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_edge_values_bit_exact(axis, h, mode):
    bits = edge_matrix()
    assert_same(bits, axis, h, mode, f"edge axis={axis} h={h} mode={mode}")


@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_edge_values_2d_lane_contiguous(h, mode):
    """Edge blocks in 32x32 tiles whose column groups are whole 256-column
    groups (the lane-contiguous 2D kernel)."""
    bits = edge_matrix(96, 512, seed=9)
    assert_same(bits, 2, h, mode, f"edge 2d 96x512 h={h} mode={mode}")


def test_col_equals_row_of_transpose():
    """The transposed column-wise output equals the row-wise output of the
    host-transposed matrix (catches LDS/register transpose mistakes)."""
    bits = heavy(256, 1024, 77)
    for h in (0, 16, 32):
        cn, cs = run_gpu(bits, 1, h, 1)
        rn, rs = run_gpu(np.ascontiguousarray(bits.T), 0, h, 1)
        assert np.array_equal(cn, rn) and np.array_equal(cs, rs)


def test_deterministic():
    bits = heavy(512, 1024, 3)
    for axis in (0, 1, 2):
        a = run_gpu(bits, axis, 16, 0)
        b = run_gpu(bits, axis, 16, 0)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


@pytest.fixture(scope="module")
def quant_workload():
    return synthetic.make("quant")["A"]


@pytest.mark.parametrize("axis", ["row", "col", "2d"])
@pytest.mark.parametrize("mode", [0, 1])
def test_quantizer_workload_full_size(quant_workload, axis, mode):
    """8192 x 4096 Student-t x log-normal workload, H16: every byte."""
    assert_same(quant_workload, AXES[axis], 16, mode, f"full axis={axis} mode={mode}")


@pytest.mark.parametrize("h", [0, 32])
def test_quantizer_workload_full_size_other_rotations(quant_workload, h):
    assert_same(quant_workload, 0, h, 0, f"full row h={h}")


@pytest.mark.parametrize("mode", [0, 1])
def test_row_quantizer_above_lane_contiguous_threshold(quant_workload, mode):
    """More than 2^20 row blocks (8448 x 4096: the workload plus its first
    256 rows again), every byte: the lane-contiguous kernel (quad-transposed
    loads), which the standalone quantizer runs whenever the block count is
    a multiple of 256 and the two-operand launch above 2^20 blocks."""
    big = np.concatenate([quant_workload, quant_workload[:256]], axis=0)
    assert_same(big, AXES["row"], 16, mode, f"row 8448x4096 mode={mode}")


# ------------------------------------------------------- dual orientation
def run_gpu_dual(bits, h, mode):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    x = to_dev_bf16(bits)
    (rn, rs), (cn, cs) = mx.quantize_dual(x, h, mode)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (rn, rs, cn, cs)]


def assert_dual_same(bits, h, mode, what=""):
    rn, rs, cn, cs = run_gpu_dual(bits, h, mode)
    orn, ors = O.quantize_chunked(bits, 0, h, mode)
    ocn, ocs = O.quantize_chunked(bits, 1, h, mode)
    for got, want, name in ((rn, orn, "row nibbles"), (rs, ors, "row scales"),
                            (cn, ocn, "col nibbles"), (cs, ocs, "col scales")):
        assert got.shape == want.shape, f"{what} {name}"
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{what}: {len(bad)} {name} bytes differ, first {bad[:4].tolist()}"


# one-read kernel (rows % 128, cols % 256) and the two-kernel path otherwise
DUAL_SHAPES = [(128, 256), (256, 512), (384, 1280), (128, 4096), (32, 32), (96, 160), (128, 288)]


@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_dual_small_shapes_bit_exact(h, mode):
    for i, (r, c) in enumerate(DUAL_SHAPES):
        bits = heavy(r, c, 4000 + 11 * i)
        assert_dual_same(bits, h, mode, f"dual h={h} mode={mode} shape={(r, c)}")


@pytest.mark.parametrize("h", [0, 16, 32])
@pytest.mark.parametrize("mode", [0, 1])
def test_dual_edge_values_bit_exact(h, mode):
    # special blocks along rows (first half) and, transposed, down columns (second half)
    bits = np.concatenate([edge_matrix(128, 256, seed=9), edge_matrix(256, 128, seed=10).T], 0)
    bits = np.ascontiguousarray(bits)
    assert_dual_same(bits, h, mode, f"dual edge h={h} mode={mode}")


@pytest.mark.parametrize("h,mode", [(16, 0), (16, 1), (32, 0), (0, 1)])
def test_dual_quantizer_workload_full_size(quant_workload, h, mode):
    assert_dual_same(quant_workload, h, mode, f"dual full h={h} mode={mode}")


def exhaustive_encode_matrix(mode):
    """Every finite bf16 value, both signs, at every shared exponent E the
    format reaches: for each bf16 exponent field f = 0..254 one anchor
    (element 0 of its blocks) fixes E -- mantissa 1.1111111b in OCP floor
    mode (so scaled values reach 7.97 and the saturation band), mantissa
    1.1b in ceil mode (scaled values reach 6 exactly) -- and the other 31
    elements of those blocks run through every finite bf16 value of
    magnitude at most the anchor. H0 row blocks, 32 blocks per row."""
    mags = np.arange(0x7F80, dtype=np.uint16)          # +0 .. bf16 max
    anchors_m = 0x7F if mode == 0 else 0x40
    blocks = []
    for f in range(255):
        anchor = np.uint16((f << 7) | anchors_m)
        vals = mags[mags <= anchor]
        vals = np.concatenate([vals, vals | 0x8000])   # both signs
        n = -(-vals.size // 31)
        body = np.zeros(n * 31, np.uint16)
        body[:vals.size] = vals
        blk = np.empty((n, 32), np.uint16)
        blk[:, 0] = anchor
        blk[:, 1:] = body.reshape(n, 31)
        blocks.append(blk)
    b = np.concatenate(blocks)
    pad = (-b.shape[0]) % 32
    b = np.concatenate([b, np.zeros((pad, 32), np.uint16)])
    return b.reshape(-1, 1024)


@pytest.mark.parametrize("mode", [0, 1])
def test_e2m1_encode_exhaustive(mode):
    """The hardware's scaled FP4 convert against the oracle's nearest-value
    rule ([P1] section A.1: round to the nearest FP4 value) over every
    finite bf16 value at every shared exponent, row-wise and column-wise."""
    bits = exhaustive_encode_matrix(mode)
    assert_same(bits, 0, 0, mode, f"exhaustive encode row mode={mode}")
    assert_same(np.ascontiguousarray(bits.T), 1, 0, mode, f"exhaustive encode col mode={mode}")


PAIRS = [
    (((300, 640), 0), ((128, 96), 0)),        # row + row
    (((4096, 8320), 0), ((96, 320), 0)),      # lane-contiguous row (> 2^20 blocks) + row
    (((64, 256), 0), ((512, 260), 1)),        # row + column (8-band staged)
    (((256, 100), 1), ((768, 36), 1)),        # column + column
    (((512, 64), 1), ((4096, 8320), 0)),      # column + lane-contiguous row
    (((4096, 8320), 0), ((512, 260), 1)),     # lane-contiguous row + column (column runs first)
    (((96, 64), 1), ((64, 96), 0)),           # column shape without the staged form: two launches
]


@pytest.mark.parametrize("pair", PAIRS)
@pytest.mark.parametrize("h,mode", [(16, 0), (32, 1), (0, 1)])
def test_pair_launch_bit_exact(pair, h, mode):
    """mxfp4_quantize_pair: both operands byte for byte the oracle's."""
    import torch
    import mxfp4_quantized_gemm_amd as mx
    bits, outs = [], []
    for k, ((r, c), axis) in enumerate(pair):
        b = heavy(r, c, 4400 + 3 * k + r % 7)
        ns, ss = mx.packed_shapes(r, c, axis)
        bits.append((b, axis))
        outs.append((to_dev_bf16(b), torch.full(ns, 0xAB, dtype=torch.uint8, device="cuda"),
                     torch.full(ss, 0xAB, dtype=torch.uint8, device="cuda")))
    (ba, axa), (bb, axb) = bits
    (xa, na, sa), (xb, nb, sb) = outs
    mx.mxfp4_quantize_pair(xa, ba.shape[0], ba.shape[1], axa, na, sa, xb, bb.shape[0], bb.shape[1],
                           axb, nb, sb, h, mode)
    torch.cuda.synchronize()
    for (b, axis), (_, n, s), w in zip(bits, outs, "AB"):
        on, os_ = O.quantize_chunked(b, axis, h, mode)
        assert np.array_equal(n.cpu().numpy(), on), f"{w} nibbles {pair} h={h} mode={mode}"
        assert np.array_equal(s.cpu().numpy(), os_), f"{w} scales {pair} h={h} mode={mode}"


@pytest.mark.parametrize("axis", [0, 1, 2])
def test_source_beyond_4gib(axis):
    """A bf16 source of 4 GiB + 16 MiB (65792 x 32768, more than 2^31
    elements; the lane-contiguous row, the staged column and the
    lane-contiguous 2D kernels): blocks on both sides of element 2^31
    against the oracle, row blocks by whole rows, column blocks by 32-row
    bands of sampled columns, 2D tiles by sampled tiles."""
    import torch
    import mxfp4_quantized_gemm_amd as mx
    rows, cols = 65536 + 256, 32768
    g = torch.Generator(device="cuda")
    g.manual_seed(77 + axis)
    x = torch.randn((rows, cols), dtype=torch.float32, device="cuda", generator=g)
    x = x.to(torch.bfloat16)
    nib, sc = mx.quantize(x, axis, 16, 0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(axis)
    edge_rows = [0, 65535, 65536, rows - 1]             # row 65536 starts at element 2^31

    def src(r0, r1, c0, c1):
        return x[r0:r1, c0:c1].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)

    if axis == 0:
        for r in edge_rows + rng.integers(0, rows, 4).tolist():
            on, os_ = O.quantize(src(r, r + 1, 0, cols), O.AXIS_ROW, 16, 0)
            assert np.array_equal(nib[r:r + 1].cpu().numpy(), on), f"row {r} nibbles"
            assert np.array_equal(sc[r:r + 1].cpu().numpy(), os_), f"row {r} scales"
    else:
        cs = sorted(set([0, cols - 1] + rng.integers(0, cols, 30).tolist()))
        for r in edge_rows:
            b = r // 32
            for c in cs[:8] if axis == 2 else [0]:
                if axis == 1:
                    blk = src(32 * b, 32 * b + 32, 0, cols)[:, cs]
                    on, os_ = O.quantize(np.ascontiguousarray(blk), O.AXIS_COL, 16, 0)
                    got_n = nib[cs, 16 * b:16 * b + 16].cpu().numpy()
                    got_s = sc[cs, b:b + 1].cpu().numpy()
                else:
                    t = c // 32
                    on, os_ = O.quantize(src(32 * b, 32 * b + 32, 32 * t, 32 * t + 32),
                                         O.AXIS_2D, 16, 0)
                    got_n = nib[32 * b:32 * b + 32, 16 * t:16 * t + 16].cpu().numpy()
                    got_s = sc[b:b + 1, t:t + 1].cpu().numpy()
                assert np.array_equal(got_n, on), f"axis {axis} band {b} col {c} nibbles"
                assert np.array_equal(got_s, os_), f"axis {axis} band {b} col {c} scales"
    del x, nib, sc
    torch.cuda.empty_cache()
