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


# ---------------------------------------------------- GEMM on MBS operands
# mxfp4_gemm_mbs against the oracle's fp64 product of dequantize_mbs
# operands, per element within the GEMM bound 1e-5 * sum |a||b| (+ 2^-8
# |C_ref| for bf16 output).
def _random_mbs_operand(rows, K, seed):
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8),
            rng.integers(112, 143, size=(rows, K // 32), dtype=np.uint8),
            rng.integers(0, 256, size=(rows, K // 128), dtype=np.uint8))


def _gemm_mbs(a, b, M, N, K, out_dtype):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    from tests.gpu_util import to_dev_u8
    C = torch.empty((M, N), dtype=torch.float32 if out_dtype == 0 else torch.bfloat16,
                    device="cuda")
    mx.mxfp4_gemm_mbs(*[to_dev_u8(x) for x in a], *[to_dev_u8(x) for x in b], M, N, K, C,
                      out_dtype)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def _check_mbs_product(C, a, b, out_bf16, what):
    Cr, S = O.gemm_ref(O.dequantize_mbs(*a), O.dequantize_mbs(*b))
    err = np.abs(C - Cr)
    bad = ~(err <= O.gemm_tolerance(S, Cr, out_bf16))
    assert np.all(C[S == 0] == 0), what
    if bad.any():
        i, j = np.argwhere(bad)[0]
        pytest.fail(f"{what}: {bad.sum()} out of tolerance, C[{i},{j}]={C[i, j]!r} "
                    f"ref={Cr[i, j]!r} S={S[i, j]!r}")


@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (130, 70, 128), (33, 257, 384), (200, 300, 640),
                                   (256, 384, 4096), (300, 129, 1152), (1100, 1300, 2048)])
@pytest.mark.parametrize("out_dtype", [0, 1])
def test_gemm_mbs_random_operands(M, N, K, out_dtype):
    """Every nibble code and mantissa byte; K % 256 == 128 leaves the last
    k-tile half empty."""
    a = _random_mbs_operand(M, K, 11 * M + K)
    b = _random_mbs_operand(N, K, 13 * N + K + 1)
    _check_mbs_product(_gemm_mbs(a, b, M, N, K, out_dtype), a, b, out_dtype == 1,
                       f"M={M} N={N} K={K} out={out_dtype}")


@pytest.mark.parametrize("mode", [0, 1])
def test_gemm_mbs_on_quantized_operands(mode):
    """Fprop-shaped: X (heavy-tailed, outlier channels) and W quantized with
    MBS on the GPU (bit-exact with the oracle above), multiplied by
    mxfp4_gemm_mbs; the product is within the bound of the oracle's, and
    closer to the exact bf16 product than without the postscale would be."""
    import torch
    import mxfp4_quantized_gemm_amd as mx
    rng = np.random.default_rng(50 + mode)
    T, N, K = 192, 160, 1024
    x = rng.standard_normal((T, K))
    x[:, rng.choice(K, 10, replace=False)] *= 40
    X = synthetic.f64_to_bf16_bits(x)
    W = synthetic.f64_to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    qa = [t.cpu().numpy() for t in mx.quantize_mbs(to_dev_bf16(X), 0, 16, mode)]
    qb = [t.cpu().numpy() for t in mx.quantize_mbs(to_dev_bf16(W), 0, 16, mode)]
    torch.cuda.synchronize()
    C = _gemm_mbs(qa, qb, T, N, K, 0)
    _check_mbs_product(C, qa, qb, False, f"quantized mode={mode}")
    P = O.unquantized_product("fprop", X, W)
    rel = np.linalg.norm(C - P) / np.linalg.norm(P)
    assert rel < 0.2
