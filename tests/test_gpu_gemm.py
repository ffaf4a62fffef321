"""GPU parity of the MXFP4 GEMM (mxfp4_gemm through the C ABI) against the
oracle's fp64 product of the dequantized operands.

Bar (per element): |C - C_ref| <= 1e-5 * S with S = sum_k |a_k| |b_k| for
fp32 output; for bf16 output the bf16 rounding of the result is added,
+ 2^-8 |C_ref|. Where S == 0 the output must be exactly 0. Operands are
seeded random packed bytes (every nibble code, scale bytes kept where the
fp32 accumulator stays in its normal range).
"""
import numpy as np
import pytest

import oracle as O
from tests.gpu_util import to_dev_u8

pytestmark = pytest.mark.gpu


def random_operand(rows, K, seed, sc_lo=112, sc_hi=142):
    rng = np.random.default_rng(seed)
    nib = rng.integers(0, 256, size=(rows, K // 2), dtype=np.uint8)
    sc = rng.integers(sc_lo, sc_hi + 1, size=(rows, K // 32), dtype=np.uint8)
    return nib, sc


def run_gemm(a, b, M, N, K, out_dtype=0):
    import torch
    import mxfp4_quantized_gemm_amd as mx
    C = torch.empty((M, N), dtype=torch.float32 if out_dtype == 0 else torch.bfloat16, device="cuda")
    mx.mxfp4_gemm(to_dev_u8(a[0]), to_dev_u8(a[1]), to_dev_u8(b[0]), to_dev_u8(b[1]), M, N, K, C,
                  out_dtype)
    torch.cuda.synchronize()
    return C.float().cpu().numpy().astype(np.float64)


def check(C, a, b, out_bf16=False, what=""):
    Cr, S = O.gemm_ref(O.dequantize(*a), O.dequantize(*b))
    tol = O.gemm_tolerance(S, Cr, out_bf16)
    err = np.abs(C - Cr)
    bad = ~(err <= tol)
    zero = S == 0
    assert np.all(C[zero] == 0), what
    if bad.any():
        i, j = np.argwhere(bad)[0]
        pytest.fail(f"{what}: {bad.sum()} elements out of tolerance, e.g. C[{i},{j}]={C[i, j]!r} "
                    f"ref={Cr[i, j]!r} S={S[i, j]!r}")


SHAPES = [
    (128, 256, 256),     # the tiny Fprop shape
    (1, 1, 32),          # smallest problem, K = one block
    (130, 70, 96),       # ragged M, N; K not a multiple of the 256-deep k-tile
    (33, 257, 288),
    (256, 384, 4096),    # Llama reduction length
    (200, 300, 544),
    (512, 512, 1024),    # several full tiles in every direction
    (1, 1, 256),         # large-tile kernel, one element
    (300, 200, 512),     # large-tile kernel, ragged M and N
    (1000, 600, 768),    # large-tile kernel, several ragged tiles, odd k-tile pairs
    (768, 1024, 2048),
    (1, 1, 2048),        # LDS-DMA kernel (K % 2048 == 0), one element
    (300, 520, 6144),    # LDS-DMA kernel, ragged M and N, three scale-group pairs
    (257, 261, 2048),    # LDS-DMA kernel, N % 4 != 0 (element-wise epilogue)
    (513, 260, 8192),    # LDS-DMA kernel, the Wgrad reduction length
    # more 256x256 tiles than the GPU has compute units, with ragged last
    # tiles: later tiles of each work-group start from operands that the
    # previous tile's k-loop prefetched
    (6448, 6504, 2048),  # 26 x 26 = 676 tiles, both edges ragged
    (4200, 4400, 4096),  # 17 x 18 = 306 tiles, the Llama reduction length
    # 2 x 130 = 260 tiles on 256 compute units: four work-groups walk to a
    # second tile; 33280 columns of output; ragged M
    (500, 33280, 2048),
    # the general kernel (K % 256 != 0) over 16 x 24 = 384 tiles, ragged
    (2000, 3000, 800),
]


@pytest.mark.parametrize("M,N,K", SHAPES)
@pytest.mark.parametrize("out_dtype", [0, 1])
def test_gemm_parity(M, N, K, out_dtype):
    a = random_operand(M, K, M * 7 + K)
    b = random_operand(N, K, N * 11 + K + 1)
    C = run_gemm(a, b, M, N, K, out_dtype)
    check(C, a, b, out_dtype == 1, f"M={M} N={N} K={K} out={out_dtype}")


def test_gemm_every_scale_byte_in_range():
    """Scale bytes 80..174 on both sides: block products span 2^-94..2^94."""
    M, N, K = 96, 160, 4064
    rng = np.random.default_rng(1)
    a = (rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8),
         rng.integers(80, 175, size=(M, K // 32), dtype=np.uint8))
    b = (rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8),
         rng.integers(80, 175, size=(N, K // 32), dtype=np.uint8))
    check(run_gemm(a, b, M, N, K), a, b, what="wide scales")


@pytest.mark.parametrize("K", [256, 2048])
def test_gemm_zero_and_nan_blocks(K):
    """All-zero operand rows give exact zeros; an E8M0 NaN byte (0xFF)
    poisons exactly the outputs that read that block, as in the oracle."""
    M, N = 64, 96
    a = random_operand(M, K, 5)
    b = random_operand(N, K, 6)
    a[0][3] = 0                # row 3 of A is all zero nibbles
    a[1][5, 2] = 255           # block 2 of A row 5 is NaN
    a[1][7, K // 32 - 1] = 255  # and the last block of row 7
    C = run_gemm(a, b, M, N, K)
    assert np.all(C[3] == 0)
    assert np.all(np.isnan(C[5])) and np.all(np.isnan(C[7]))
    Cr, _ = O.gemm_ref(O.dequantize(*a), O.dequantize(*b))
    assert np.array_equal(np.isnan(C), np.isnan(Cr))
    keep = np.ones(M, bool)
    keep[[5, 7]] = False
    a2 = (a[0][keep], a[1][keep])
    check(C[keep], a2, b, what="rows without NaN")


def test_gemm_deterministic():
    M, N, K = 300, 200, 1024
    a = random_operand(M, K, 8)
    b = random_operand(N, K, 9)
    c1 = run_gemm(a, b, M, N, K)
    c2 = run_gemm(a, b, M, N, K)
    assert np.array_equal(c1, c2)


def test_gemm_operand_beyond_4gib():
    """An A operand of 4 GiB + 1 MiB (2^21 + 512 rows of 2048 bytes, K = 4096)
    takes the general kernel with 64-bit offsets (the large-tile kernels
    address operands with 32-bit offsets). Rows on both sides of byte
    offset 2^32 are checked against the oracle on every output column."""
    import torch
    import mxfp4_quantized_gemm_amd as mx
    M, N, K = (1 << 21) + 512, 128, 4096
    g = torch.Generator(device="cuda")
    g.manual_seed(4242)
    A = torch.randint(0, 256, (M, K // 2), dtype=torch.uint8, device="cuda", generator=g)
    As = torch.randint(120, 135, (M, K // 32), dtype=torch.uint8, device="cuda", generator=g)
    b = random_operand(N, K, 77, 120, 134)
    B, Bs = to_dev_u8(b[0]), to_dev_u8(b[1])
    C = torch.empty((M, N), dtype=torch.float32, device="cuda")
    mx.mxfp4_gemm(A, As, B, Bs, M, N, K, C, mx.OUT_F32)
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 1, 1 << 20, (1 << 21) - 1, 1 << 21, (1 << 21) + 1, M - 1],
                                     rng.integers(0, M, 24)]))
    idx = torch.from_numpy(rows).to("cuda")
    a = (A[idx].cpu().numpy(), As[idx].cpu().numpy())
    got = C[idx].cpu().numpy().astype(np.float64)
    del A, As, C
    torch.cuda.empty_cache()
    check(got, a, b, what=f"A of {M * K // 2} bytes, rows {rows.tolist()}")
