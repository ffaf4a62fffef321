"""CPU oracle for the H16 + MXFP4 quantize + MXFP4 GEMM path.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import this
module: only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
CPU-baseline leg use it. It shares no code with the HIP library.

Plain, slow, obviously correct numpy. Floating point is fp64 except where
the method fixes fp32 (the rotation butterfly, the values entering the
quantizer). No fusion, no blocking beyond what the definitions state.

Pages cited (by title and section):

[P1] "Pretraining Large Language Models with MXFP4 on Native FP4 Hardware"
     (arXiv:2605.09825, summary page): quick-read block (reconstruction
     formula, H H^T = I, the three cancellations), section A.1 (MX micro-
     scaling, shared exponent = block max exponent, round to nearest FP4),
     section A.2 (deterministic, tiled 16x16 Hadamard injected before the
     GEMM), section C.1/C.2/C.3 (Fprop/Dgrad/Wgrad cancellation), section D
     (1x32 row-wise, 32x1 column-wise, 32x32 2D block scales).
[P2] "FP4 training" article on arXiv:2501.17116 (techwalker), section 1
     (E2M1: 2 exponent bits, 1 mantissa bit, range -6..6).
[P3] "Decomposing MXFP4 quantization error" blog (arXiv:2605.20402):
     "pain point" section (OCP MX block of 32, E8M0 scale = 2^n, E2M1 grid
     {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}), "core insight" section
     (ideal scale s* = max|x|/q_max, ceiling-rounded E8M0 scale, the three-way
     error decomposition, deadzone |x| < m_b/24), "Property 1" (exact
     orthogonality and the one-cross-term MSE identity), "scale bias"
     section (gamma = s_b/s* = 2^delta, delta in [0, 1)), and the note that
     native MXFP4 accumulates in FP32.

Readings where the pages are silent (each is also listed in the design
notes): block size exactly 32 (P3); OCP floor rule E = floor(log2 m_b) - 2,
i.e. the max exponent offset by E2M1's emax = 2 (P1 A.1 read with P3's OCP
MX reference); ceil rule = smallest E with 6 * 2^E >= m_b (P3); ties to the
even code; saturation at 6; all-zero block -> E = -127; E clamped to
[-127, 127]; sign of zero kept; butterfly stages 1, 2, 4, 8 (, 16)
ascending with one multiply by c_h after the adds (c_16 = 0.25,
c_32 = RN_fp32(2^-2.5)); a block holding a non-finite value after rotation
gets scale byte 0xFF and zero nibbles.
"""
from __future__ import annotations

import numpy as np

AXIS_ROW, AXIS_COL, AXIS_2D = 0, 1, 2
MODE_OCP_FLOOR, MODE_CEIL = 0, 1
BLOCK = 32

# E2M1 magnitudes by 3-bit code ([P3] pain-point section; [P2] section 1).
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

# Normalisation of the Sylvester matrix: H_h = c_h * (+-1 matrix), so that
# H H^T = I ([P1] quick-read block). 1/4 is exact; 1/sqrt(32) is rounded
# once to fp32.
C_H16 = np.float32(0.25)
C_H32 = np.uint32(0x3E3504F3).view(np.float32)


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values, exactly (a 16-bit left shift)."""
    return np.left_shift(np.asarray(bits, dtype=np.uint16).astype(np.uint32),
                         np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# Rotation ([P1] A.2: deterministic Hadamard before the GEMM, tiled blocks)
# --------------------------------------------------------------------------
def hadamard_rotate(x: np.ndarray, h: int) -> np.ndarray:
    """Rotate every aligned group of ``h`` elements along the last axis.

    y = x_group * H_h, computed as the fp32 butterfly: for stage
    s = 1, 2, 4, ... h/2, each pair (i, i+s) with (i & s) == 0 becomes
    (a + b, a - b); then one multiply by c_h. Each operation is a single
    fp32 round-to-nearest-even step. In exact arithmetic the result is
    x * H with H[i][j] = c_h * (-1)^popcount(i & j).
    ``h == 0`` returns the input unchanged (no rotation).
    """
    x = np.asarray(x, dtype=np.float32)
    if h == 0:
        return x.copy()
    if h not in (16, 32):
        raise ValueError("hadamard size must be 0, 16 or 32")
    n = x.shape[-1]
    if n % h:
        raise ValueError("rotated axis must be a multiple of the Hadamard size")
    lead = x.shape[:-1]
    y = x.reshape(lead + (n // h, h)).copy()
    s = 1
    while s < h:
        # index i = q*2s + t*s + r: t == 0 are the (i & s) == 0 elements,
        # t == 1 their partners i + s.
        v = y.reshape(lead + (n // h, h // (2 * s), 2, s))
        a = v[..., 0, :].copy()
        b = v[..., 1, :].copy()
        v[..., 0, :] = a + b
        v[..., 1, :] = a - b
        s *= 2
    y *= C_H16 if h == 16 else C_H32
    return y.reshape(x.shape)


# --------------------------------------------------------------------------
# E8M0 shared scale ([P1] A.1; [P3] core insight, scale-bias section)
# --------------------------------------------------------------------------
def e8m0_exponent(m_b: np.ndarray, mode: int) -> np.ndarray:
    """Shared exponent E (int64) of blocks with absolute maximum ``m_b``.

    Write m_b = m * 2^e with m in [1, 2) (the true exponent, also for
    subnormal m_b).
    ocp_floor: E = e - 2, the block's max exponent minus E2M1's emax.
    ceil:      the smallest E with 6 * 2^E >= m_b: E = e - 2 if m <= 1.5,
               else e - 1 (so 2^E >= m_b / 6 = s*).
    m_b == 0 gives E = -127. E is clamped to [-127, 127].
    """
    mb = np.asarray(m_b, dtype=np.float64)  # fp32 -> fp64 is exact
    frac, e1 = np.frexp(mb)                 # mb = frac * 2^e1, frac in [0.5, 1)
    m = 2.0 * frac
    e = e1.astype(np.int64) - 1
    if mode == MODE_OCP_FLOOR:
        E = e - 2
    elif mode == MODE_CEIL:
        E = np.where(m <= 1.5, e - 2, e - 1)
    else:
        raise ValueError("unknown scale mode")
    E = np.where(mb == 0.0, -127, E)
    return np.clip(E, -127, 127).astype(np.int64)


# --------------------------------------------------------------------------
# E2M1 element code ([P1] A.1: round to the nearest FP4 value; [P3] grid)
# --------------------------------------------------------------------------
def e2m1_code(y: np.ndarray, E: np.ndarray) -> np.ndarray:
    """4-bit codes (sign << 3 | magnitude) of y / 2^E.

    v = y * 2^-E is exact in fp64. The magnitude code is the nearest grid
    value with ties to the even code and saturation at 6:
      a <= 0.25 -> 0, a < 0.75 -> 1, a <= 1.25 -> 2, a < 1.75 -> 3,
      a <= 2.5  -> 4, a < 3.5  -> 5, a <= 5    -> 6, otherwise 7.
    The sign bit of y is kept, also when the magnitude rounds to 0.
    """
    y = np.asarray(y, dtype=np.float32)
    v = np.ldexp(y.astype(np.float64), -np.asarray(E, dtype=np.int64))
    a = np.abs(v)
    mag = ((a > 0.25).astype(np.uint8) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
           + (a > 2.5) + (a >= 3.5) + (a > 5.0)).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8)
    return (sign << 3) | mag


def _pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """Byte j of a row = code[2j] | code[2j+1] << 4."""
    c = codes.reshape(codes.shape[:-1] + (codes.shape[-1] // 2, 2))
    return (c[..., 0] | (c[..., 1] << 4)).astype(np.uint8)


def _quantize_rows(y: np.ndarray, mode: int):
    """1x32 blocks along the last axis of fp32 ``y`` -> (nibbles, scales)."""
    r, c = y.shape
    yb = y.reshape(r, c // BLOCK, BLOCK)
    m_b = np.max(np.abs(yb), axis=2)
    finite = np.all(np.isfinite(yb), axis=2)
    m_b = np.where(finite, m_b, np.float32(0))
    E = e8m0_exponent(m_b, mode)
    codes = e2m1_code(yb, E[:, :, None])
    codes = np.where(finite[:, :, None], codes, np.uint8(0))
    sc = np.where(finite, E + 127, 255).astype(np.uint8)
    return _pack_nibbles(codes.reshape(r, c)), sc


def _quantize_2d(y: np.ndarray, mode: int):
    """32x32 tiles of fp32 ``y`` -> (nibbles [r][c/2], scales [r/32][c/32])."""
    r, c = y.shape
    yt = y.reshape(r // BLOCK, BLOCK, c // BLOCK, BLOCK)
    m_b = np.max(np.abs(yt), axis=(1, 3))
    finite = np.all(np.isfinite(yt), axis=(1, 3))
    m_b = np.where(finite, m_b, np.float32(0))
    E = e8m0_exponent(m_b, mode)
    codes = e2m1_code(yt, E[:, None, :, None])
    codes = np.where(finite[:, None, :, None], codes, np.uint8(0))
    sc = np.where(finite, E + 127, 255).astype(np.uint8)
    return _pack_nibbles(codes.reshape(r, c)), sc


def quantize(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int):
    """Rotate and MXFP4-quantize a bf16 matrix [rows][cols].

    axis=row  ([P1] D, 1x32): rotate and block along cols.
              nibbles [rows][cols/2], scales [rows][cols/32].
    axis=col  ([P1] D, 32x1): rotate and block down rows; the output is
              transposed so the blocked axis is contiguous:
              nibbles [cols][rows/2], scales [cols][rows/32]. This is the row
              rule applied to the transposed matrix.
    axis=2d   ([P1] D, 32x32): rotate along cols, one scale per 32x32 tile.
              nibbles [rows][cols/2], scales [rows/32][cols/32].
    """
    x = bf16_to_f32(src_bf16)
    if x.ndim != 2:
        raise ValueError("expected a matrix")
    if axis == AXIS_COL:
        x = np.ascontiguousarray(x.T)
    if x.shape[1] % BLOCK or (axis == AXIS_2D and x.shape[0] % BLOCK):
        raise ValueError("blocked axis must be a multiple of 32")
    y = hadamard_rotate(x, hadamard)
    if axis == AXIS_2D:
        return _quantize_2d(y, mode)
    return _quantize_rows(y, mode)


def quantize_chunked(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int,
                     chunk: int = 1024, threads: int = 1):
    """``quantize`` over row (or, for col, column) slabs to bound memory.

    Blocks never straddle slabs (slab sizes are multiples of 32), so the
    result equals ``quantize`` on the whole matrix. With ``threads`` > 1 the
    slabs are quantized by a thread pool (numpy's array operations release
    the interpreter lock); the slabs and their order are the same.
    """
    r, c = src_bf16.shape
    if axis == AXIS_COL:
        slabs = [src_bf16[:, j:j + chunk] for j in range(0, c, chunk)]
    else:
        slabs = [src_bf16[i:i + chunk] for i in range(0, r, chunk)]
    if threads > 1 and len(slabs) > 1:
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(max_workers=threads) as ex:
            parts = list(ex.map(lambda s: quantize(s, axis, hadamard, mode), slabs))
    else:
        parts = [quantize(s, axis, hadamard, mode) for s in slabs]
    return (np.concatenate([p[0] for p in parts], axis=0),
            np.concatenate([p[1] for p in parts], axis=0))


# --------------------------------------------------------------------------
# Error-only comparison arms that [P1] reports as diverging under full MXFP4
# training (quick-read block, section A.2, hypothesis H2: random Hadamard
# transforms and stochastic rounding). They are built here to measure their quantization
# error next to the deterministic H16 + round-to-nearest path; the random
# numbers are inputs.
# --------------------------------------------------------------------------
def quantize_rs(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int,
                signs: np.ndarray):
    """Random-sign Hadamard: rotate diag(s) x instead of x, s_i = -1 where
    ``signs[i]`` is 1 and +1 where it is 0, i indexing the blocked
    (reduction) axis: ``signs`` has ``cols`` entries for row blocks and
    ``rows`` for column blocks. Both operands of a product take the same
    signs, so (X D H)(W D H)^T = X W^T. A sign flip of a bf16 value is
    exact, so this is ``quantize`` of the sign-flipped matrix."""
    bits = np.asarray(src_bf16, dtype=np.uint16)
    s = np.asarray(signs, dtype=np.uint8)
    if axis == AXIS_ROW:
        if s.shape != (bits.shape[1],):
            raise ValueError("row blocks take one sign per column")
        flip = s[None, :]
    elif axis == AXIS_COL:
        if s.shape != (bits.shape[0],):
            raise ValueError("column blocks take one sign per row")
        flip = s[:, None]
    else:
        raise ValueError("random signs are defined here for 1x32 and 32x1 blocks")
    if np.any(s > 1):
        raise ValueError("signs are 0 or 1")
    return quantize(bits ^ (flip.astype(np.uint16) << np.uint16(15)), axis, hadamard, mode)


def sr_codes(y: np.ndarray, E: np.ndarray, rnd: np.ndarray) -> np.ndarray:
    """Stochastic-rounding codes (sign << 3 | magnitude) of y / 2^E.

    a = |y| 2^-E (exact in fp64). Below 6, with g_lo <= a < g_hi the two
    neighbouring grid values, p = (a - g_lo) / (g_hi - g_lo) (exact: the
    gap is 0.5, 1 or 2) and the magnitude rounds up to g_hi exactly when
    rnd < p 2^32, i.e. with probability p for a uniform 32-bit rnd, so
    that the expected value is a. a >= 6 saturates to 6. The sign bit of
    y is kept, as in ``e2m1_code``.
    """
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(np.ldexp(y.astype(np.float64), -np.asarray(E, dtype=np.int64)))
    lo = ((a >= 0.5).astype(np.int64) + (a >= 1.0) + (a >= 1.5) + (a >= 2.0) + (a >= 3.0)
          + (a >= 4.0) + (a >= 6.0))
    g_lo = E2M1_GRID[lo]
    gap = E2M1_GRID[np.minimum(lo + 1, 7)] - g_lo
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(lo < 7, (a - g_lo) / np.where(gap > 0, gap, 1.0), 0.0)
    up = np.asarray(rnd, dtype=np.uint32).astype(np.float64) < p * 4294967296.0
    mag = np.where(lo >= 7, 7, lo + up).astype(np.uint8)
    sign = np.signbit(y).astype(np.uint8)
    return (sign << 3) | mag


def quantize_sr(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int,
                rand_u32: np.ndarray):
    """Stochastic-rounding operand: the scales of ``quantize`` (same E8M0
    rule on the same block maxima), element codes from ``sr_codes`` with
    one uniform 32-bit integer per source element (``rand_u32`` has the
    source's shape [rows][cols]; element (r, c) uses rand_u32[r][c] for
    either axis). Non-finite blocks are 0xFF with zero nibbles."""
    x = bf16_to_f32(src_bf16)
    rnd = np.asarray(rand_u32, dtype=np.uint32)
    if rnd.shape != x.shape:
        raise ValueError("one random integer per source element")
    if axis == AXIS_COL:
        x = np.ascontiguousarray(x.T)
        rnd = np.ascontiguousarray(rnd.T)
    elif axis != AXIS_ROW:
        raise ValueError("stochastic rounding is defined here for 1x32 and 32x1 blocks")
    if x.shape[1] % BLOCK:
        raise ValueError("blocked axis must be a multiple of 32")
    y = hadamard_rotate(x, hadamard)
    r, c = y.shape
    yb = y.reshape(r, c // BLOCK, BLOCK)
    m_b = np.max(np.abs(yb), axis=2)
    finite = np.all(np.isfinite(yb), axis=2)
    m_b = np.where(finite, m_b, np.float32(0))
    E = e8m0_exponent(m_b, mode)
    codes = sr_codes(yb, E[:, :, None], rnd.reshape(r, c // BLOCK, BLOCK))
    codes = np.where(finite[:, :, None], codes, np.uint8(0))
    sc = np.where(finite, E + 127, 255).astype(np.uint8)
    return _pack_nibbles(codes.reshape(r, c)), sc


# --------------------------------------------------------------------------
# Outlier fallback ([P3] "three targeted fixes" section, OF: two-step
# residual quantization x_OF = Q(x) + alpha Q(x - Q(x)), alpha = 0.5)
# --------------------------------------------------------------------------
OF_ALPHA = 0.5


def quantize_of(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int):
    """OF operand of a bf16 matrix as one K-concatenated packed operand.

    y = the rotated values ``quantize`` encodes (row or col axis);
    q1 = Q(y) (this module's quantizer, ``mode``); r = fl32(y - q1);
    q2 = Q(fl32(alpha r)) with alpha = 1/2 applied as a prescale of the
    residual (equal to alpha Q(r) whenever the residual block's scale is
    above the E8M0 floor, the only place the two can differ).
    Returns (nibbles [R][2 Kb/2], scales [R][2 Kb/32]): row i holds q1's
    row followed by q2's row, so a GEMM of depth 2 Kb against the other
    operand repeated twice along K computes sum (q1 + q2) b. A block with a
    non-finite rotated value is 0xFF in both halves.
    """
    x = bf16_to_f32(src_bf16)
    if axis == AXIS_COL:
        x = np.ascontiguousarray(x.T)
    elif axis != AXIS_ROW:
        raise ValueError("OF is defined here for 1x32 and 32x1 blocks")
    if x.shape[1] % BLOCK:
        raise ValueError("blocked axis must be a multiple of 32")
    y = hadamard_rotate(x, hadamard)
    n1, s1 = _quantize_rows(y, mode)
    q1 = dequantize(n1, s1)                       # exact in fp32 where finite
    with np.errstate(invalid="ignore"):
        r = (y - q1.astype(np.float32)).astype(np.float32)
        h = (np.float32(OF_ALPHA) * r).astype(np.float32)
    n2, s2 = _quantize_rows(h, mode)
    return np.concatenate([n1, n2], axis=1), np.concatenate([s1, s2], axis=1)


# --------------------------------------------------------------------------
# Macro-block scaling ([P3] "three targeted fixes" section, MBS: an 8-bit
# mantissa (1 + m) per macro-block of B_M = 128 elements, used as
# x_hat = Q((1 + m) x) / (1 + m))
# --------------------------------------------------------------------------
MBS_BLOCK = 128


def mbs_mantissa(M: np.ndarray) -> np.ndarray:
    """8-bit mantissa byte m of macro-blocks with absolute maximum ``M``.

    Reading of the pages (which fix the form, not the rule): c = 1 + m/256
    is the largest such factor with c M <= 6 2^k, k the smallest integer
    with 6 2^k >= M, so the prescaled macro maximum sits at the top of its
    E8M0 bracket: m = floor(256 (6 2^k / M - 1)), evaluated in fp64.
    M == 0 or non-finite gives m = 0.
    """
    Md = np.asarray(M, dtype=np.float64)
    ok = np.isfinite(Md) & (Md > 0)
    safe = np.where(ok, Md, 1.0)
    frac, e1 = np.frexp(safe)                  # safe = frac 2^e1, frac in [0.5, 1)
    f, e = 2.0 * frac, e1.astype(np.int64) - 1
    k = np.where(f <= 1.5, e - 2, e - 1)
    c = np.ldexp(6.0, k) / safe
    m = np.floor((c - 1.0) * 256.0)
    return np.where(ok, np.clip(m, 0, 255), 0).astype(np.uint8)


def quantize_mbs(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int):
    """MBS operand: (nibbles, scales, mbs) with mbs [R][Kb/128] the mantissa
    bytes; nibbles and E8M0 scales are this module's quantizer applied to
    fl32(c y), c = 1 + m/256 of y's macro-block (y the rotated values, row or
    col axis, Kb % 128 == 0). Dequantize with ``dequantize_mbs``."""
    x = bf16_to_f32(src_bf16)
    if axis == AXIS_COL:
        x = np.ascontiguousarray(x.T)
    elif axis != AXIS_ROW:
        raise ValueError("MBS is defined here for 1x32 and 32x1 blocks")
    if x.shape[1] % MBS_BLOCK:
        raise ValueError("blocked axis must be a multiple of 128")
    y = hadamard_rotate(x, hadamard)
    r, kb = y.shape
    yb = y.reshape(r, kb // MBS_BLOCK, MBS_BLOCK)
    with np.errstate(invalid="ignore"):
        M = np.max(np.abs(yb), axis=2)
    m = mbs_mantissa(M)
    c = (1.0 + m.astype(np.float32) / np.float32(256)).astype(np.float32)
    yp = (yb * c[:, :, None]).astype(np.float32).reshape(r, kb)
    nib, sc = _quantize_rows(yp, mode)
    return nib, sc, m


def dequantize_mbs(nib: np.ndarray, sc: np.ndarray, mbs: np.ndarray) -> np.ndarray:
    """fp64 values Q(c y) / c of an MBS operand."""
    c = 1.0 + np.asarray(mbs, dtype=np.float64) / 256.0
    return dequantize(nib, sc) / np.repeat(c, MBS_BLOCK, axis=1)


# --------------------------------------------------------------------------
# Reconstruction ([P1] quick-read block: x_rec = 2^E * Q_FP4(x / 2^E))
# --------------------------------------------------------------------------
def dequantize(nib: np.ndarray, sc: np.ndarray, two_d: bool = False) -> np.ndarray:
    """fp64 values of a packed operand [R][C] (nibbles [R][C/2]).

    deq = (-1)^(code >> 3) * G[code & 7] * 2^(sc - 127); sc = 0xFF is NaN.
    ``sc`` is [R][C/32], or [R/32][C/32] when ``two_d``.
    """
    nib = np.asarray(nib, dtype=np.uint8)
    r = nib.shape[0]
    c = nib.shape[1] * 2
    codes = np.empty((r, c), dtype=np.uint8)
    codes[:, 0::2] = nib & 0xF
    codes[:, 1::2] = nib >> 4
    mag = E2M1_GRID[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    sc = np.asarray(sc, dtype=np.uint8)
    if two_d:
        sc_full = np.repeat(np.repeat(sc, BLOCK, axis=0), BLOCK, axis=1)
    else:
        sc_full = np.repeat(sc, BLOCK, axis=1)
    out = np.ldexp(val, sc_full.astype(np.int64) - 127)
    return np.where(sc_full == 255, np.nan, out)


# --------------------------------------------------------------------------
# GEMM on dequantized operands ([P1] A.2 / section B: MXFP4 GEMM per
# product; [P3]: native MXFP4 accumulates in FP32 -- the oracle sums in fp64)
# --------------------------------------------------------------------------
def gemm_ref(a_deq: np.ndarray, b_deq: np.ndarray):
    """C = A B^T and S = |A| |B|^T in fp64 (A [M][K], B [N][K])."""
    a = np.asarray(a_deq, dtype=np.float64)
    b = np.asarray(b_deq, dtype=np.float64)
    return a @ b.T, np.abs(a) @ np.abs(b).T


def gemm_tolerance(S: np.ndarray, c_ref: np.ndarray, out_bf16: bool) -> np.ndarray:
    """Per-element bound: 1e-5 * S (fp32 out); + 2^-8 |C_ref| for bf16 out."""
    tol = 1e-5 * S
    if out_bf16:
        tol = tol + np.abs(c_ref) * 2.0 ** -8
    return tol


# --------------------------------------------------------------------------
# The three linear-layer products ([P1] C.1, C.2, C.3) as quantized operands
# --------------------------------------------------------------------------
def product_operands(op: str, P: np.ndarray, Q: np.ndarray, hadamard: int, mode: int):
    """Quantized GEMM operands (A, B) for one product, each as (nib, sc).

    fprop: Y[T,N]  = X[T,K] W[N,K]^T   A = q_row(X),  B = q_row(W)     (P=X, Q=W)
    dgrad: dX[T,K] = dY[T,N] W[N,K]    A = q_row(dY), B = q_col(W)     (P=dY, Q=W)
    wgrad: dW[N,K] = dY[T,N]^T X[T,K]  A = q_col(dY), B = q_col(X)     (P=dY, Q=X)
    The rotation runs along each product's reduction axis (K, N and T).
    """
    if op == "fprop":
        return (quantize_chunked(P, AXIS_ROW, hadamard, mode),
                quantize_chunked(Q, AXIS_ROW, hadamard, mode))
    if op == "dgrad":
        return (quantize_chunked(P, AXIS_ROW, hadamard, mode),
                quantize_chunked(Q, AXIS_COL, hadamard, mode))
    if op == "wgrad":
        return (quantize_chunked(P, AXIS_COL, hadamard, mode),
                quantize_chunked(Q, AXIS_COL, hadamard, mode))
    raise ValueError(op)


def unquantized_product(op: str, P: np.ndarray, Q: np.ndarray) -> np.ndarray:
    """fp64 product of the original bf16 operands (no rotation, no quantization)."""
    p = bf16_to_f32(P).astype(np.float64)
    q = bf16_to_f32(Q).astype(np.float64)
    if op == "fprop":
        return p @ q.T
    if op == "dgrad":
        return p @ q
    if op == "wgrad":
        return p.T @ q
    raise ValueError(op)


def rotated_unquantized_product(op: str, P: np.ndarray, Q: np.ndarray, hadamard: int):
    """fp64 GEMM of the rotated fp32 operands, skipping quantization.

    Used for the cancellation check: with H H^T = I the result equals the
    unrotated product up to the fp32 rounding of the rotation.
    """
    p = bf16_to_f32(P)
    q = bf16_to_f32(Q)
    if op == "fprop":
        a, b = hadamard_rotate(p, hadamard), hadamard_rotate(q, hadamard)
    elif op == "dgrad":
        a, b = hadamard_rotate(p, hadamard), hadamard_rotate(np.ascontiguousarray(q.T), hadamard)
    elif op == "wgrad":
        a = hadamard_rotate(np.ascontiguousarray(p.T), hadamard)
        b = hadamard_rotate(np.ascontiguousarray(q.T), hadamard)
    else:
        raise ValueError(op)
    return a.astype(np.float64) @ b.astype(np.float64).T


# --------------------------------------------------------------------------
# Ideal-scale quantizer and the three-way error decomposition ([P3] core
# insight and Property 1)
# --------------------------------------------------------------------------
def _grid_round(t: np.ndarray) -> np.ndarray:
    """Nearest E2M1 value of fp64 t (ties to the even code, clamp at 6)."""
    a = np.abs(t)
    mag = ((a > 0.25).astype(np.int64) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
           + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    return np.where(np.signbit(t), -1.0, 1.0) * E2M1_GRID[mag]


def error_decomposition(x_blocks: np.ndarray, mode: int) -> dict:
    """Decompose the MXFP4 error of fp32 blocks ``x_blocks`` [nblocks][32].

    Q(x)  = 2^E * grid(x / 2^E)            (E8M0 scale, ``mode``)
    Q*(x) = s* * grid(x / s*), s* = m_b / 6 (ideal scale, no E8M0 rounding)
    deadzone D = {i : 24 |x_i| < m_b}
    e_scale = Q - Q*, e_DZ = (Q* - x) 1_D, e_grid = (Q* - x) 1_{not D}
    so e = Q - x = e_scale + e_DZ + e_grid exactly.
    """
    x = np.asarray(x_blocks, dtype=np.float32)
    m_b = np.max(np.abs(x), axis=1)
    E = e8m0_exponent(m_b, mode)
    x64 = x.astype(np.float64)
    codes = e2m1_code(x, E[:, None])
    mag = E2M1_GRID[codes & 7]
    Q = np.ldexp(np.where(codes & 8, -mag, mag), E[:, None])
    s_star = m_b.astype(np.float64)[:, None] / 6.0
    with np.errstate(invalid="ignore", divide="ignore"):
        t = np.where(s_star > 0, x64 / s_star, 0.0)
    Qs = s_star * _grid_round(t)
    dz = 24.0 * np.abs(x64) < m_b.astype(np.float64)[:, None]
    e_scale = Q - Qs
    e_dz = np.where(dz, Qs - x64, 0.0)
    e_grid = np.where(dz, 0.0, Qs - x64)
    return {"Q": Q, "Q_star": Qs, "e": Q - x64, "e_scale": e_scale, "e_dz": e_dz,
            "e_grid": e_grid, "deadzone": dz, "E": E, "m_b": m_b}


STAT_FIELDS = ("sum_e_scale2", "sum_e_dz2", "sum_e_grid2", "dot_scale_grid", "dot_scale_dz",
               "sum_e2", "sum_x2", "n_deadzone", "n_elements", "n_nonfinite_blocks")


def error_stats(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int) -> dict:
    """Tensor-level sums of the three-way decomposition of the MXFP4 error of
    the values ``quantize`` encodes (the rotated operand), over its 1x32
    (row) or 32x1 (col) blocks ([P3] core insight and Property 1; the
    deadzone share is the statistic [P3] reports for weights):
    sum e_scale^2, sum e_DZ^2, sum e_grid^2, sum e_scale e_grid,
    sum e_scale e_DZ, sum e^2, sum x^2, deadzone count, element count.
    Blocks holding a non-finite rotated value are left out and counted.
    """
    x = bf16_to_f32(src_bf16)
    if axis == AXIS_COL:
        x = np.ascontiguousarray(x.T)
    elif axis != AXIS_ROW:
        raise ValueError("error statistics are defined for 1x32 and 32x1 blocks")
    y = hadamard_rotate(x, hadamard).reshape(-1, BLOCK)
    finite = np.all(np.isfinite(y), axis=1)
    d = error_decomposition(y[finite], mode)
    es, edz, eg, e = d["e_scale"], d["e_dz"], d["e_grid"], d["e"]
    x64 = y[finite].astype(np.float64)
    vals = (np.sum(es * es), np.sum(edz * edz), np.sum(eg * eg), np.sum(es * eg),
            np.sum(es * edz), np.sum(e * e), np.sum(x64 * x64), np.count_nonzero(d["deadzone"]),
            x64.size, np.count_nonzero(~finite))
    return {k: float(v) for k, v in zip(STAT_FIELDS, vals)}


def error_stats_chunked(src_bf16: np.ndarray, axis: int, hadamard: int, mode: int,
                        chunk: int = 512) -> dict:
    """``error_stats`` summed over slabs (rows for row blocks, columns for
    column blocks) to bound memory; blocks never straddle slabs."""
    r, c = src_bf16.shape
    if axis == AXIS_COL:
        parts = [error_stats(src_bf16[:, j:j + chunk], axis, hadamard, mode)
                 for j in range(0, c, chunk)]
    else:
        parts = [error_stats(src_bf16[i:i + chunk], axis, hadamard, mode)
                 for i in range(0, r, chunk)]
    return {k: float(sum(p[k] for p in parts)) for k in STAT_FIELDS}


def error_report(C: np.ndarray, P: np.ndarray) -> dict:
    """MSE, cosine, relative Frobenius error and SNR (dB) of C against P."""
    C = np.asarray(C, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    d = C - P
    nd = float(np.sum(d * d))
    npp = float(np.sum(P * P))
    nc = float(np.sum(C * C))
    return {
        "mse": nd / d.size,
        "cosine": float(np.sum(C * P)) / np.sqrt(nc * npp) if nc > 0 and npp > 0 else float("nan"),
        "rel_fro": np.sqrt(nd / npp) if npp > 0 else float("nan"),
        "snr_db": 10.0 * np.log10(npp / nd) if nd > 0 else float("inf"),
    }
