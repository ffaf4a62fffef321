"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here is independent of the oracle's own formulas: closed forms
(Sylvester/Kronecker Hadamard, exact rational rounding with ``fractions``),
brute force on tiny inputs, invariants the pages state, and constants the
pages print (``tests/golden``). A plausible slip in the oracle -- a dropped
butterfly stage, a wrong sign, a swapped nibble, a mis-rounded tie, a wrong
scale rule, a transposed operand -- fails at least one of them.

Pages: [P1] "Pretraining Large Language Models with MXFP4 on Native FP4
Hardware" (arXiv:2605.09825 summary); [P2] FP4 training article on
arXiv:2501.17116; [P3] "Decomposing MXFP4 quantization error" blog
(arXiv:2605.20402).
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle as O
import synthetic

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


def sylvester(h):
    """Natural-order Sylvester matrix by Kronecker powers of [[1,1],[1,-1]]."""
    H = np.array([[1.0]])
    while H.shape[0] < h:
        H = np.kron(np.array([[1.0, 1.0], [1.0, -1.0]]), H)
    return H


def all_bf16_f32(finite_only=True):
    bits = np.arange(65536, dtype=np.uint32)
    v = np.left_shift(bits, np.uint32(16)).view(np.float32)
    return v[np.isfinite(v)] if finite_only else v


# ---------------------------------------------------------------- (a) H H^T = I
def test_h16_rows_are_sylvester_and_orthonormal_bit_exact():
    """[P1] quick-read block and section C: H H^T = I, H a +-1 (scaled) matrix."""
    H = O.hadamard_rotate(np.eye(16, dtype=np.float32), 16)
    assert H.dtype == np.float32
    assert np.array_equal(H.astype(np.float64), sylvester(16) / 4.0)
    # products are +-1/16 and 16-term sums are exact: bit-exact identity
    HHt = np.zeros((16, 16), dtype=np.float32)
    for i in range(16):
        for j in range(16):
            acc = np.float32(0)
            for k in range(16):
                acc = np.float32(acc + H[i, k] * H[j, k])
            HHt[i, j] = acc
    assert np.array_equal(HHt, np.eye(16, dtype=np.float32))


def test_h32_orthonormal_to_rounding_only():
    """H32's 1/sqrt(32) is irrational: H H^T = I holds to ~1e-7, not exactly."""
    H = O.hadamard_rotate(np.eye(32, dtype=np.float32), 32).astype(np.float64)
    c = float(np.float32(2.0 ** -2.5))
    assert np.array_equal(H, sylvester(32) * c)
    err = np.abs(H @ H.T - np.eye(32)).max()
    assert 0 < err < 1e-6


def test_butterfly_exact_on_small_integers():
    """Small integers keep every fp32 add exact, so the butterfly equals x H."""
    rng = np.random.default_rng(11)
    x = rng.integers(-1024, 1025, size=(64, 128)).astype(np.float32)
    for h in (16, 32):
        y = O.hadamard_rotate(x, h).astype(np.float64)
        H = sylvester(h) * (0.25 if h == 16 else float(np.float32(2.0 ** -2.5)))
        ref = (x.astype(np.float64).reshape(64, 128 // h, h) @ H).reshape(64, 128)
        if h == 16:
            assert np.array_equal(y, ref)
        else:  # one extra fp32 rounding in the final multiply
            assert np.allclose(y, ref, rtol=2 ** -23, atol=0)


def test_rotation_is_blockwise_and_aligned():
    """Tiled layout ([P1] A.2): groups of h aligned at 0, no mixing across groups."""
    x = np.zeros((1, 64), dtype=np.float32)
    x[0, 17] = 1.0
    y = O.hadamard_rotate(x, 16)
    assert np.count_nonzero(y[0, :16]) == 0 and np.count_nonzero(y[0, 32:]) == 0
    assert np.array_equal(y[0, 16:32].astype(np.float64), sylvester(16)[1] / 4.0)
    assert np.array_equal(O.hadamard_rotate(x, 0), x)


# ------------------------------------------------------------ (b) cancellation
@pytest.mark.parametrize("op", ["fprop", "dgrad", "wgrad"])
@pytest.mark.parametrize("h", [16, 32])
def test_cancellation_identities(op, h):
    """[P1] C.1-C.3: rotating both operands along the reduction axis leaves
    the product unchanged (H H^T = I)."""
    rng = np.random.default_rng(5)
    T, N, K = 256, 96, 128
    if op == "fprop":
        P = synthetic.f64_to_bf16_bits(rng.normal(size=(T, K)))
        Q = synthetic.f64_to_bf16_bits(rng.normal(size=(N, K)))
    elif op == "dgrad":
        P = synthetic.f64_to_bf16_bits(rng.normal(size=(T, N)))
        Q = synthetic.f64_to_bf16_bits(rng.normal(size=(N, K)))
    else:
        P = synthetic.f64_to_bf16_bits(rng.normal(size=(T, N)))
        Q = synthetic.f64_to_bf16_bits(rng.normal(size=(T, K)))
    ref = O.unquantized_product(op, P, Q)
    rot = O.rotated_unquantized_product(op, P, Q, h)
    rel = np.linalg.norm(rot - ref) / np.linalg.norm(ref)
    assert rel <= 1e-5
    # and the rotation really changed the operands (not a no-op)
    if op == "fprop":
        assert not np.array_equal(O.hadamard_rotate(O.bf16_to_f32(P), h), O.bf16_to_f32(P))


def test_cancellation_tiny_workload():
    w = synthetic.make("tiny")
    ref = O.unquantized_product("fprop", w["X"], w["W"])
    rot = O.rotated_unquantized_product("fprop", w["X"], w["W"], 16)
    assert np.linalg.norm(rot - ref) / np.linalg.norm(ref) <= 1e-5


# --------------------------------------------------- (c) grid and saturation
def test_grid_matches_pages():
    """All 16 codes at scale byte 127 dequantize to the printed grid."""
    table = {int(c): float(v) for c, v in _golden_table("e2m1_grid.txt")}
    assert sorted(table) == list(range(8))
    nib = np.array([[c | (c + 1) << 4 for c in range(0, 16, 2)] * 2], dtype=np.uint8)
    vals = O.dequantize(nib, np.array([[127]], dtype=np.uint8))[0, :16]
    for code in range(16):
        want = table[code & 7] * (-1.0 if code & 8 else 1.0)
        assert vals[code] == want
        assert math.copysign(1.0, vals[code]) == (-1.0 if code & 8 else 1.0)
    assert max(table.values()) == 6.0  # range +-6 ([P2] section 1)


def test_saturation_at_six():
    for v in (6.0, 6.5, 7.99, 1e30, np.inf):
        assert O.e2m1_code(np.array([v], np.float32), np.array([0]))[0] == 7
        assert O.e2m1_code(np.array([-v], np.float32), np.array([0]))[0] == 15


_GRID_Q = [Fraction(g) for g in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]


def _nearest_code_exact(v: Fraction) -> int:
    """Nearest grid value by exact distance; ties to the even code; clamp at 6."""
    a = abs(v)
    if a >= 6:
        return 7
    return min(range(8), key=lambda c: (abs(a - _GRID_Q[c]), c & 1))


def test_e2m1_exhaustive_against_exact_rounding():
    """Every finite bf16 value, at several shared exponents, against an
    independent exact-arithmetic nearest-value rule."""
    v = all_bf16_f32()
    for E in (0, -3, 2, 5):
        codes = O.e2m1_code(v, np.full(v.shape, E))
        for x, c in zip(v.tolist(), codes.tolist()):
            want = _nearest_code_exact(Fraction(x) / Fraction(2) ** E)
            if math.copysign(1.0, x) < 0:
                want |= 8
            assert c == want, (x, E, c, want)


def test_e2m1_tie_cases_round_to_even_code():
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for t, code in ties.items():
        assert O.e2m1_code(np.array([t], np.float32), np.array([0]))[0] == code
        assert O.e2m1_code(np.array([-t], np.float32), np.array([0]))[0] == code | 8


# --------------------------------------------------------- E8M0 scale rules
def _e_floor_exact(mb: Fraction) -> int:
    """Largest E with 4 * 2^E <= m_b (max exponent minus emax = 2)."""
    E = 200
    while Fraction(4) * Fraction(2) ** E > mb:
        E -= 1
    return E


def _e_ceil_exact(mb: Fraction) -> int:
    """Smallest E with 6 * 2^E >= m_b ([P3]: ceiling of s* = m_b / 6)."""
    E = -300
    while Fraction(6) * Fraction(2) ** E < mb:
        E += 1
    return E


def test_e8m0_exhaustive_over_bf16_amax():
    v = all_bf16_f32()
    v = v[v > 0]
    Ef = O.e8m0_exponent(v, O.MODE_OCP_FLOOR)
    Ec = O.e8m0_exponent(v, O.MODE_CEIL)
    # coarse bisection keeps the exact search fast
    for x, ef, ec in zip(v.tolist(), Ef.tolist(), Ec.tolist()):
        mb = Fraction(x)
        wf = max(-127, min(127, _e_floor_exact_fast(mb)))
        wc = max(-127, min(127, _e_ceil_exact_fast(mb)))
        assert ef == wf, (x, ef, wf)
        assert ec == wc, (x, ec, wc)


def _e_floor_exact_fast(mb):
    E = mb.numerator.bit_length() - mb.denominator.bit_length() - 2 + 2
    while Fraction(4) * Fraction(2) ** E > mb:
        E -= 1
    while Fraction(4) * Fraction(2) ** (E + 1) <= mb:
        E += 1
    return E


def _e_ceil_exact_fast(mb):
    E = mb.numerator.bit_length() - mb.denominator.bit_length() - 4
    while Fraction(6) * Fraction(2) ** E < mb:
        E += 1
    while Fraction(6) * Fraction(2) ** (E - 1) >= mb:
        E -= 1
    return E


def test_e8m0_search_helpers_agree_with_plain_search():
    for x in (1.0, 1.5, 1.50390625, 6.0, 7.0, 2.0 ** -130, 3.0e38, 0.1):
        mb = Fraction(x)
        assert _e_floor_exact_fast(mb) == _e_floor_exact(mb)
        assert _e_ceil_exact_fast(mb) == _e_ceil_exact(mb)


def test_scale_bracket():
    """ceil: 1 <= 2^E / (m_b / 6) < 2 ([P3] scale-bias section, gamma = 2^delta);
    floor: 4 * 2^E <= m_b < 8 * 2^E (block max lands in [4, 8) after scaling).
    Over every positive finite bf16 m_b above the E clamp."""
    v = all_bf16_f32()
    v = v[(v > 0) & (v >= 2.0 ** -124)].astype(np.float64)
    Ec = O.e8m0_exponent(v, O.MODE_CEIL)
    gamma = np.ldexp(1.0, Ec) / (v / 6.0)
    assert np.all(gamma >= 1.0) and np.all(gamma < 2.0)
    Ef = O.e8m0_exponent(v, O.MODE_OCP_FLOOR)
    assert np.all(np.ldexp(4.0, Ef) <= v) and np.all(v < np.ldexp(8.0, Ef))
    assert O.e8m0_exponent(np.array([0.0]), O.MODE_CEIL)[0] == -127
    assert O.e8m0_exponent(np.array([0.0]), O.MODE_OCP_FLOOR)[0] == -127


def test_mean_gamma_is_one_over_ln2():
    """[P3] scale-bias section: gamma = 2^delta, delta ~ U[0, 1), about 44%
    average overshoot; E[2^delta] = 1/ln 2."""
    consts = dict(_golden_table("format_constants.txt"))
    rng = np.random.default_rng(7)
    m_b = np.exp2(rng.uniform(0, 20, size=400_000)).astype(np.float32)
    E = O.e8m0_exponent(m_b, O.MODE_CEIL)
    gamma = np.ldexp(1.0, E) / (m_b.astype(np.float64) / 6.0)
    assert abs(gamma.mean() - 1 / math.log(2)) < 4e-3
    assert round(100 * (gamma.mean() - 1)) == int(consts["gamma_mean_excess_percent"])


# ------------------------------------------------- whole-block scalar encoder
def _encode_block_exact(y32, mode):
    """Independent scalar encoder of one 32-element fp32 block with exact
    rationals: returns (scale byte, list of codes)."""
    vals = [Fraction(float(t)) for t in y32]
    mb = max(abs(t) for t in vals)
    if mb == 0:
        E = -127
    else:
        E = _e_floor_exact_fast(mb) if mode == O.MODE_OCP_FLOOR else _e_ceil_exact_fast(mb)
        E = max(-127, min(127, E))
    codes = []
    for t, f in zip(vals, y32):
        c = _nearest_code_exact(t / Fraction(2) ** E)
        if math.copysign(1.0, float(f)) < 0:
            c |= 8
        codes.append(c)
    return E + 127, codes


def _reference_quantize_scalar(src_bits, axis, h, mode):
    """Loops over blocks with the scalar encoder, rotating with the explicit
    Sylvester matrix product (fp64 exact on these inputs, then fp32)."""
    x = synthetic.bf16_bits_to_f32(src_bits).astype(np.float64)
    if axis == O.AXIS_COL:
        x = x.T
    R, C = x.shape
    if h:
        H = sylvester(h) * (0.25 if h == 16 else float(np.float32(2.0 ** -2.5)))
        x = (x.reshape(R, C // h, h) @ H).reshape(R, C)
    y = x.astype(np.float32)
    codes = np.zeros((R, C), dtype=np.uint8)
    if axis == O.AXIS_2D:
        sc = np.zeros((R // 32, C // 32), dtype=np.uint8)
        for bi in range(R // 32):
            for bj in range(C // 32):
                tile = y[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32].ravel()
                s, cs = _encode_block_exact(tile, mode)
                sc[bi, bj] = s
                codes[bi * 32:(bi + 1) * 32, bj * 32:(bj + 1) * 32] = np.array(cs).reshape(32, 32)
    else:
        sc = np.zeros((R, C // 32), dtype=np.uint8)
        for i in range(R):
            for b in range(C // 32):
                s, cs = _encode_block_exact(y[i, b * 32:(b + 1) * 32], mode)
                sc[i, b] = s
                codes[i, b * 32:(b + 1) * 32] = cs
    nib = np.zeros((R, C // 2), dtype=np.uint8)
    for j in range(C // 2):
        nib[:, j] = codes[:, 2 * j] | (codes[:, 2 * j + 1] << 4)
    return nib, sc


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL, O.AXIS_2D])
@pytest.mark.parametrize("mode", [O.MODE_OCP_FLOOR, O.MODE_CEIL])
@pytest.mark.parametrize("h", [0, 16])
def test_oracle_matches_scalar_exact_encoder(axis, mode, h):
    """Small integer-valued inputs make the fp64 matrix rotation exact, so the
    scalar encoder sees the same fp32 values as the butterfly."""
    rng = np.random.default_rng(100 + axis * 10 + mode * 3 + h)
    base = rng.integers(-64, 65, size=(64, 96)).astype(np.float64)
    base *= np.exp2(rng.integers(-3, 4, size=(1, 96)))
    src = synthetic.f64_to_bf16_bits(base)
    nib, sc = O.quantize(src, axis, h, mode)
    rnib, rsc = _reference_quantize_scalar(src, axis, h, mode)
    assert np.array_equal(sc, rsc)
    assert np.array_equal(nib, rnib)


def test_oracle_matches_scalar_encoder_heavy_tails():
    """Student-t data (the quantizer workload's distribution), no rotation,
    both modes, row axis."""
    a = synthetic.make("quant", scale=512)["A"][:, :256]
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        nib, sc = O.quantize(a, O.AXIS_ROW, 0, mode)
        rnib, rsc = _reference_quantize_scalar(a, O.AXIS_ROW, 0, mode)
        assert np.array_equal(sc, rsc) and np.array_equal(nib, rnib)


def test_reconstruction_error_bound_and_positions():
    """x_rec = 2^E Q(x / 2^E) ([P1] A.1): every element's reconstruction is
    within half a grid gap of its input (gaps 0.5, 1, 2 on [0,2], [2,4],
    [4,6]; saturated values lose |v| - 6); a swapped nibble or a misplaced
    scale breaks this on random data."""
    rng = np.random.default_rng(3)
    src = synthetic.f64_to_bf16_bits(rng.standard_t(3, size=(64, 256)))
    for axis in (O.AXIS_ROW, O.AXIS_COL, O.AXIS_2D):
        for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
            nib, sc = O.quantize(src, axis, 16, mode)
            deq = O.dequantize(nib, sc, two_d=(axis == O.AXIS_2D))
            x = O.bf16_to_f32(src)
            y = O.hadamard_rotate(x.T if axis == O.AXIS_COL else x, 16).astype(np.float64)
            if axis == O.AXIS_2D:
                scale = np.repeat(np.repeat(np.ldexp(1.0, sc.astype(int) - 127), 32, 0), 32, 1)
            else:
                scale = np.repeat(np.ldexp(1.0, sc.astype(int) - 127), 32, 1)
            assert deq.shape == y.shape
            err = np.abs(deq - y)
            a = np.abs(y) / scale
            half_gap = np.select([a <= 2, a <= 4, a <= 6], [0.25, 0.5, 1.0], a - 6)
            assert np.all(err <= half_gap * scale)


# ------------------------------------------------------------- (d) deadzone
def test_deadzone_rule():
    """[P3] core insight: |x| < m_b / 24 is the deadzone. Ideal scale: such
    x quantize to 0 under Q*; with the ceiling scale (s_b >= s*) also under Q.
    With either mode, a scaled magnitude <= 1/4 is exactly code 0."""
    consts = dict(_golden_table("format_constants.txt"))
    div = int(consts["deadzone_divisor"])
    assert div == 4 * int(consts["q_max"])  # m_b/24 = s* * (q_min / 2), q_min = 0.5
    a = synthetic.make("quant", scale=64)["A"]
    x = O.hadamard_rotate(O.bf16_to_f32(a), 16)
    blocks = x.reshape(-1, 32)
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        d = O.error_decomposition(blocks, mode)
        dz = div * np.abs(blocks.astype(np.float64)) < d["m_b"].astype(np.float64)[:, None]
        assert np.array_equal(dz, d["deadzone"])
        assert np.all(d["Q_star"][dz] == 0)
        if mode == O.MODE_CEIL:
            assert np.all(d["Q"][dz] == 0)
        codes = O.e2m1_code(blocks, d["E"][:, None])
        v = np.abs(np.ldexp(blocks.astype(np.float64), -d["E"][:, None]))
        assert np.array_equal((codes & 7) == 0, v <= 0.25)


# ------------------------------------------------------- (e) orthogonality
def _pair_blocks():
    v = all_bf16_f32()
    v = v[(v >= 2.0 ** -4) & (v <= 2.0 ** 4)]
    a = np.repeat(v, v.size)
    x = np.tile(v, v.size)
    blocks = np.zeros((a.size, 32), dtype=np.float32)
    blocks[:, 0] = a
    blocks[:, 1] = x
    return blocks


def test_orthogonality_bruteforce_pairs():
    """[P3] Property 1: <e_DZ, e_scale> = <e_DZ, e_grid> = 0, pointwise, under
    the ceiling scale. Every block {a, x, 0 x 30} with a, x over all bf16
    values in [2^-4, 2^4] (covers every deadzone edge)."""
    blocks = _pair_blocks()
    assert blocks.shape[0] > 1_000_000
    d = O.error_decomposition(blocks, O.MODE_CEIL)
    assert np.all(d["e_dz"] * d["e_scale"] == 0.0)
    assert np.all(d["e_dz"] * d["e_grid"] == 0.0)
    assert np.sum(d["e_dz"] * d["e_scale"]) == 0.0
    assert np.sum(d["e_dz"] * d["e_grid"]) == 0.0
    assert np.array_equal(d["e"], d["e_scale"] + d["e_dz"] + d["e_grid"]) or \
        np.allclose(d["e"], d["e_scale"] + d["e_dz"] + d["e_grid"], rtol=0, atol=1e-12)
    # deadzone edges are really exercised
    assert d["deadzone"][:, 1].any() and (~d["deadzone"][:, 1]).any()


def test_orthogonality_random_blocks_and_mse_identity():
    rng = np.random.default_rng(9)
    a = rng.standard_t(3, size=(100_000, 32)) * rng.lognormal(0, 1, size=(100_000, 1))
    blocks = O.bf16_to_f32(synthetic.f64_to_bf16_bits(a))
    d = O.error_decomposition(blocks, O.MODE_CEIL)
    assert np.sum(d["e_dz"] * d["e_scale"]) == 0.0
    assert np.sum(d["e_dz"] * d["e_grid"]) == 0.0
    es, ez, eg, e = d["e_scale"], d["e_dz"], d["e_grid"], d["e"]
    lhs = np.sum(e * e)
    rhs = np.sum(es * es) + np.sum(ez * ez) + np.sum(eg * eg) + 2 * np.sum(es * eg)
    assert abs(lhs - rhs) <= 1e-12 * lhs
    # cross term is anti-correlated under the ceiling scale ([P3] Property 1)
    cos = np.sum(es * eg) / np.sqrt(np.sum(es * es) * np.sum(eg * eg))
    assert cos < 0


def test_floor_mode_breaks_the_lemma_premise():
    """Under the OCP floor rule s_b can be below s* (m_b = 7: s_b = 1 < 7/6),
    so <e_DZ, e_scale> need not vanish; the disjoint-support term still does.
    Hand-worked: block {7, 0.27, 0...}: floor E = 0, 0.27 -> code 1 (0.5);
    ideal s* = 7/6, 0.27 / s* = 0.2314 < 0.25 -> 0 (deadzone: 24*0.27 < 7)."""
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, 0] = 7.0
    blk[0, 1] = np.float32(0.27)
    d = O.error_decomposition(blk, O.MODE_OCP_FLOOR)
    assert d["E"][0] == 0
    assert d["Q"][0, 0] == 6.0 and d["Q"][0, 1] == 0.5
    assert d["deadzone"][0, 1] and d["Q_star"][0, 1] == 0.0
    x1 = float(np.float32(0.27))
    assert np.sum(d["e_dz"] * d["e_scale"]) == pytest.approx(-x1 * 0.5, rel=1e-12)
    assert np.sum(d["e_dz"] * d["e_grid"]) == 0.0
    dc = O.error_decomposition(blk, O.MODE_CEIL)
    assert dc["E"][0] == 1 and dc["Q"][0, 1] == 0.0


# ----------------------------------------------- tensor-level error sums
def _stat_src(rows=256, cols=512, seed=21):
    rng = np.random.default_rng(seed)
    a = rng.standard_t(3, size=(rows, cols)) * rng.lognormal(0, 1, size=(1, cols))
    return synthetic.f64_to_bf16_bits(a)


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
@pytest.mark.parametrize("mode", [O.MODE_OCP_FLOOR, O.MODE_CEIL])
@pytest.mark.parametrize("h", [0, 16, 32])
def test_error_stats_pins(axis, mode, h):
    """error_stats against what fixes it independently: (1) sum e^2 is the
    squared error of the packed operand itself (dequantize(quantize(src))
    against the rotated source, a different code path); (2) the MSE
    identity of [P3] Property 1 with both cross terms; (3) in ceil mode
    <e_DZ, e_scale> = 0 exactly; (4) the deadzone count is bounded by the
    zero codes in ceil mode (deadzone values quantize to 0) and counts
    elements with 24|x| < m_b; (5) the element count."""
    src = _stat_src()
    st = O.error_stats(src, axis, h, mode)
    x = O.bf16_to_f32(src)
    if axis == O.AXIS_COL:
        x = np.ascontiguousarray(x.T)
    y = O.hadamard_rotate(x, h).astype(np.float64)
    nib, sc = O.quantize(src, axis, h, mode)
    deq = O.dequantize(nib, sc)
    e2 = float(np.sum((deq - y) ** 2))
    assert st["sum_e2"] == pytest.approx(e2, rel=1e-12)
    rhs = (st["sum_e_scale2"] + st["sum_e_dz2"] + st["sum_e_grid2"] + 2 * st["dot_scale_grid"]
           + 2 * st["dot_scale_dz"])
    assert st["sum_e2"] == pytest.approx(rhs, rel=1e-10)
    if mode == O.MODE_CEIL:
        assert st["dot_scale_dz"] == 0.0
        assert st["n_deadzone"] <= np.count_nonzero(deq == 0.0)
    blocks = y.reshape(-1, 32)
    mb = np.max(np.abs(blocks), axis=1, keepdims=True)
    assert st["n_deadzone"] == np.count_nonzero(24.0 * np.abs(blocks) < mb)
    assert st["n_elements"] == src.size and st["n_nonfinite_blocks"] == 0
    assert st["sum_x2"] == pytest.approx(float(np.sum(y * y)), rel=1e-12)


def test_error_stats_skips_nonfinite_blocks_and_chunks_agree():
    src = _stat_src(128, 256, 5)
    src[3, 40] = 0x7FC0   # NaN in row 3, block 1
    src[70, 5] = 0x7F80   # +Inf in row 70, block 0
    st = O.error_stats(src, O.AXIS_ROW, 16, O.MODE_CEIL)
    assert st["n_nonfinite_blocks"] == 2 and st["n_elements"] == src.size - 64
    assert np.isfinite(st["sum_e2"])
    ch = O.error_stats_chunked(src, O.AXIS_ROW, 16, O.MODE_CEIL, chunk=32)
    for k in O.STAT_FIELDS:
        assert ch[k] == pytest.approx(st[k], rel=1e-12, abs=0)
    stc = O.error_stats(src, O.AXIS_COL, 16, O.MODE_CEIL)
    chc = O.error_stats_chunked(src, O.AXIS_COL, 16, O.MODE_CEIL, chunk=64)
    assert stc["n_nonfinite_blocks"] == 2
    for k in O.STAT_FIELDS:
        assert chc[k] == pytest.approx(stc[k], rel=1e-12, abs=0)


# ------------------------------------------------------- outlier fallback
@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
@pytest.mark.parametrize("mode", [O.MODE_OCP_FLOOR, O.MODE_CEIL])
def test_of_first_half_is_the_plain_operand(axis, mode):
    src = _stat_src(128, 256, 31)
    n, s = O.quantize_of(src, axis, 16, mode)
    n1, s1 = O.quantize(src, axis, 16, mode)
    kb = n1.shape[1]
    assert n.shape == (n1.shape[0], 2 * kb) and s.shape == (s1.shape[0], 2 * s1.shape[1])
    assert np.array_equal(n[:, :kb], n1) and np.array_equal(s[:, :s1.shape[1]], s1)


def test_of_hand_worked_deadzone_rescue():
    """[P3] OF: the outlier sets the first scale and 0.1 falls in the deadzone
    (code 0); the residual {0, 0.1} quantized at half weight brings it back.
    Block {6, 0.10009765625 (bf16 of 0.1), 0, ...}, no rotation:
    ceil:  q1 = {6, 0} (E = 0); r/2 = 0.050048828125, E = -6 (6 * 2^-6 =
           0.09375 >= r/2 > 6 * 2^-7), r/2 / 2^-6 = 3.203 -> 3 -> 0.046875.
    floor: E = -7 (r/2 = 1.6 * 2^-5), 6.406 saturates to 6 -> 0.046875."""
    blk = np.zeros((1, 32), dtype=np.uint16)
    blk[0, 0] = synthetic.f64_to_bf16_bits(np.array([6.0]))[0]
    blk[0, 1] = synthetic.f64_to_bf16_bits(np.array([0.1]))[0]
    assert O.bf16_to_f32(blk)[0, 1] == np.float32(0.10009765625)
    for mode, e2 in ((O.MODE_CEIL, -6), (O.MODE_OCP_FLOOR, -7)):
        n, s = O.quantize_of(blk, O.AXIS_ROW, 0, mode)
        d = O.dequantize(n, s)
        assert s[0, 0] == 127 and s[0, 1] == 127 + e2
        assert d[0, 0] == 6.0 and d[0, 1] == 0.0
        assert d[0, 32] == 0.0 and d[0, 33] == 0.046875
        assert np.all(d[0, 34:] == 0) and np.all(d[0, 2:32] == 0)


def test_of_reduces_the_error_and_keeps_nonfinite_blocks():
    src = _stat_src(256, 512, 3)
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        n, s = O.quantize_of(src, O.AXIS_ROW, 16, mode)
        y = O.hadamard_rotate(O.bf16_to_f32(src), 16).astype(np.float64)
        d = O.dequantize(n, s)
        of = d[:, :512] + d[:, 512:]
        plain = O.dequantize(*O.quantize(src, O.AXIS_ROW, 16, mode))
        # half-weight residual: the error roughly quarters
        assert np.mean((of - y) ** 2) < 0.35 * np.mean((plain - y) ** 2)
    bad = src.copy()
    bad[5, 70] = 0x7FC0
    n, s = O.quantize_of(bad, O.AXIS_ROW, 16, O.MODE_CEIL)
    assert s[5, 2] == 255 and s[5, 16 + 2] == 255
    assert np.all(n[5, 32:48] == 0) and np.all(n[5, 256 + 32:256 + 48] == 0)


# ---------------------------------------------------- macro-block scaling
def test_mbs_mantissa_against_exact_search():
    """m = the largest j in [0, 255] with (1 + j/256) M <= 6 2^k, k the
    smallest integer with 6 2^k >= M: exact rational search over bf16-like
    and random fp32 maxima (the rule is a reading; this pins its arithmetic)."""
    rng = np.random.default_rng(12)
    Ms = np.concatenate([rng.lognormal(0, 3, 3000).astype(np.float32),
                         np.float32([6.0, 5.0, 3.0, 1.5, 0.75, 6.0 * 2.0 ** -20, 1e-30, 3e30])])
    got = O.mbs_mantissa(Ms)
    for M, m in zip(Ms, got):
        F = Fraction(float(M))
        k = -200
        while 6 * Fraction(2) ** k < F:
            k += 1
        best = max(j for j in range(256) if (1 + Fraction(j, 256)) * F <= 6 * Fraction(2) ** k)
        assert m == best, (float(M), int(m), best)
    assert list(O.mbs_mantissa(np.float32([0.0, np.inf, np.nan]))) == [0, 0, 0]


def test_mbs_hand_worked_block():
    """Macro max 5: k = 0, c = 1 + floor(256 * 0.2) / 256 = 1 + 51/256; 5 c =
    5.996 -> E = 0, code 6.0 -> 6 / c = 1536/307 (plain ceil: 5 -> 4, the tie
    rounds to the even code). bf16(0.3) = 0.30078125 -> c x = 0.3607 -> 0.5 ->
    0.5 / c. A block of max 6 needs no correction: m = 0, plain operand."""
    blk = np.zeros((1, 128), dtype=np.float64)
    blk[0, 0], blk[0, 1] = 5.0, 0.3
    src = synthetic.f64_to_bf16_bits(blk)
    n, s, m = O.quantize_mbs(src, O.AXIS_ROW, 0, O.MODE_CEIL)
    assert m[0, 0] == 51 and s[0, 0] == 127
    d = O.dequantize_mbs(n, s, m)
    c = 1 + 51 / 256
    assert d[0, 0] == 6.0 / c and d[0, 1] == 0.5 / c
    assert O.dequantize(*O.quantize(src, O.AXIS_ROW, 0, O.MODE_CEIL))[0, 0] == 4.0
    blk[0, 0] = 6.0
    src = synthetic.f64_to_bf16_bits(blk)
    n, s, m = O.quantize_mbs(src, O.AXIS_ROW, 0, O.MODE_CEIL)
    n0, s0 = O.quantize(src, O.AXIS_ROW, 0, O.MODE_CEIL)
    assert m[0, 0] == 0 and np.array_equal(n, n0) and np.array_equal(s, s0)


@pytest.mark.parametrize("mode", [O.MODE_OCP_FLOOR, O.MODE_CEIL])
def test_mbs_removes_the_scale_bias_of_the_macro_max_block(mode):
    """After the prescale the macro maximum's block has gamma = 2^E / s* in
    [1, 1 + 2^-7) (E8M0 over the ideal scale of the prescaled block), in both
    rules; without MBS gamma spreads over [1, 2). The operand is also
    dequantized through a different path (dequantize / c)."""
    src = _stat_src(256, 1024, 8)
    n, s, m = O.quantize_mbs(src, O.AXIS_ROW, 16, mode)
    y = O.hadamard_rotate(O.bf16_to_f32(src), 16)
    yb = y.reshape(256, 8, 128)
    c = (1 + m.astype(np.float64) / 256)
    M = np.max(np.abs(yb), axis=2).astype(np.float64)
    blk = np.argmax(np.abs(yb), axis=2) // 32
    E = s.reshape(256, 8, 4)[np.arange(256)[:, None], np.arange(8)[None, :], blk].astype(np.int64) - 127
    cM = (yb.astype(np.float32) * c[:, :, None].astype(np.float32)).astype(np.float32)
    cM = np.max(np.abs(cM), axis=2).astype(np.float64)
    gamma = np.ldexp(1.0, E) / (cM / 6)
    assert np.all(gamma >= 1.0) and np.all(gamma < 1 + 2 ** -7)
    g0 = np.ldexp(1.0, O.e8m0_exponent(M.astype(np.float32), O.MODE_CEIL)) / (M / 6)
    assert g0.max() > 1.5
    d = O.dequantize_mbs(n, s, m)
    assert np.allclose(d * np.repeat(c, 128, axis=1), O.dequantize(n, s), rtol=1e-15, atol=0)


# ------------------------------------------------------- hand-worked blocks
def test_hand_worked_blocks():
    """Blocks whose encodings follow from the definitions by hand."""
    # max 7 = 1.75 * 2^2: floor E = 0 (7 -> 6 saturates); ceil needs
    # 6 * 2^E >= 7 -> E = 1 (7/2 = 3.5 is a tie -> 4, code 6).
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, :4] = [7.0, -1.0, 0.25, 3.0]
    src = synthetic.f64_to_bf16_bits(blk)
    nib, sc = O.quantize(src, O.AXIS_ROW, 0, O.MODE_OCP_FLOOR)
    assert sc[0, 0] == 127
    assert nib[0, 0] == (7 | (8 | 2) << 4) and nib[0, 1] == (0 | 5 << 4)
    nib, sc = O.quantize(src, O.AXIS_ROW, 0, O.MODE_CEIL)
    assert sc[0, 0] == 128
    # 7/2 = 3.5 -> 4 (code 6); -1/2 -> -0.5 (code 9); 0.125 -> 0; 1.5 -> code 3
    assert nib[0, 0] == (6 | 9 << 4) and nib[0, 1] == (0 | 3 << 4)
    # all-zero block (with a negative zero): scale byte 0, codes keep the sign
    z = np.zeros((1, 32), dtype=np.uint16)
    z[0, 1] = 0x8000
    nib, sc = O.quantize(z, O.AXIS_ROW, 0, O.MODE_CEIL)
    assert sc[0, 0] == 0 and nib[0, 0] == 0x80 and np.all(nib[0, 1:] == 0)
    # a non-finite value poisons its block: scale 0xFF, zero nibbles
    z[0, 5] = 0x7F80
    nib, sc = O.quantize(z, O.AXIS_ROW, 0, O.MODE_CEIL)
    assert sc[0, 0] == 255 and np.all(nib == 0)
    # H16 of a constant group: all energy moves to element 0 of the group
    c = np.full((1, 32), 2.0)
    y = O.hadamard_rotate(c.astype(np.float32), 16)
    assert y[0, 0] == 8.0 and y[0, 16] == 8.0 and np.count_nonzero(y) == 2


# -------------------------------------------------------------- GEMM oracle
def test_gemm_ref_against_exact_sum():
    """fp64 product of dequantized operands vs exact rational sums."""
    rng = np.random.default_rng(21)
    A = synthetic.f64_to_bf16_bits(rng.normal(size=(5, 64)))
    B = synthetic.f64_to_bf16_bits(rng.normal(size=(3, 64)) * 30)
    qa = O.quantize(A, O.AXIS_ROW, 16, O.MODE_OCP_FLOOR)
    qb = O.quantize(B, O.AXIS_ROW, 16, O.MODE_OCP_FLOOR)
    da, db = O.dequantize(*qa), O.dequantize(*qb)
    C, S = O.gemm_ref(da, db)
    for i in range(5):
        for j in range(3):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(da[i], db[j]))
            sabs = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(da[i], db[j]))
            assert abs(Fraction(C[i, j]) - exact) <= Fraction(64) * Fraction(2) ** -52 * sabs
            assert abs(Fraction(S[i, j]) - sabs) <= Fraction(64) * Fraction(2) ** -52 * sabs
    # orientation: C[i, j] pairs A's row i with B's row j
    assert C.shape == (5, 3)


def test_product_operand_orientation():
    """dgrad quantizes W column-wise (so B is W^T, [K][N]); wgrad quantizes
    both operands column-wise (A = dY^T, B = X^T). Dequantized products of
    unrotated small-integer operands reproduce the plain products exactly
    when every block is exactly representable."""
    rng = np.random.default_rng(4)
    T, N, K = 64, 32, 96
    # values in {0, +-1, +-2, +-4} * 2^k fit the E2M1 grid after scaling
    def grid_ints(shape):
        return rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0], size=shape)
    P_f = grid_ints((T, N))
    Q_f = grid_ints((N, K))
    X_f = grid_ints((T, K))
    for op, P, Q, want in (
        ("dgrad", P_f, Q_f, P_f @ Q_f),
        ("wgrad", P_f, X_f, P_f.T @ X_f),
        ("fprop", X_f, grid_ints((N, K)), None),
    ):
        Pb, Qb = synthetic.f64_to_bf16_bits(P), synthetic.f64_to_bf16_bits(Q)
        (an, asc), (bn, bsc) = O.product_operands(op, Pb, Qb, 0, O.MODE_CEIL)
        C, _ = O.gemm_ref(O.dequantize(an, asc), O.dequantize(bn, bsc))
        if want is None:
            want = P @ Q.T
        assert np.array_equal(C, want), op


# ------------------------------------------- comparison arms: random signs, SR
def _codes_of(nib):
    """Unpack [R][C/2] nibble bytes to [R][C] codes."""
    c = np.empty((nib.shape[0], nib.shape[1] * 2), np.uint8)
    c[:, 0::2] = nib & 0xF
    c[:, 1::2] = nib >> 4
    return c


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
@pytest.mark.parametrize("h", [0, 16, 32])
def test_random_signs_zero_and_all_flipped(axis, h):
    """No flips is the plain operand; flipping every sign negates every
    rotated value (the butterfly and the nearest-value rule are odd
    functions), so only the nibbles' sign bits change."""
    x = synthetic.f64_to_bf16_bits(np.random.default_rng(5).standard_t(3, size=(64, 96)))
    n = x.shape[1] if axis == O.AXIS_ROW else x.shape[0]
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        nib, sc = O.quantize(x, axis, h, mode)
        z = O.quantize_rs(x, axis, h, mode, np.zeros(n, np.uint8))
        f = O.quantize_rs(x, axis, h, mode, np.ones(n, np.uint8))
        assert np.array_equal(z[0], nib) and np.array_equal(z[1], sc)
        assert np.array_equal(f[0], nib ^ 0x88) and np.array_equal(f[1], sc)


def test_random_signs_column_rule_is_row_rule_of_transpose():
    x = synthetic.f64_to_bf16_bits(np.random.default_rng(6).standard_normal((96, 64)))
    s = synthetic.random_signs(96, 7)
    a = O.quantize_rs(x, O.AXIS_COL, 16, 1, s)
    b = O.quantize_rs(np.ascontiguousarray(x.T), O.AXIS_ROW, 16, 1, s)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_random_signs_cancel_in_the_product():
    """With the same signs on both operands along the reduction axis,
    (X D H)(W D H)^T = X W^T: the quantized product stays within MXFP4's
    error of the exact one (rel. Frobenius ~0.1), while signs drawn
    independently for the two operands destroy it (~1.4)."""
    rng = np.random.default_rng(8)
    X = synthetic.f64_to_bf16_bits(rng.standard_normal((64, 256)))
    W = synthetic.f64_to_bf16_bits(rng.standard_normal((48, 256)))
    P = synthetic.bf16_bits_to_f32(X).astype(np.float64) @ synthetic.bf16_bits_to_f32(W).astype(np.float64).T
    s = synthetic.random_signs(256, 9)
    t = synthetic.random_signs(256, 10)
    for h in (16, 32):
        a = O.dequantize(*O.quantize_rs(X, O.AXIS_ROW, h, 1, s))
        same = O.dequantize(*O.quantize_rs(W, O.AXIS_ROW, h, 1, s))
        other = O.dequantize(*O.quantize_rs(W, O.AXIS_ROW, h, 1, t))
        rel = lambda C: np.linalg.norm(C - P) / np.linalg.norm(P)
        assert rel(a @ same.T) < 0.2
        assert rel(a @ other.T) > 0.9


def _grid_floor_ceil(v):
    """Largest grid value <= |v| and smallest grid value >= |v| (capped at
    6), by exact rational comparison."""
    g = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3),
         Fraction(4), Fraction(6)]
    a = abs(Fraction(float(v)))
    lo = max(i for i in range(8) if g[i] <= a)
    hi = lo if (a == g[lo] or lo == 7) else lo + 1
    return lo, hi


@pytest.mark.parametrize("mode", [O.MODE_OCP_FLOOR, O.MODE_CEIL])
def test_sr_extreme_random_values_floor_and_ceil(mode):
    """rand = 2^32 - 1 never rounds up (p < 1 - 2^-32 for every fp32
    input), so SR is the grid floor of |v|; rand = 0 rounds up whenever
    p > 0, so SR is the grid ceiling (6 at most). Scales equal the
    round-to-nearest operand's. No rotation, so v = x / 2^E with E from
    the scale byte."""
    rng = np.random.default_rng(11 + mode)
    x = synthetic.f64_to_bf16_bits(rng.standard_t(3, size=(16, 64)))
    nib_rtn, sc_rtn = O.quantize(x, O.AXIS_ROW, 0, mode)
    xf = synthetic.bf16_bits_to_f32(x)
    for r, which in ((np.uint32(0xFFFFFFFF), 0), (np.uint32(0), 1)):
        nib, sc = O.quantize_sr(x, O.AXIS_ROW, 0, mode, np.full(x.shape, r, np.uint32))
        assert np.array_equal(sc, sc_rtn)
        codes = _codes_of(nib)
        for i in range(16):
            for j in range(64):
                E = int(sc[i, j // 32]) - 127
                lohi = _grid_floor_ceil(math.ldexp(float(xf[i, j]), -E))
                want = lohi[which] | (8 if np.signbit(xf[i, j]) else 0)
                assert codes[i, j] == want, (r, i, j)


def test_sr_exact_threshold():
    """A block with amax 4 has scale 2^0 in both rules; its value 0.375 lies
    3/4 of the way from 0 to 0.5 and rounds up for rand < 0.75 * 2^32;
    5.0 lies half way from 4 to 6 (threshold 2^31); 3.5 half way from 3
    to 4."""
    row = np.zeros(32)
    row[0], row[1], row[2], row[3] = 4.0, 0.375, 5.0, -3.5
    x = synthetic.f64_to_bf16_bits(row[None, :])
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        for r1, c1 in ((3221225471, 1), (3221225472, 0)):
            for r2, c2 in ((2 ** 31 - 1, 7), (2 ** 31, 6)):
                rnd = np.full((1, 32), 0xFFFFFFFF, np.uint32)
                rnd[0, 1], rnd[0, 2], rnd[0, 3] = r1, r2, r2
                nib, sc = O.quantize_sr(x, O.AXIS_ROW, 0, mode, rnd)
                assert sc[0, 0] == 127
                codes = _codes_of(nib)[0]
                assert codes[0] == 6 and codes[1] == c1 and codes[2] == c2
                assert codes[3] == 8 | (6 if r2 < 2 ** 31 else 5)


def test_sr_is_unbiased():
    """Averaged over independent draws, the dequantized SR value is the
    scaled input (the expected value of a stochastic rounding): each mean is
    within 6 standard errors (gap / 2 / sqrt(n)) of x; a reversed
    probability would miss by up to half a gap."""
    rng = np.random.default_rng(13)
    x = synthetic.f64_to_bf16_bits(rng.standard_normal((8, 64)))
    xf = synthetic.bf16_bits_to_f32(x).astype(np.float64)
    n = 400
    acc = np.zeros(xf.shape)
    for k in range(n):
        nib, sc = O.quantize_sr(x, O.AXIS_ROW, 0, O.MODE_CEIL, synthetic.random_u32(x.shape, 100 + k))
        acc += O.dequantize(nib, sc)
    mean = acc / n
    scale = np.repeat(np.ldexp(1.0, sc.astype(np.int64) - 127), 32, axis=1)
    gap = np.where(np.abs(xf) / scale < 2, 0.5, np.where(np.abs(xf) / scale < 4, 1.0, 2.0)) * scale
    assert np.all(np.abs(mean - xf) <= 6 * gap / 2 / math.sqrt(n))


# ------------------------------------ ideal quantizer Q* ([P3] core insight)
def _exact_ideal(block):
    """Q*(x) of one block by exact rational arithmetic, written from [P3]'s
    core insight: s* = max|x| / q_max, and each x maps to s* times the grid
    value nearest x / s* (ties to the even code; nothing lies beyond q_max,
    so the nearest value of a larger t is q_max itself). Grid and q_max are
    the printed ones (tests/golden)."""
    grid = [Fraction(g) for _, g in _golden_table("e2m1_grid.txt")]
    q_max = Fraction(dict(_golden_table("format_constants.txt"))["q_max"])
    xs = [Fraction(float(v)) for v in block]
    m_b = max(abs(v) for v in xs)
    if m_b == 0:
        return [Fraction(0)] * len(xs)
    s = m_b / q_max
    out = []
    for v in xs:
        t = abs(v) / s
        code = min(range(8), key=lambda c: (abs(t - grid[c]), c % 2))
        out.append((s * grid[code]) * (-1 if v < 0 else 1))
    return out


def test_ideal_quantizer_hand_worked_blocks():
    """Hand-worked Q* outside the deadzone ([P3] core insight).
    m_b = 6, s* = 1: the seven ties 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5 go to
    the even code (0, 1, 1, 2, 2, 4, 4); 0.3 -> 0.5, 4.9 -> 4, -0.75 -> -1.
    m_b = 7, s* = 7/6: 1 -> t = 6/7 -> 1, Q* = 7/6; 3.5 -> t = 3, Q* = 3.5;
    0.5 -> t = 3/7 -> 0.5, Q* = 7/12; 7 -> 7.
    m_b = 3, s* = 1/2: 1.25 -> t = 2.5 (tie) -> 2, Q* = 1; 0.375 -> t = 0.75
    (tie) -> 1, Q* = 0.5; 0.1 is in the deadzone (24 * 0.1 < 3) -> 0."""
    cases = [
        ([6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 0.3, 4.9, -0.75],
         [6, 0, 1, 1, 2, 2, 4, 4, 0.5, 4, -1]),
        ([7, 1, 3.5, 0.5], [7, Fraction(7, 6), 3.5, Fraction(7, 12)]),
        ([3, 1.25, 0.375, 0.1], [3, 1, 0.5, 0]),
    ]
    for vals, want in cases:
        blk = np.zeros((1, 32), dtype=np.float32)
        blk[0, :len(vals)] = vals
        for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
            d = O.error_decomposition(blk, mode)
            for i, w in enumerate(want):
                assert Fraction(d["Q_star"][0, i]) == pytest.approx(Fraction(w), rel=1e-15, abs=0), \
                    (vals, i)
    # the m_b = 3 block: 0.1 is the only deadzone element among the non-zero ones
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, :4] = [3, 1.25, 0.375, 0.1]
    d = O.error_decomposition(blk, O.MODE_CEIL)
    assert list(d["deadzone"][0, :4]) == [False, False, False, True]
    # m_b = 7 in floor mode: E = 0, Q(1) = 1, so e_scale = 1 - 7/6 = -1/6;
    # Q(3.5) = 4 (tie to the even code), e_scale = 1/2; e_grid(3.5) = 0
    blk = np.zeros((1, 32), dtype=np.float32)
    blk[0, :4] = [7, 1, 3.5, 0.5]
    d = O.error_decomposition(blk, O.MODE_OCP_FLOOR)
    assert d["e_scale"][0, 1] == pytest.approx(-1 / 6, rel=1e-14)
    assert d["e_scale"][0, 2] == 0.5 and d["e_grid"][0, 2] == 0.0
    assert d["e_grid"][0, 3] == pytest.approx(7 / 12 - 0.5, rel=1e-14)


def test_ideal_quantizer_against_exact_rationals():
    """Q* of the oracle against the exact rational rule on heavy-tailed
    blocks, plus blocks built to hold exact ties of x / s* (x = tie * m_b / 6
    for m_b = 6 * 2^k and for m_b = 3 * 2^k)."""
    rng = np.random.default_rng(41)
    a = rng.standard_t(3, size=(300, 32)) * rng.lognormal(0, 1, size=(300, 1))
    blocks = [O.bf16_to_f32(synthetic.f64_to_bf16_bits(a))]
    ties = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    for k in range(-6, 7):
        for base in (6.0, 3.0, 4.5):
            m_b = base * 2.0 ** k
            t = np.zeros((1, 32), dtype=np.float32)
            t[0, 0] = m_b
            t[0, 1:8] = ties * m_b / 6
            t[0, 8:15] = -ties * m_b / 6
            t[0, 15:32] = rng.uniform(-m_b, m_b, 17)
            blocks.append(t)
    blocks = np.concatenate(blocks)
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        d = O.error_decomposition(blocks, mode)
        for b in range(blocks.shape[0]):
            want = _exact_ideal(blocks[b])
            for i in range(32):
                got = Fraction(d["Q_star"][b, i])
                assert abs(got - want[i]) <= abs(want[i]) * Fraction(1, 2 ** 50), (b, i)
            dz = [24 * abs(Fraction(float(v))) < max(abs(Fraction(float(u))) for u in blocks[b])
                  for v in blocks[b]]
            assert list(d["deadzone"][b]) == dz


# --------------------------------------------- GEMM tolerance and the report
def test_gemm_tolerance_matches_the_stated_bound():
    """gemm_tolerance is the stated bound and nothing looser: 1e-5 * S for
    fp32 output, plus bf16's round-to-nearest step 2^-8 |C_ref| for bf16
    output (tests/golden/format_constants.txt)."""
    consts = dict(_golden_table("format_constants.txt"))
    tol = float(consts["gemm_abs_sum_tol"])
    u = 2.0 ** int(consts["bf16_roundoff_log2"])
    S = np.array([0.0, 1.0, 3.5, 1e6])
    c = np.array([0.0, -2.0, 0.5, 7e5])
    assert np.array_equal(O.gemm_tolerance(S, c, False), tol * S)
    assert np.array_equal(O.gemm_tolerance(S, c, True), tol * S + u * np.abs(c))


def test_bf16_roundoff_constant_is_the_rounding_bound():
    """The 2^-8 of the bf16 output term is the largest relative change that
    rounding fp32 to bf16 (torch's round-to-nearest-even cast, a library
    routine) makes, and it is approached: a smaller constant would reject
    correctly rounded outputs."""
    import torch
    rng = np.random.default_rng(3)
    bits = rng.integers(0x00800000, 0x7F000000, size=1 << 20, dtype=np.uint32)
    # values just above 1 + 2^-8 * k: the worst case sits at half an ulp
    bits[:4096] = (0x3F800000 + 0x7FFF + np.arange(4096, dtype=np.uint32) * 0x10000) & 0x7FFFFFFF
    x = bits.view(np.float32)
    xb = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    rel = np.abs(xb.astype(np.float64) - x) / np.abs(x.astype(np.float64))
    u = 2.0 ** int(dict(_golden_table("format_constants.txt"))["bf16_roundoff_log2"])
    assert rel.max() <= u
    assert rel.max() > u * (1 - 2.0 ** -6)


def test_error_report_closed_forms():
    """MSE, cosine, relative Frobenius error and SNR on perturbations with
    closed-form values: C = P (1 + eps) gives rel_fro = eps, cosine = 1,
    SNR = -20 log10(eps); C = P + D with D orthogonal to P gives
    cosine = |P| / sqrt(|P|^2 + |D|^2) and MSE = |D|^2 / n."""
    rng = np.random.default_rng(5)
    P = rng.standard_normal((16, 24))
    r = O.error_report(P * 1.125, P)
    assert r["rel_fro"] == pytest.approx(0.125, rel=1e-12)
    assert r["cosine"] == pytest.approx(1.0, rel=1e-12)
    assert r["snr_db"] == pytest.approx(-20 * math.log10(0.125), rel=1e-12)
    D = rng.standard_normal(P.shape)
    D -= P * np.sum(D * P) / np.sum(P * P)
    r = O.error_report(P + D, P)
    nP, nD = np.sum(P * P), np.sum(D * D)
    assert r["cosine"] == pytest.approx(math.sqrt(nP / (nP + nD)), rel=1e-10)
    assert r["mse"] == pytest.approx(nD / P.size, rel=1e-12)
    assert r["snr_db"] == pytest.approx(10 * math.log10(nP / nD), rel=1e-12)


def test_sr_scaled_value_below_the_fp32_range():
    """A scaled value far below fp32's range still has p > 0 in the exact
    definition, so rand = 0 rounds it up to 0.5 and rand = 1 does not.
    Block {2^19, 2^-133, 0...}, no rotation: E = 17 in both rules, and the
    bf16 subnormal 2^-133 scales to 2^-150, which an fp32 multiply would
    round to 0."""
    row = np.zeros((1, 32), dtype=np.uint16)
    row[0, 0] = synthetic.f64_to_bf16_bits(np.array([2.0 ** 19]))[0]
    row[0, 1] = 0x0001            # 2^-133, the smallest bf16 subnormal
    row[0, 2] = 0x8001            # -2^-133
    assert synthetic.bf16_bits_to_f32(row)[0, 1] == 2.0 ** -133
    for mode in (O.MODE_OCP_FLOOR, O.MODE_CEIL):
        for r, want in ((0, 1), (1, 0)):
            rnd = np.full((1, 32), r, np.uint32)
            nib, sc = O.quantize_sr(row, O.AXIS_ROW, 0, mode, rnd)
            assert sc[0, 0] == 127 + 17
            codes = _codes_of(nib)[0]
            assert codes[1] == want and codes[2] == 8 | want
            assert np.all(codes[3:] == 0)


@pytest.mark.parametrize("axis", [O.AXIS_ROW, O.AXIS_COL])
def test_threaded_slabs_equal_the_whole_matrix(axis):
    """The thread-pool form of the slab quantizer (the CPU baseline's) gives
    the bytes of one call on the whole matrix."""
    x = synthetic.f64_to_bf16_bits(np.random.default_rng(17).standard_t(3, size=(160, 224)))
    whole = O.quantize(x, axis, 16, O.MODE_OCP_FLOOR)
    for chunk, threads in ((32, 4), (64, 8), (1, 3)):
        got = O.quantize_chunked(x, axis, 16, O.MODE_OCP_FLOOR, chunk=chunk, threads=threads)
        assert np.array_equal(got[0], whole[0]) and np.array_equal(got[1], whole[1])
