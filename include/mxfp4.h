/*
 * mxfp4.h -- C ABI of the MI355X (gfx950) H16 + MXFP4 quantize + MXFP4 GEMM
 * library (libmxfp4.so).
 *
 * Pages cited (by title and section):
 *  [P1] "Pretraining Large Language Models with MXFP4 on Native FP4 Hardware"
 *       (arXiv:2605.09825, summary page): quick-read block and section A.1
 *       (MX block reconstruction x_rec = 2^E * Q_FP4(x / 2^E), shared exponent
 *       taken from the block maximum, round to the nearest FP4 value);
 *       section A.2 (deterministic tiled 16x16 Hadamard injected before each
 *       MXFP4 GEMM; FP8 GEMMs replaced per product Fprop/Dgrad/Wgrad);
 *       sections C.1-C.3 (cancellation H H^T = I in the three products);
 *       section D (1x32 row-wise, 32x1 column-wise, 32x32 2D block scales).
 *  [P3] "Decomposing MXFP4 quantization error" blog (arXiv:2605.20402),
 *       pain-point section (OCP MX: 32 elements, E8M0 scale 2^n, E2M1 grid
 *       {0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6}); core-insight section
 *       (ceiling-rounded E8M0 scale of s* = max|x| / 6); note that native
 *       MXFP4 GEMMs accumulate in FP32.
 *
 * Conventions shared by every entry point
 *  - All data pointers are DEVICE pointers owned by the caller. The library
 *    never allocates, frees or synchronizes; every call only enqueues
 *    kernels on `stream` (0 = the null stream) and returns.
 *  - bf16 inputs are row-major with a dense row pitch.
 *  - Packed MXFP4 operand ("nibbles + E8M0 bytes"): nibble byte j of a row
 *    holds element 2j in bits 0-3 and element 2j+1 in bits 4-7; an element
 *    code is sign << 3 | magnitude code (magnitudes 0, .5, 1, 1.5, 2, 3, 4, 6
 *    for codes 0..7). One E8M0 byte (value 2^(byte - 127), 0xFF = NaN) per
 *    block of 32 elements along the row.
 *  - Every check runs on the host before any HIP call; a failed check
 *    returns its status and launches nothing. After launching, a pending
 *    HIP launch error is returned as MXFP4_ERR_HIP.
 *  - Pointers handed to vector loads/stores must be 16-byte aligned
 *    (bf16 sources, nibble outputs, GEMM operands); scale arrays and C need
 *    no alignment beyond their element size.
 *  - Calls are thread-safe. The only state shared between calls is a
 *    per-device cache of the compute-unit count (set once, atomically) and
 *    the static array of mxfp4_error_stats_noalloc (see there). Calls on
 *    one stream run in stream order.
 */
#ifndef MXFP4_H_
#define MXFP4_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MXFP4_OK = 0,
  MXFP4_ERR_NULL = 1,      /* a required pointer is NULL                       */
  MXFP4_ERR_SHAPE = 2,     /* a size is negative, zero where not allowed, or not
                              a multiple of the block / Hadamard size           */
  MXFP4_ERR_MODE = 3,      /* axis, hadamard, scale_mode or out_dtype invalid  */
  MXFP4_ERR_WORKSPACE = 4, /* ws_bytes below mxfp4_workspace_bytes()           */
  MXFP4_ERR_HIP = 5,       /* the HIP runtime reported an error on launch      */
  MXFP4_ERR_ALIGN = 6      /* a vector-accessed pointer is not 16-byte aligned */
} mxfp4_status;

typedef enum {
  MXFP4_AXIS_ROW = 0,  /* 1x32 blocks along cols ([P1] D, row-wise)            */
  MXFP4_AXIS_COL = 1,  /* 32x1 blocks down rows, transposed output ([P1] D)    */
  MXFP4_AXIS_2D32 = 2  /* one scale per 32x32 tile ([P1] D, 2D)                */
} mxfp4_axis;

typedef enum {
  MXFP4_SCALE_OCP_FLOOR = 0, /* E = floor(log2 amax) - 2 ([P1] A.1 with the OCP
                                MX offset of E2M1's largest exponent)          */
  MXFP4_SCALE_CEIL = 1       /* smallest E with 6 * 2^E >= amax ([P3])         */
} mxfp4_scale_mode;

typedef enum { MXFP4_OUT_F32 = 0, MXFP4_OUT_BF16 = 1 } mxfp4_out;

typedef enum { MXFP4_OP_FPROP = 0, MXFP4_OP_DGRAD = 1, MXFP4_OP_WGRAD = 2 } mxfp4_op;

/*
 * mxfp4_quantize -- rotate then MXFP4-quantize a bf16 matrix src[rows][cols].
 * ([P1] A.1 and D; rotation [P1] A.2; grid and scale rules [P3].)
 *
 * hadamard: 0 (no rotation), 16 or 32. Each aligned group of `hadamard`
 *   elements along the rotated axis becomes x * H, H the Sylvester matrix
 *   scaled by 1/4 (H16) or RN_fp32(2^-2.5) (H32), evaluated as the fp32
 *   butterfly with stages 1, 2, 4, 8 (, 16) and one final multiply.
 * Per block of 32 rotated values: amax m_b; E8M0 exponent E by scale_mode
 *   (zero block: E = -127; clamp to [-127, 127]); element codes are the
 *   nearest E2M1 value of y / 2^E, ties to the even code, saturating at 6,
 *   sign bit kept. A block holding a non-finite rotated value gets scale
 *   byte 0xFF and all-zero nibbles.
 *
 * axis = MXFP4_AXIS_ROW: rotate and block along cols. cols % 32 == 0.
 *   out_nibbles [rows][cols/2], out_e8m0 [rows][cols/32].
 * axis = MXFP4_AXIS_COL: rotate and block down rows; the output is the
 *   transposed operand (K-contiguous for the GEMM). rows % 32 == 0.
 *   out_nibbles [cols][rows/2], out_e8m0 [cols][rows/32].
 * axis = MXFP4_AXIS_2D32: rotate along cols, one scale per 32x32 tile.
 *   rows % 32 == 0, cols % 32 == 0.
 *   out_nibbles [rows][cols/2], out_e8m0 [rows/32][cols/32].
 * rows == 0 or cols == 0 is a valid empty call (nothing is launched).
 * Outputs are fully overwritten. Deterministic: identical inputs give
 * identical bytes.
 */
int mxfp4_quantize(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                   int hadamard, int scale_mode, void* out_nibbles, void* out_e8m0,
                   hipStream_t stream);

/*
 * mxfp4_quantize_pair -- the two operands of a product in one call: the
 * outputs of mxfp4_quantize(src_a, rows_a, cols_a, axis_a, ...) and
 * mxfp4_quantize(src_b, ...) with the same hadamard and scale_mode, byte
 * for byte. Where both shapes allow it (row-wise operands; column-wise
 * operands with rows % 256 == 0, cols % 4 == 0 and e8m0 8-byte aligned)
 * both run in ONE launch over the two grids, which saves one launch's ramp
 * and tail ([P1] Table 2 note: memory bandwidth is the bottleneck of these
 * steps); otherwise two launches. Axes ROW or COL (2D32 returns
 * MXFP4_ERR_MODE); each operand validated as by mxfp4_quantize, errors of
 * operand A first; an empty operand launches nothing. The outputs must not
 * overlap each other or the sources.
 */
int mxfp4_quantize_pair(const void* src_a, int64_t rows_a, int64_t cols_a, int axis_a,
                        void* nibbles_a, void* e8m0_a, const void* src_b, int64_t rows_b,
                        int64_t cols_b, int axis_b, void* nibbles_b, void* e8m0_b, int hadamard,
                        int scale_mode, hipStream_t stream);

/*
 * mxfp4_quantize_dual -- one read of src[rows][cols], both orientations.
 * ([P1] A.2 and D: the activation X feeds Fprop rotated and blocked along
 * its feature axis and Wgrad rotated and blocked along the token axis;
 * [P1] C.1 and C.3.)
 *
 * Writes exactly what two mxfp4_quantize calls with the same hadamard and
 * scale_mode would write: the row-wise operand (MXFP4_AXIS_ROW) into
 * row_nibbles [rows][cols/2] and row_e8m0 [rows][cols/32], and the
 * column-wise transposed operand (MXFP4_AXIS_COL) into col_nibbles
 * [cols][rows/2] and col_e8m0 [cols][rows/32]. Each output is rotated along
 * its own blocking axis. rows % 32 == 0 and cols % 32 == 0. When
 * rows % 128 == 0, cols % 256 == 0, row_e8m0 is 8-byte and col_e8m0 4-byte
 * aligned, one kernel reads src once (2 B per element instead of 4);
 * otherwise the two single-orientation kernels run back to back. Errors,
 * alignment and empty shapes as mxfp4_quantize (both checks apply).
 */
int mxfp4_quantize_dual(const void* src_bf16, int64_t rows, int64_t cols,
                        int hadamard, int scale_mode, void* row_nibbles, void* row_e8m0,
                        void* col_nibbles, void* col_e8m0, hipStream_t stream);

/*
 * mxfp4_quantize_of -- outlier-fallback (OF) operand ([P3] "three targeted
 * fixes" section: x_OF = Q(x) + alpha Q(x - Q(x)), alpha = 0.5, which
 * brings deadzone values back onto the grid).
 *
 * With y the rotated values mxfp4_quantize encodes (axis ROW or COL),
 * q1 = Q(y) and r = fl32(y - q1): q2 = Q(fl32(r / 2)) (alpha applied as a
 * prescale of the residual; equal to Q(r) / 2 unless the residual block's
 * E8M0 exponent is at its floor of -127). The result is ONE packed operand
 * twice as deep: row i of out_nibbles / out_e8m0 is q1's row followed by
 * q2's row, i.e. out_nibbles [R][Kb] and out_e8m0 [R][2 Kb/32] with R, Kb =
 * rows, cols (axis ROW) or cols, rows (axis COL, transposed). A GEMM of
 * depth 2 Kb against the other operand's packed rows repeated twice along
 * K then computes sum_k (q1 + q2) b. A block holding a non-finite rotated
 * value is 0xFF with zero nibbles in both halves. Shapes, alignment and
 * errors as mxfp4_quantize; axis MXFP4_AXIS_2D32 returns MXFP4_ERR_MODE.
 */
int mxfp4_quantize_of(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                      int hadamard, int scale_mode, void* out_nibbles, void* out_e8m0,
                      hipStream_t stream);

/*
 * mxfp4_quantize_mbs -- macro-block-scaled (MBS) operand ([P3] "three
 * targeted fixes" section: an 8-bit mantissa correction s = 2^e (1 + m)
 * per macro-block of 128 elements, x_hat = Q((1 + m) x) / (1 + m)).
 *
 * With y the rotated values mxfp4_quantize encodes (axis ROW or COL) and
 * M the absolute maximum of each run of 128 along the blocked axis:
 * c = 1 + m/256 with m the largest byte such that c M <= 6 2^k, k the
 * smallest integer with 6 2^k >= M (m = floor(256 (6 2^k / M - 1)) in
 * fp64; 0 for a zero or non-finite M). out_nibbles / out_e8m0 receive
 * exactly mxfp4_quantize's output for fl32(c y); out_mbs receives m,
 * [rows][cols/128] (ROW) or [cols][rows/128] (COL). The value is
 * dequant(nibbles, e8m0) / c; a GEMM consuming it needs that per-128-k
 * factor on each operand (mxfp4_gemm_mbs; not mxfp4_gemm). The blocked axis
 * must be a multiple of 128; otherwise as mxfp4_quantize (axis 2D32 returns
 * MXFP4_ERR_MODE).
 */
int mxfp4_quantize_mbs(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                       int hadamard, int scale_mode, void* out_nibbles, void* out_e8m0,
                       void* out_mbs, hipStream_t stream);

/*
 * mxfp4_quantize_rs -- random-sign Hadamard comparison arm. [P1]'s
 * quick-read block, section A.2 and hypothesis H2 report that random
 * Hadamard transforms (random sign flips before the rotation) diverge
 * under full MXFP4 training, where the deterministic H16 trains; this entry
 * point produces such an operand so that its quantization error can be
 * measured.
 *
 * Writes exactly what mxfp4_quantize (axis ROW or COL) writes for diag(s)
 * src, s_i = -1 where bit 0 of signs[i] is set and +1 where it is clear,
 * i indexing the blocked (rotated) axis. signs: DEVICE bytes, [cols] for
 * MXFP4_AXIS_ROW (16-byte aligned) or [rows] for MXFP4_AXIS_COL, owned by
 * the caller. The two operands of a product take the same signs along the
 * reduction axis, so the signs cancel in the product. A NULL signs with a
 * non-empty shape returns MXFP4_ERR_NULL, a misaligned one (row axis)
 * MXFP4_ERR_ALIGN; otherwise errors as mxfp4_quantize (axis 2D32 returns
 * MXFP4_ERR_MODE).
 */
int mxfp4_quantize_rs(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                      int hadamard, int scale_mode, const void* signs, void* out_nibbles,
                      void* out_e8m0, hipStream_t stream);

/*
 * mxfp4_quantize_sr -- stochastic-rounding comparison arm ([P1]'s
 * quick-read block and hypothesis H2: stochastic rounding diverges under full
 * MXFP4 training; this operand lets its quantization error be measured).
 *
 * The E8M0 bytes are mxfp4_quantize's (same rule on the same rotated block
 * maxima). Element codes: with y the rotated value, E its block's exponent
 * and u its random integer, a = |y| 2^-E (exact, fp64); a >= 6 gives 6;
 * otherwise, between the neighbouring E2M1 values g_lo <= a < g_hi, the
 * magnitude is g_hi exactly when u < 2^32 (a - g_lo) / (g_hi - g_lo) (a
 * probability equal to the distance, so the expected value is a) and g_lo
 * otherwise; the sign bit is y's. rand_u32: DEVICE uint32 [rows][cols]
 * (16-byte aligned, caller-owned), one per source element, element (r, c)
 * using rand_u32[r][c] for either axis. A NULL rand_u32 with a non-empty
 * shape returns MXFP4_ERR_NULL, a misaligned one MXFP4_ERR_ALIGN;
 * otherwise errors as mxfp4_quantize (axis 2D32 returns MXFP4_ERR_MODE).
 */
int mxfp4_quantize_sr(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                      int hadamard, int scale_mode, const void* rand_u32, void* out_nibbles,
                      void* out_e8m0, hipStream_t stream);

/*
 * mxfp4_error_stats -- tensor-level decomposition of the MXFP4 error of the
 * operand mxfp4_quantize would produce ([P3] core insight: ideal scale
 * s* = m_b / 6, e = e_scale + e_DZ + e_grid, deadzone |x| < m_b / 24;
 * [P3] Property 1: orthogonality and the MSE identity).
 *
 * For every 1x32 (axis MXFP4_AXIS_ROW) or 32x1 (MXFP4_AXIS_COL) block of
 * the rotated source x (fp32, as mxfp4_quantize computes it) with amax m_b:
 * Q = the block's dequantized MXFP4 values (E8M0 by scale_mode, E2M1 codes);
 * Q* = s* * nearest E2M1 value of x / s* (ties to the even code, clamp 6),
 * computed in fp64; D = {i : 24 |x_i| < m_b}; e_scale = Q - Q*,
 * e_DZ = (Q* - x) on D, e_grid = (Q* - x) off D, e = Q - x.
 * out_stats (DEVICE, 10 doubles, 8-byte aligned) receives, summed over the
 * tensor in fp64:
 *   [0] sum e_scale^2   [1] sum e_DZ^2    [2] sum e_grid^2
 *   [3] sum e_scale*e_grid               [4] sum e_scale*e_DZ
 *   [5] sum e^2         [6] sum x^2       [7] deadzone count
 *   [8] elements counted                 [9] blocks skipped (non-finite)
 * Blocks holding a non-finite rotated value are skipped. The sums are added
 * in a fixed order: repeated calls give identical bits. ws: caller
 * workspace of at least MXFP4_ERROR_STATS_WS_BYTES (16-byte aligned).
 * axis MXFP4_AXIS_2D32 returns MXFP4_ERR_MODE; shapes, hadamard, scale_mode
 * and the src alignment as mxfp4_quantize. rows == 0 or cols == 0 writes
 * zeros. Two launches on `stream`.
 */
#define MXFP4_ERROR_STATS_COUNT 10
#define MXFP4_ERROR_STATS_WS_BYTES (1024 * MXFP4_ERROR_STATS_COUNT * 8)
int mxfp4_error_stats(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                      int hadamard, int scale_mode, void* ws, size_t ws_bytes,
                      double* out_stats, hipStream_t stream);

/*
 * mxfp4_error_stats_noalloc -- mxfp4_error_stats without a workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same arguments, results and errors as mxfp4_error_stats minus ws and
 * ws_bytes; out_stats (DEVICE, 10 doubles, 8-byte aligned) is still the
 * caller's. The per-work-group partial sums go to a static device array of
 * the library, 1024 x 10 doubles (80 KiB), that every GPU the library runs
 * on holds until the process ends. Any input size fits: the first pass
 * never launches more than 1024 work-groups. Allocates nothing and calls no
 * allocating routine; the array's device address is looked up on the first
 * call on each device (with that device current), so `stream` must belong
 * to the current device. Every call on one GPU shares that GPU's array:
 * calls that overlap on one GPU (concurrent streams, or threads) race and
 * give wrong sums; calls ordered on one stream are safe. Nothing needs
 * clearing: each call writes every partial it reads.
 */
int mxfp4_error_stats_noalloc(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                              int hadamard, int scale_mode, double* out_stats,
                              hipStream_t stream);

/*
 * mxfp4_gemm -- C[M][N] = sum_k deqA[m][k] * deqB[n][k] on gfx950's
 * block-scaled FP4 MFMA with FP32 accumulation ([P1] A.2; [P3]).
 *
 * A: Aq [M][K/2] nibbles, As [M][K/32] E8M0 bytes.
 * B: Bq [N][K/2] nibbles, Bs [N][K/32] E8M0 bytes (both K-contiguous).
 * C: row-major [M][N], fp32 (out_dtype 0) or bf16 (1, round to nearest
 *    even from the fp32 accumulator). C is overwritten, not accumulated.
 * M >= 1, N >= 1, K >= 32, K % 32 == 0. Any M and N (edge tiles are
 * predicated).
 */
int mxfp4_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs,
               int64_t M, int64_t N, int64_t K, void* C, int out_dtype,
               hipStream_t stream);

/*
 * mxfp4_gemm_mbs -- the product of two macro-block-scaled operands
 * (mxfp4_quantize_mbs outputs; [P3] "three targeted fixes" section, MBS:
 * prescale by c = 1 + m/256, quantize, postscale by 1/c per 128-element
 * macro-block):
 *   C[m][n] = sum_k (deqA[m][k] / cA[m][k/128]) (deqB[n][k] / cB[n][k/128]).
 * A: Aq [M][K/2], As [M][K/32], Am [M][K/128] mantissa bytes; B likewise
 * with N rows; all K-contiguous. Each 128-k macro-block's MXFP4 product is
 * accumulated in fp32 and added to C times fl32(1/cA) fl32(1/cB) (FP32
 * accumulation as in mxfp4_gemm). C: as mxfp4_gemm (fp32 or bf16,
 * overwritten). M >= 1, N >= 1, K >= 128, K % 128 == 0; other errors as
 * mxfp4_gemm (Am and Bm may have any alignment). One launch on `stream`.
 */
int mxfp4_gemm_mbs(const void* Aq, const void* As, const void* Am, const void* Bq,
                   const void* Bs, const void* Bm, int64_t M, int64_t N, int64_t K, void* C,
                   int out_dtype, hipStream_t stream);

/*
 * Fused linear-layer products ([P1] C.1, C.2, C.3). Each quantizes both
 * operands with the same `hadamard` and `scale_mode`, rotating along the
 * product's reduction axis, into the caller's workspace `ws` (ws_bytes >=
 * mxfp4_workspace_bytes(op, T, N, K), 256-byte aligned), then runs
 * mxfp4_gemm. The two operands are quantized as by mxfp4_quantize_pair (one
 * launch for every Llama-shaped product), then one GEMM launch, on `stream`. Shapes follow Y = X W^T with
 * X [T][K], W [N][K], Y [T][N]:
 *
 * mxfp4_fprop: Y[T][N]  = X[T][K] W[N][K]^T. X, W quantized row-wise along
 *              K. K % 32 == 0.
 * mxfp4_dgrad: dX[T][K] = dY[T][N] W[N][K]. dY row-wise along N, W
 *              column-wise along N (transposed to [K][N]). N % 32 == 0.
 * mxfp4_wgrad: dW[N][K] = dY[T][N]^T X[T][K]. dY and X column-wise along
 *              the token axis T. T % 32 == 0.
 */
int mxfp4_fprop(const void* X, const void* W, int64_t T, int64_t N, int64_t K,
                int hadamard, int scale_mode, void* ws, size_t ws_bytes, void* Y,
                int out_dtype, hipStream_t stream);
int mxfp4_dgrad(const void* dY, const void* W, int64_t T, int64_t N, int64_t K,
                int hadamard, int scale_mode, void* ws, size_t ws_bytes, void* dX,
                int out_dtype, hipStream_t stream);
int mxfp4_wgrad(const void* dY, const void* X, int64_t T, int64_t N, int64_t K,
                int hadamard, int scale_mode, void* ws, size_t ws_bytes, void* dW,
                int out_dtype, hipStream_t stream);

/* Workspace bytes of a fused product (op: mxfp4_op): both packed operands,
 * each piece rounded up to 256 bytes. Returns 0 for invalid arguments. */
size_t mxfp4_workspace_bytes(int op, int64_t T, int64_t N, int64_t K);

/* Static text of a status code ("MXFP4_OK", ...); never NULL. */
const char* mxfp4_status_string(int status);

#ifdef __cplusplus
}
#endif
#endif /* MXFP4_H_ */
