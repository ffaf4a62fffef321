// C ABI of libmxfp4: argument validation (host only, before any HIP call),
// workspace carving for the fused products, and status strings.
//
// The fused products follow the three cancellations of [P1] "Pretraining
// Large Language Models with MXFP4 on Native FP4 Hardware" (arXiv:2605.09825
// summary), sections C.1 (Fprop: X H and W H), C.2 (Dgrad: dY H and W^T H)
// and C.3 (Wgrad: dY^T H and X^T H): both operands are rotated along the
// product's reduction axis and quantized into K-contiguous packed operands,
// then one MXFP4 GEMM runs on them.
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/mxfp4.h"
#include "internal.h"

static_assert(MXFP4_ERROR_STATS_WS_BYTES ==
                  mx::kStatsMaxGroups * MXFP4_ERROR_STATS_COUNT * sizeof(double),
              "error-statistics workspace size");

namespace {

constexpr int64_t kMaxDim = int64_t(1) << 31;   // per-dimension limit (grid and index math)
constexpr int64_t kMaxElems = int64_t(1) << 40; // per-matrix element limit

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned2(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 1u) == 0; }
size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

bool valid_hadamard(int h) { return h == 0 || h == 16 || h == 32; }
bool valid_mode(int m) { return m == MXFP4_SCALE_OCP_FLOOR || m == MXFP4_SCALE_CEIL; }
bool valid_out(int o) { return o == MXFP4_OUT_F32 || o == MXFP4_OUT_BF16; }

bool dims_ok(int64_t a, int64_t b) {
  return a >= 0 && b >= 0 && a < kMaxDim && b < kMaxDim && (a == 0 || b <= kMaxElems / a);
}

// Modes, shape and the bf16 source of a rotate + quantize pass.
int check_source(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                 int scale_mode) {
  if (axis < MXFP4_AXIS_ROW || axis > MXFP4_AXIS_2D32 || !valid_hadamard(hadamard) ||
      !valid_mode(scale_mode))
    return MXFP4_ERR_MODE;
  if (!dims_ok(rows, cols)) return MXFP4_ERR_SHAPE;
  const int64_t blocked = axis == MXFP4_AXIS_COL ? rows : cols;
  if (blocked % 32) return MXFP4_ERR_SHAPE;
  if (axis == MXFP4_AXIS_2D32 && rows % 32) return MXFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXFP4_OK;
  if (!src) return MXFP4_ERR_NULL;
  if (!aligned16(src)) return MXFP4_ERR_ALIGN;
  return MXFP4_OK;
}

int check_quantize(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                   int scale_mode, const void* nib, const void* sc) {
  const int st = check_source(src, rows, cols, axis, hadamard, scale_mode);
  if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
  if (!nib || !sc) return MXFP4_ERR_NULL;
  if (!aligned16(nib)) return MXFP4_ERR_ALIGN;
  return MXFP4_OK;
}

int check_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs, int64_t M,
               int64_t N, int64_t K, const void* C, int out_dtype) {
  if (!valid_out(out_dtype)) return MXFP4_ERR_MODE;
  if (M < 1 || N < 1 || K < 32 || K % 32 || !dims_ok(M, K) || !dims_ok(N, K) || !dims_ok(M, N))
    return MXFP4_ERR_SHAPE;
  if (!Aq || !As || !Bq || !Bs || !C) return MXFP4_ERR_NULL;
  if (!aligned16(Aq) || !aligned16(Bq)) return MXFP4_ERR_ALIGN;
  if (out_dtype == MXFP4_OUT_F32 ? (reinterpret_cast<uintptr_t>(C) & 3u) : !aligned2(C))
    return MXFP4_ERR_ALIGN;
  return MXFP4_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MXFP4_OK : MXFP4_ERR_HIP; }

// Sizes of the two packed operands of a fused product.
struct Operand {
  int64_t rows, cols;  // shape of the bf16 source
  int axis;            // quantization axis
  size_t nib_bytes() const {
    return axis == MXFP4_AXIS_COL ? size_t(cols) * size_t(rows / 2) : size_t(rows) * size_t(cols / 2);
  }
  size_t sc_bytes() const {
    return axis == MXFP4_AXIS_COL ? size_t(cols) * size_t(rows / 32) : size_t(rows) * size_t(cols / 32);
  }
  size_t ws() const { return round256(nib_bytes()) + round256(sc_bytes()); }
};

struct Plan {
  Operand a, b;
  int64_t M, N, K;  // GEMM sizes
};

// fprop: A = q_row(X[T][K]), B = q_row(W[N][K]), GEMM (T, N, K)
// dgrad: A = q_row(dY[T][N]), B = q_col(W[N][K]) -> [K][N], GEMM (T, K, N)
// wgrad: A = q_col(dY[T][N]) -> [N][T], B = q_col(X[T][K]) -> [K][T], GEMM (N, K, T)
bool make_plan(int op, int64_t T, int64_t N, int64_t K, Plan* p) {
  if (T < 1 || N < 1 || K < 1) return false;
  switch (op) {
    case MXFP4_OP_FPROP:
      *p = {{T, K, MXFP4_AXIS_ROW}, {N, K, MXFP4_AXIS_ROW}, T, N, K};
      return K % 32 == 0 && dims_ok(T, K) && dims_ok(N, K) && dims_ok(T, N);
    case MXFP4_OP_DGRAD:
      *p = {{T, N, MXFP4_AXIS_ROW}, {N, K, MXFP4_AXIS_COL}, T, K, N};
      return N % 32 == 0 && dims_ok(T, N) && dims_ok(N, K) && dims_ok(T, K);
    case MXFP4_OP_WGRAD:
      *p = {{T, N, MXFP4_AXIS_COL}, {T, K, MXFP4_AXIS_COL}, N, K, T};
      return T % 32 == 0 && dims_ok(T, N) && dims_ok(T, K) && dims_ok(N, K);
    default:
      return false;
  }
}

int run_fused(int op, const void* P, const void* Q, int64_t T, int64_t N, int64_t K,
              int hadamard, int scale_mode, void* ws, size_t ws_bytes, void* out,
              int out_dtype, hipStream_t stream) {
  if (op < MXFP4_OP_FPROP || op > MXFP4_OP_WGRAD || !valid_hadamard(hadamard) ||
      !valid_mode(scale_mode) || !valid_out(out_dtype))
    return MXFP4_ERR_MODE;
  Plan p;
  if (!make_plan(op, T, N, K, &p)) return MXFP4_ERR_SHAPE;
  if (!P || !Q || !ws || !out) return MXFP4_ERR_NULL;
  if (ws_bytes < p.a.ws() + p.b.ws()) return MXFP4_ERR_WORKSPACE;
  if (!aligned16(P) || !aligned16(Q) || (reinterpret_cast<uintptr_t>(ws) & 255u))
    return MXFP4_ERR_ALIGN;
  if (out_dtype == MXFP4_OUT_F32 ? (reinterpret_cast<uintptr_t>(out) & 3u) : !aligned2(out))
    return MXFP4_ERR_ALIGN;
  uint8_t* w = static_cast<uint8_t*>(ws);
  uint8_t* a_nib = w;
  uint8_t* a_sc = a_nib + round256(p.a.nib_bytes());
  uint8_t* b_nib = a_sc + round256(p.a.sc_bytes());
  uint8_t* b_sc = b_nib + round256(p.b.nib_bytes());
  const hipError_t e = mx::launch_quantize_pair(P, p.a.rows, p.a.cols, p.a.axis, a_nib, a_sc, Q,
                                                p.b.rows, p.b.cols, p.b.axis, b_nib, b_sc,
                                                hadamard, scale_mode, stream);
  if (e != hipSuccess) return MXFP4_ERR_HIP;
  return hip_status(mx::launch_gemm(a_nib, a_sc, b_nib, b_sc, p.M, p.N, p.K, out, out_dtype, stream));
}

}  // namespace

extern "C" {

int mxfp4_quantize(const void* src_bf16, int64_t rows, int64_t cols, int axis, int hadamard,
                   int scale_mode, void* out_nibbles, void* out_e8m0, hipStream_t stream) {
  const int st = check_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode, out_nibbles,
                                out_e8m0);
  if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
  return hip_status(mx::launch_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode,
                                        out_nibbles, out_e8m0, stream));
}

int mxfp4_quantize_pair(const void* src_a, int64_t rows_a, int64_t cols_a, int axis_a,
                        void* nibbles_a, void* e8m0_a, const void* src_b, int64_t rows_b,
                        int64_t cols_b, int axis_b, void* nibbles_b, void* e8m0_b, int hadamard,
                        int scale_mode, hipStream_t stream) {
  if (axis_a == MXFP4_AXIS_2D32 || axis_b == MXFP4_AXIS_2D32) return MXFP4_ERR_MODE;
  int st = check_quantize(src_a, rows_a, cols_a, axis_a, hadamard, scale_mode, nibbles_a, e8m0_a);
  if (st == MXFP4_OK)
    st = check_quantize(src_b, rows_b, cols_b, axis_b, hadamard, scale_mode, nibbles_b, e8m0_b);
  if (st != MXFP4_OK) return st;
  const bool ea = rows_a == 0 || cols_a == 0, eb = rows_b == 0 || cols_b == 0;
  if (ea && eb) return MXFP4_OK;
  if (ea || eb) {  // one empty operand: the other alone
    return hip_status(ea ? mx::launch_quantize(src_b, rows_b, cols_b, axis_b, hadamard, scale_mode,
                                               nibbles_b, e8m0_b, stream)
                         : mx::launch_quantize(src_a, rows_a, cols_a, axis_a, hadamard, scale_mode,
                                               nibbles_a, e8m0_a, stream));
  }
  return hip_status(mx::launch_quantize_pair(src_a, rows_a, cols_a, axis_a, nibbles_a, e8m0_a,
                                             src_b, rows_b, cols_b, axis_b, nibbles_b, e8m0_b,
                                             hadamard, scale_mode, stream));
}

int mxfp4_quantize_dual(const void* src_bf16, int64_t rows, int64_t cols, int hadamard,
                        int scale_mode, void* row_nibbles, void* row_e8m0, void* col_nibbles,
                        void* col_e8m0, hipStream_t stream) {
  int st = check_quantize(src_bf16, rows, cols, MXFP4_AXIS_ROW, hadamard, scale_mode,
                          row_nibbles, row_e8m0);
  if (st == MXFP4_OK)
    st = check_quantize(src_bf16, rows, cols, MXFP4_AXIS_COL, hadamard, scale_mode, col_nibbles,
                        col_e8m0);
  if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
  return hip_status(mx::launch_quantize_dual(src_bf16, rows, cols, hadamard, scale_mode,
                                             row_nibbles, row_e8m0, col_nibbles, col_e8m0,
                                             stream));
}

int mxfp4_quantize_of(const void* src_bf16, int64_t rows, int64_t cols, int axis, int hadamard,
                      int scale_mode, void* out_nibbles, void* out_e8m0, hipStream_t stream) {
  if (axis != MXFP4_AXIS_ROW && axis != MXFP4_AXIS_COL) return MXFP4_ERR_MODE;
  const int st = check_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode, out_nibbles,
                                out_e8m0);
  if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
  return hip_status(mx::launch_quantize_of(src_bf16, rows, cols, axis, hadamard, scale_mode,
                                           out_nibbles, out_e8m0, stream));
}

int mxfp4_quantize_mbs(const void* src_bf16, int64_t rows, int64_t cols, int axis, int hadamard,
                       int scale_mode, void* out_nibbles, void* out_e8m0, void* out_mbs,
                       hipStream_t stream) {
  if (axis != MXFP4_AXIS_ROW && axis != MXFP4_AXIS_COL) return MXFP4_ERR_MODE;
  const int st = check_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode, out_nibbles,
                                out_e8m0);
  if (st != MXFP4_OK) return st;
  if ((axis == MXFP4_AXIS_ROW ? cols : rows) % 128) return MXFP4_ERR_SHAPE;
  if (rows == 0 || cols == 0) return MXFP4_OK;
  if (!out_mbs) return MXFP4_ERR_NULL;
  return hip_status(mx::launch_quantize_mbs(src_bf16, rows, cols, axis, hadamard, scale_mode,
                                            out_nibbles, out_e8m0, out_mbs, stream));
}

int mxfp4_quantize_rs(const void* src_bf16, int64_t rows, int64_t cols, int axis, int hadamard,
                      int scale_mode, const void* signs, void* out_nibbles, void* out_e8m0,
                      hipStream_t stream) {
  if (axis != MXFP4_AXIS_ROW && axis != MXFP4_AXIS_COL) return MXFP4_ERR_MODE;
  const int st = check_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode, out_nibbles,
                                out_e8m0);
  if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
  if (!signs) return MXFP4_ERR_NULL;
  if (axis == MXFP4_AXIS_ROW && !aligned16(signs)) return MXFP4_ERR_ALIGN;
  return hip_status(mx::launch_quantize_rs(src_bf16, rows, cols, axis, hadamard, scale_mode,
                                           signs, out_nibbles, out_e8m0, stream));
}

int mxfp4_quantize_sr(const void* src_bf16, int64_t rows, int64_t cols, int axis, int hadamard,
                      int scale_mode, const void* rand_u32, void* out_nibbles, void* out_e8m0,
                      hipStream_t stream) {
  if (axis != MXFP4_AXIS_ROW && axis != MXFP4_AXIS_COL) return MXFP4_ERR_MODE;
  const int st = check_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode, out_nibbles,
                                out_e8m0);
  if (st != MXFP4_OK || rows == 0 || cols == 0) return st;
  if (!rand_u32) return MXFP4_ERR_NULL;
  if (!aligned16(rand_u32)) return MXFP4_ERR_ALIGN;
  return hip_status(mx::launch_quantize_sr(src_bf16, rows, cols, axis, hadamard, scale_mode,
                                           rand_u32, out_nibbles, out_e8m0, stream));
}

int mxfp4_error_stats(const void* src_bf16, int64_t rows, int64_t cols, int axis, int hadamard,
                      int scale_mode, void* ws, size_t ws_bytes, double* out_stats,
                      hipStream_t stream) {
  if (axis != MXFP4_AXIS_ROW && axis != MXFP4_AXIS_COL) return MXFP4_ERR_MODE;
  const int st = check_quantize(src_bf16, rows, cols, axis, hadamard, scale_mode, ws, out_stats);
  if (st != MXFP4_OK) return st;
  if (!ws || !out_stats || ((rows == 0 || cols == 0) ? false : !src_bf16)) return MXFP4_ERR_NULL;
  if (ws_bytes < MXFP4_ERROR_STATS_WS_BYTES) return MXFP4_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(out_stats) & 7u) || (reinterpret_cast<uintptr_t>(ws) & 7u))
    return MXFP4_ERR_ALIGN;
  return hip_status(mx::launch_error_stats(src_bf16, rows, cols, axis, hadamard, scale_mode, ws,
                                           out_stats, stream));
}

int mxfp4_error_stats_noalloc(const void* src_bf16, int64_t rows, int64_t cols, int axis,
                              int hadamard, int scale_mode, double* out_stats,
                              hipStream_t stream) {
  if (axis != MXFP4_AXIS_ROW && axis != MXFP4_AXIS_COL) return MXFP4_ERR_MODE;
  const int st = check_source(src_bf16, rows, cols, axis, hadamard, scale_mode);
  if (st != MXFP4_OK) return st;
  if (!out_stats) return MXFP4_ERR_NULL;
  if (reinterpret_cast<uintptr_t>(out_stats) & 7u) return MXFP4_ERR_ALIGN;
  return hip_status(mx::launch_error_stats_noalloc(src_bf16, rows, cols, axis, hadamard,
                                                   scale_mode, out_stats, stream));
}

int mxfp4_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs, int64_t M,
               int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  const int st = check_gemm(Aq, As, Bq, Bs, M, N, K, C, out_dtype);
  if (st != MXFP4_OK) return st;
  return hip_status(mx::launch_gemm(Aq, As, Bq, Bs, M, N, K, C, out_dtype, stream));
}

int mxfp4_gemm_mbs(const void* Aq, const void* As, const void* Am, const void* Bq,
                   const void* Bs, const void* Bm, int64_t M, int64_t N, int64_t K, void* C,
                   int out_dtype, hipStream_t stream) {
  const int st = check_gemm(Aq, As, Bq, Bs, M, N, K, C, out_dtype);
  if (st != MXFP4_OK) return st;
  if (K % 128) return MXFP4_ERR_SHAPE;
  if (!Am || !Bm) return MXFP4_ERR_NULL;
  return hip_status(
      mx::launch_gemm_mbs(Aq, As, Am, Bq, Bs, Bm, M, N, K, C, out_dtype, stream));
}

int mxfp4_fprop(const void* X, const void* W, int64_t T, int64_t N, int64_t K, int hadamard,
                int scale_mode, void* ws, size_t ws_bytes, void* Y, int out_dtype,
                hipStream_t stream) {
  return run_fused(MXFP4_OP_FPROP, X, W, T, N, K, hadamard, scale_mode, ws, ws_bytes, Y,
                   out_dtype, stream);
}

int mxfp4_dgrad(const void* dY, const void* W, int64_t T, int64_t N, int64_t K, int hadamard,
                int scale_mode, void* ws, size_t ws_bytes, void* dX, int out_dtype,
                hipStream_t stream) {
  return run_fused(MXFP4_OP_DGRAD, dY, W, T, N, K, hadamard, scale_mode, ws, ws_bytes, dX,
                   out_dtype, stream);
}

int mxfp4_wgrad(const void* dY, const void* X, int64_t T, int64_t N, int64_t K, int hadamard,
                int scale_mode, void* ws, size_t ws_bytes, void* dW, int out_dtype,
                hipStream_t stream) {
  return run_fused(MXFP4_OP_WGRAD, dY, X, T, N, K, hadamard, scale_mode, ws, ws_bytes, dW,
                   out_dtype, stream);
}

size_t mxfp4_workspace_bytes(int op, int64_t T, int64_t N, int64_t K) {
  Plan p;
  if (!make_plan(op, T, N, K, &p)) return 0;
  return p.a.ws() + p.b.ws();
}

const char* mxfp4_status_string(int status) {
  switch (status) {
    case MXFP4_OK: return "MXFP4_OK";
    case MXFP4_ERR_NULL: return "MXFP4_ERR_NULL";
    case MXFP4_ERR_SHAPE: return "MXFP4_ERR_SHAPE";
    case MXFP4_ERR_MODE: return "MXFP4_ERR_MODE";
    case MXFP4_ERR_WORKSPACE: return "MXFP4_ERR_WORKSPACE";
    case MXFP4_ERR_HIP: return "MXFP4_ERR_HIP";
    case MXFP4_ERR_ALIGN: return "MXFP4_ERR_ALIGN";
    default: return "MXFP4_ERR_UNKNOWN";
  }
}

}  // extern "C"
