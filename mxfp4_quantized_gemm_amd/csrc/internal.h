// Internal launch interface between the host API (api.cpp) and the gfx950
// kernels (quant.hip, gemm.hip). Arguments are validated by the caller.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace mx {

// Rotate + quantize (see mxfp4_quantize in include/mxfp4.h for semantics).
hipError_t launch_quantize(const void* src, int64_t rows, int64_t cols, int axis,
                           int hadamard, int scale_mode, void* nib, void* sc,
                           hipStream_t stream);

// Two operands (as two launch_quantize calls with the same rotation and
// scale rule) in one launch where both shapes allow it, else two launches.
hipError_t launch_quantize_pair(const void* src_a, int64_t rows_a, int64_t cols_a, int axis_a,
                                void* nib_a, void* sc_a, const void* src_b, int64_t rows_b,
                                int64_t cols_b, int axis_b, void* nib_b, void* sc_b,
                                int hadamard, int scale_mode, hipStream_t stream);

// One read of src, two outputs: row-wise (rnib, rsc) and column-wise
// transposed (cnib, csc), each as launch_quantize with axis ROW / COL.
hipError_t launch_quantize_dual(const void* src, int64_t rows, int64_t cols, int hadamard,
                                int scale_mode, void* rnib, void* rsc, void* cnib, void* csc,
                                hipStream_t stream);

// Outlier-fallback operand: [Q(y) | Q((y - Q(y)) / 2)] per output row,
// 2x the nibble and scale bytes of launch_quantize (axis ROW or COL).
hipError_t launch_quantize_of(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, void* nib, void* sc, hipStream_t stream);

// Macro-block-scaled operand: launch_quantize of fl32(c y) plus one mantissa
// byte per 128 elements along the blocked axis (axis ROW or COL).
hipError_t launch_quantize_mbs(const void* src, int64_t rows, int64_t cols, int axis,
                               int hadamard, int scale_mode, void* nib, void* sc, void* mbs,
                               hipStream_t stream);

// Comparison arms: random-sign Hadamard (signs: one byte per index of the
// blocked axis, bit 0 set = flip) and stochastic rounding (rnd: one uint32
// per source element, [rows][cols]); axis ROW or COL.
hipError_t launch_quantize_rs(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, const void* signs, void* nib, void* sc,
                              hipStream_t stream);
hipError_t launch_quantize_sr(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, const void* rnd, void* nib, void* sc,
                              hipStream_t stream);

// Tensor-level error decomposition sums (mxfp4_error_stats): ws holds
// kStatsMaxGroups x 10 doubles of partial sums, out receives 10 doubles.
constexpr int kStatsMaxGroups = 1024;
hipError_t launch_error_stats(const void* src, int64_t rows, int64_t cols, int axis,
                              int hadamard, int scale_mode, void* ws, void* out,
                              hipStream_t stream);

// The same sums with the partials in a static device array of
// kStatsMaxGroups x 10 doubles per GPU (no workspace, no allocation).
hipError_t launch_error_stats_noalloc(const void* src, int64_t rows, int64_t cols, int axis,
                                      int hadamard, int scale_mode, void* out,
                                      hipStream_t stream);

// Block-scaled MXFP4 GEMM, C[M][N] = A[M][K] B[N][K]^T.
hipError_t launch_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs,
                       int64_t M, int64_t N, int64_t K, void* C, int out_dtype,
                       hipStream_t stream);

// GEMM of two macro-block-scaled operands (mantissa bytes Am [M][K/128],
// Bm [N][K/128]): C = sum over 128-k macro-blocks of the MXFP4 product times
// 1 / ((1 + mA / 256) (1 + mB / 256)). K % 128 == 0.
hipError_t launch_gemm_mbs(const void* Aq, const void* As, const void* Am, const void* Bq,
                           const void* Bs, const void* Bm, int64_t M, int64_t N, int64_t K,
                           void* C, int out_dtype, hipStream_t stream);

}  // namespace mx
