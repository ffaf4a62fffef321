// Host-only stand-in for the kernel launch layer (internal.h): every launch
// records its arguments and returns hipSuccess, so the C ABI's validation and
// workspace carving run on the CPU, without a GPU, under the address and
// undefined-behaviour sanitizers. Nothing here touches device memory.
#include "launch_stub.h"

namespace stub {
Call g_calls[kMaxCalls];
PairB g_pair_b[kMaxCalls];
int g_ncalls = 0;
hipError_t g_result = hipSuccess;

void reset(hipError_t result) {
  g_ncalls = 0;
  g_result = result;
}

hipError_t record(const char* what, const void* src, int64_t rows, int64_t cols, int axis,
                  int hadamard, int mode, void* out0, void* out1, void* out2, void* out3) {
  if (g_ncalls < kMaxCalls)
    g_calls[g_ncalls] = {what, src, {rows, cols, 0}, {axis, hadamard, mode},
                         {out0, out1, out2, out3}};
  ++g_ncalls;
  return g_result;
}
}  // namespace stub

namespace mx {

hipError_t launch_quantize(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                           int scale_mode, void* nib, void* sc, hipStream_t) {
  return stub::record("quantize", src, rows, cols, axis, hadamard, scale_mode, nib, sc, nullptr,
                      nullptr);
}

hipError_t launch_quantize_pair(const void* src_a, int64_t rows_a, int64_t cols_a, int axis_a,
                                void* nib_a, void* sc_a, const void* src_b, int64_t rows_b,
                                int64_t cols_b, int axis_b, void* nib_b, void* sc_b,
                                int hadamard, int scale_mode, hipStream_t) {
  const hipError_t r = stub::record("pair", src_a, rows_a, cols_a, axis_a, hadamard, scale_mode,
                                    nib_a, sc_a, nib_b, sc_b);
  if (stub::g_ncalls <= stub::kMaxCalls) {
    stub::g_calls[stub::g_ncalls - 1].d[2] = rows_b;
    stub::g_pair_b[stub::g_ncalls - 1] = {src_b, cols_b, axis_b};
  }
  return r;
}

hipError_t launch_quantize_dual(const void* src, int64_t rows, int64_t cols, int hadamard,
                                int scale_mode, void* rnib, void* rsc, void* cnib, void* csc,
                                hipStream_t) {
  return stub::record("dual", src, rows, cols, -1, hadamard, scale_mode, rnib, rsc, cnib, csc);
}

hipError_t launch_quantize_of(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, void* nib, void* sc, hipStream_t) {
  return stub::record("of", src, rows, cols, axis, hadamard, scale_mode, nib, sc, nullptr,
                      nullptr);
}

hipError_t launch_quantize_mbs(const void* src, int64_t rows, int64_t cols, int axis,
                               int hadamard, int scale_mode, void* nib, void* sc, void* mbs,
                               hipStream_t) {
  return stub::record("mbs", src, rows, cols, axis, hadamard, scale_mode, nib, sc, mbs, nullptr);
}

hipError_t launch_quantize_rs(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, const void* signs, void* nib, void* sc,
                              hipStream_t) {
  return stub::record("rs", src, rows, cols, axis, hadamard, scale_mode, nib, sc,
                      const_cast<void*>(signs), nullptr);
}

hipError_t launch_quantize_sr(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, const void* rnd, void* nib, void* sc, hipStream_t) {
  return stub::record("sr", src, rows, cols, axis, hadamard, scale_mode, nib, sc,
                      const_cast<void*>(rnd), nullptr);
}

hipError_t launch_error_stats(const void* src, int64_t rows, int64_t cols, int axis,
                              int hadamard, int scale_mode, void* ws, void* out, hipStream_t) {
  return stub::record("stats", src, rows, cols, axis, hadamard, scale_mode, ws, out, nullptr,
                      nullptr);
}

hipError_t launch_error_stats_noalloc(const void* src, int64_t rows, int64_t cols, int axis,
                                      int hadamard, int scale_mode, void* out, hipStream_t) {
  return stub::record("stats_noalloc", src, rows, cols, axis, hadamard, scale_mode, out, nullptr,
                      nullptr, nullptr);
}

hipError_t launch_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs, int64_t M,
                       int64_t N, int64_t K, void* C, int out_dtype, hipStream_t) {
  const hipError_t r = stub::record("gemm", Aq, M, N, out_dtype, 0, 0, const_cast<void*>(As),
                                    const_cast<void*>(Bq), const_cast<void*>(Bs), C);
  if (stub::g_ncalls <= stub::kMaxCalls) stub::g_calls[stub::g_ncalls - 1].d[2] = K;
  return r;
}

hipError_t launch_gemm_mbs(const void* Aq, const void* As, const void* Am, const void* Bq,
                           const void* Bs, const void* Bm, int64_t M, int64_t N, int64_t K,
                           void* C, int out_dtype, hipStream_t) {
  const hipError_t r = stub::record("gemm_mbs", Aq, M, N, out_dtype, 0, 0, const_cast<void*>(As),
                                    const_cast<void*>(Bq), const_cast<void*>(Bs), C);
  if (stub::g_ncalls <= stub::kMaxCalls) {
    stub::g_calls[stub::g_ncalls - 1].d[2] = K;
    stub::g_calls[stub::g_ncalls - 1].i[1] = Am != nullptr && Bm != nullptr;
  }
  return r;
}

}  // namespace mx
