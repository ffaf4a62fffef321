// Record of the launches the C ABI asks for, filled by the host-only stand-in
// for the kernel launch layer (launch_stub.cpp).
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../mxfp4_quantized_gemm_amd/csrc/internal.h"

namespace stub {
struct Call {
  const char* what;
  const void* src;    // source (quantizers) or A nibbles (GEMM)
  int64_t d[3];       // rows, cols (quantizers) or M, N, K (GEMM)
  int i[3];           // axis, hadamard, scale mode (quantizers) or out dtype (GEMM)
  void* out[4];       // outputs in argument order (GEMM: As, Bq, Bs, C)
};
constexpr int kMaxCalls = 16;
extern Call g_calls[kMaxCalls];
// operand B of a pair launch (rows in Call::d[2], outputs in Call::out[2..3])
struct PairB {
  const void* src;
  int64_t cols;
  int axis;
};
extern PairB g_pair_b[kMaxCalls];
extern int g_ncalls;
extern hipError_t g_result;  // what every launch returns
void reset(hipError_t result);
}  // namespace stub
