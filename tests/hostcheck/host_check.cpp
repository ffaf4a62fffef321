// Host-only check of the C ABI (api.cpp) against the launch stand-in
// (launch_stub.cpp), built with the address and undefined-behaviour
// sanitizers: argument validation returns the documented status before any
// launch, a valid call launches exactly what the header describes, the fused
// products carve the caller's workspace into the two packed operands without
// overlap, and a failed launch maps to MXFP4_ERR_HIP. Exit status 0 when
// every case holds; the first failing case is printed.
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/mxfp4.h"
#include "launch_stub.h"

namespace {

int g_cases = 0;

#define CHECK(cond)                                                              \
  do {                                                                           \
    ++g_cases;                                                                   \
    if (!(cond)) {                                                               \
      fprintf(stderr, "host_check: %s:%d: failed: %s\n", __FILE__, __LINE__, #cond); \
      exit(1);                                                                   \
    }                                                                            \
  } while (0)

// Stand-in device addresses: never dereferenced by the ABI or the stand-in.
alignas(256) unsigned char g_mem[1 << 16];
void* at(size_t off) { return g_mem + off; }

size_t r256(size_t x) { return (x + 255) & ~size_t(255); }

void quantize_cases() {
  void* src = at(0);
  void* nib = at(4096);
  void* sc = at(8192);
  stub::reset(hipSuccess);
  CHECK(mxfp4_quantize(src, 64, 64, 3, 16, 0, nib, sc, nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_quantize(src, 64, 64, 0, 8, 0, nib, sc, nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_quantize(src, 64, 64, 0, 16, 2, nib, sc, nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_quantize(src, 64, 48, 0, 16, 0, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(src, 48, 64, 1, 16, 0, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(src, 48, 64, 2, 16, 0, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(src, -1, 64, 0, 16, 0, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(src, int64_t(1) << 31, 64, 0, 16, 0, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(src, int64_t(1) << 30, int64_t(1) << 30, 0, 16, 0, nib, sc, nullptr) ==
        MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize(nullptr, 64, 64, 0, 16, 0, nib, sc, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize(src, 64, 64, 0, 16, 0, nullptr, sc, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize(src, 64, 64, 0, 16, 0, nib, nullptr, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize(at(8), 64, 64, 0, 16, 0, nib, sc, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_quantize(src, 64, 64, 0, 16, 0, at(4100), sc, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(stub::g_ncalls == 0);
  // empty matrices are valid and launch nothing, even with null pointers
  CHECK(mxfp4_quantize(nullptr, 0, 64, 0, 16, 0, nullptr, nullptr, nullptr) == MXFP4_OK);
  CHECK(mxfp4_quantize(nullptr, 64, 0, 1, 16, 0, nullptr, nullptr, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_quantize(src, 96, 64, 1, 32, 1, nib, sc, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 1 && strcmp(stub::g_calls[0].what, "quantize") == 0);
  CHECK(stub::g_calls[0].src == src && stub::g_calls[0].d[0] == 96 && stub::g_calls[0].d[1] == 64);
  CHECK(stub::g_calls[0].i[0] == 1 && stub::g_calls[0].i[1] == 32 && stub::g_calls[0].i[2] == 1);
  CHECK(stub::g_calls[0].out[0] == nib && stub::g_calls[0].out[1] == sc);
  stub::reset(hipErrorInvalidValue);
  CHECK(mxfp4_quantize(src, 64, 64, 0, 16, 0, nib, sc, nullptr) == MXFP4_ERR_HIP);

  // variants: axis restrictions and their extra arguments
  stub::reset(hipSuccess);
  CHECK(mxfp4_quantize_of(src, 64, 64, 2, 16, 0, nib, sc, nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_quantize_mbs(src, 64, 64, 0, 16, 0, nib, sc, at(12288), nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize_mbs(src, 64, 128, 0, 16, 0, nib, sc, nullptr, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize_rs(src, 64, 64, 0, 16, 0, nullptr, nib, sc, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize_rs(src, 64, 64, 0, 16, 0, at(12289), nib, sc, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_quantize_sr(src, 64, 64, 0, 16, 0, at(12292), nib, sc, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_quantize_dual(src, 64, 48, 16, 0, nib, sc, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize_dual(src, 48, 64, 16, 0, nib, sc, nib, sc, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_quantize_mbs(src, 128, 256, 1, 16, 1, nib, sc, at(12288), nullptr) == MXFP4_OK);
  CHECK(mxfp4_quantize_dual(src, 64, 96, 0, 0, nib, sc, at(16384), at(20480), nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 2 && stub::g_calls[0].out[2] == at(12288));
  CHECK(stub::g_calls[1].out[2] == at(16384) && stub::g_calls[1].out[3] == at(20480));

  // error statistics: workspace size and alignment
  double* out = reinterpret_cast<double*>(at(24576));
  stub::reset(hipSuccess);
  CHECK(mxfp4_error_stats(src, 64, 64, 0, 16, 0, at(32768), MXFP4_ERROR_STATS_WS_BYTES - 1, out,
                          nullptr) == MXFP4_ERR_WORKSPACE);
  CHECK(mxfp4_error_stats(src, 64, 64, 0, 16, 0, at(32772), MXFP4_ERROR_STATS_WS_BYTES, out,
                          nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_error_stats(src, 64, 64, 2, 16, 0, at(32768), MXFP4_ERROR_STATS_WS_BYTES, out,
                          nullptr) == MXFP4_ERR_MODE);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_error_stats(src, 64, 64, 1, 16, 0, at(32768), MXFP4_ERROR_STATS_WS_BYTES, out,
                          nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 1 && stub::g_calls[0].out[1] == out);
  // the variant without a workspace: same checks on the source, out_stats
  // 8-byte aligned, no workspace argument
  stub::reset(hipSuccess);
  CHECK(mxfp4_error_stats_noalloc(src, 64, 64, 2, 16, 0, out, nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_error_stats_noalloc(src, 64, 48, 0, 16, 0, out, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_error_stats_noalloc(src, 64, 64, 0, 16, 0, nullptr, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_error_stats_noalloc(nullptr, 64, 64, 0, 16, 0, out, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_error_stats_noalloc(src, 64, 64, 0, 16, 0, reinterpret_cast<double*>(at(24580)),
                                  nullptr) == MXFP4_ERR_ALIGN);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_error_stats_noalloc(nullptr, 0, 64, 0, 16, 0, reinterpret_cast<double*>(at(24584)),
                                  nullptr) == MXFP4_OK);
  CHECK(mxfp4_error_stats_noalloc(src, 32, 64, 1, 32, 1, out, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 2 && strcmp(stub::g_calls[1].what, "stats_noalloc") == 0);
  CHECK(stub::g_calls[1].out[0] == out && stub::g_calls[1].i[1] == 32);

  // two operands in one call: each validated as mxfp4_quantize, A first
  void* src2 = at(36864);
  void* nib2 = at(40960);
  void* sc2 = at(45056);
  stub::reset(hipSuccess);
  CHECK(mxfp4_quantize_pair(src, 64, 64, 2, nib, sc, src2, 64, 64, 0, nib2, sc2, 16, 0,
                            nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_quantize_pair(src, 64, 48, 0, nib, sc, src2, 64, 64, 0, nib2, sc2, 16, 0,
                            nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize_pair(src, 64, 64, 0, nib, sc, src2, 48, 64, 1, nib2, sc2, 16, 0,
                            nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_quantize_pair(src, 64, 64, 0, nib, sc, nullptr, 64, 64, 1, nib2, sc2, 16, 0,
                            nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_quantize_pair(src, 64, 64, 0, nib, sc, src2, 64, 64, 1, at(40961), sc2, 16, 0,
                            nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_quantize_pair(src, 64, 64, 0, nib, sc, src2, 64, 64, 1, nib2, sc2, 12, 0,
                            nullptr) == MXFP4_ERR_MODE);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_quantize_pair(nullptr, 0, 64, 0, nullptr, nullptr, nullptr, 64, 0, 1, nullptr,
                            nullptr, 16, 0, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_quantize_pair(nullptr, 0, 64, 0, nullptr, nullptr, src2, 64, 96, 1, nib2, sc2, 32,
                            1, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 1 && strcmp(stub::g_calls[0].what, "quantize") == 0 &&
        stub::g_calls[0].src == src2 && stub::g_calls[0].i[0] == 1);
  CHECK(mxfp4_quantize_pair(src, 64, 96, 0, nib, sc, src2, 128, 64, 1, nib2, sc2, 16, 1,
                            nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 2 && strcmp(stub::g_calls[1].what, "pair") == 0);
  CHECK(stub::g_calls[1].d[0] == 64 && stub::g_calls[1].d[1] == 96 && stub::g_calls[1].d[2] == 128);
  CHECK(stub::g_pair_b[1].src == src2 && stub::g_pair_b[1].cols == 64 && stub::g_pair_b[1].axis == 1);
  CHECK(stub::g_calls[1].out[2] == nib2 && stub::g_calls[1].out[3] == sc2);
}

void gemm_cases() {
  void* a = at(0);
  void* as = at(4096);
  void* b = at(8192);
  void* bs = at(12288);
  void* c = at(16384);
  stub::reset(hipSuccess);
  CHECK(mxfp4_gemm(a, as, b, bs, 0, 32, 64, c, 0, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 0, 64, c, 0, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 48, c, 0, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 0, c, 0, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 64, c, 2, nullptr) == MXFP4_ERR_MODE);
  CHECK(mxfp4_gemm(a, nullptr, b, bs, 32, 32, 64, c, 0, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 64, nullptr, 0, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_gemm(at(8), as, b, bs, 32, 32, 64, c, 0, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 64, at(16386), 0, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 64, at(16385), 1, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_gemm(a, as, b, bs, 130, 70, 96, at(16386), 1, nullptr) == MXFP4_OK);
  const stub::Call& g = stub::g_calls[0];
  CHECK(stub::g_ncalls == 1 && strcmp(g.what, "gemm") == 0 && g.src == a);
  CHECK(g.d[0] == 130 && g.d[1] == 70 && g.d[2] == 96 && g.i[0] == 1);
  CHECK(g.out[0] == as && g.out[1] == b && g.out[2] == bs && g.out[3] == at(16386));
  stub::reset(hipErrorLaunchFailure);
  CHECK(mxfp4_gemm(a, as, b, bs, 32, 32, 64, c, 0, nullptr) == MXFP4_ERR_HIP);
  // the macro-block-scaled product: K % 128, both mantissa arrays
  void* am = at(20480);
  void* bm = at(20481);
  stub::reset(hipSuccess);
  CHECK(mxfp4_gemm_mbs(a, as, am, b, bs, bm, 32, 32, 96, c, 0, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(mxfp4_gemm_mbs(a, as, nullptr, b, bs, bm, 32, 32, 128, c, 0, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_gemm_mbs(a, as, am, b, bs, nullptr, 32, 32, 128, c, 0, nullptr) == MXFP4_ERR_NULL);
  CHECK(mxfp4_gemm_mbs(a, as, am, b, bs, bm, 32, 32, 128, at(16386), 0, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(mxfp4_gemm_mbs(a, as, am, b, bs, bm, 0, 32, 128, c, 0, nullptr) == MXFP4_ERR_SHAPE);
  CHECK(stub::g_ncalls == 0);
  CHECK(mxfp4_gemm_mbs(a, as, am, b, bs, bm, 33, 70, 384, c, 1, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 1 && strcmp(stub::g_calls[0].what, "gemm_mbs") == 0);
  CHECK(stub::g_calls[0].d[0] == 33 && stub::g_calls[0].d[1] == 70 && stub::g_calls[0].d[2] == 384);
  CHECK(stub::g_calls[0].i[0] == 1 && stub::g_calls[0].i[1] == 1);
}

// One fused product: the two-operand quantize launch and the GEMM, with the
// workspace carved as A nibbles | A scales | B nibbles | B scales, each part
// rounded up to 256 bytes.
void fused_case(int op, int64_t T, int64_t N, int64_t K) {
  alignas(256) static unsigned char ws[1 << 20];
  void* P = at(0);
  void* Q = at(4096);
  void* Y = at(8192);
  const size_t need = mxfp4_workspace_bytes(op, T, N, K);
  CHECK(need > 0 && need <= sizeof(ws));
  auto fn = op == MXFP4_OP_FPROP ? mxfp4_fprop : op == MXFP4_OP_DGRAD ? mxfp4_dgrad : mxfp4_wgrad;
  stub::reset(hipSuccess);
  CHECK(fn(P, Q, T, N, K, 16, 0, ws, need - 1, Y, 0, nullptr) == MXFP4_ERR_WORKSPACE);
  CHECK(fn(P, Q, T, N, K, 16, 0, ws + 16, need, Y, 0, nullptr) == MXFP4_ERR_ALIGN);
  CHECK(fn(P, Q, T, N, K, 16, 0, nullptr, need, Y, 0, nullptr) == MXFP4_ERR_NULL);
  CHECK(fn(P, Q, T, N, K, 12, 0, ws, need, Y, 0, nullptr) == MXFP4_ERR_MODE);
  CHECK(stub::g_ncalls == 0);
  CHECK(fn(P, Q, T, N, K, 16, 1, ws, need, Y, 1, nullptr) == MXFP4_OK);
  CHECK(stub::g_ncalls == 2 && strcmp(stub::g_calls[0].what, "pair") == 0);
  const stub::Call& q = stub::g_calls[0];
  const stub::PairB& pb = stub::g_pair_b[0];
  const stub::Call& g = stub::g_calls[1];
  // source shapes and axes of the two operands, GEMM sizes
  int64_t ar, ac, br, bc, M, NN, KK;
  int aax, bax;
  if (op == MXFP4_OP_FPROP) {
    ar = T; ac = K; aax = 0; br = N; bc = K; bax = 0; M = T; NN = N; KK = K;
  } else if (op == MXFP4_OP_DGRAD) {
    ar = T; ac = N; aax = 0; br = N; bc = K; bax = 1; M = T; NN = K; KK = N;
  } else {
    ar = T; ac = N; aax = 1; br = T; bc = K; bax = 1; M = N; NN = K; KK = T;
  }
  CHECK(q.src == P && q.d[0] == ar && q.d[1] == ac && q.i[0] == aax);
  CHECK(pb.src == Q && q.d[2] == br && pb.cols == bc && pb.axis == bax);
  CHECK(q.i[1] == 16 && q.i[2] == 1);
  CHECK(g.d[0] == M && g.d[1] == NN && g.d[2] == KK && g.i[0] == 1 && g.out[3] == Y);
  const size_t anib = size_t(M) * size_t(KK / 2), asc = size_t(M) * size_t(KK / 32);
  const size_t bnib = size_t(NN) * size_t(KK / 2), bsc = size_t(NN) * size_t(KK / 32);
  unsigned char* w = ws;
  CHECK(q.out[0] == w && q.out[1] == w + r256(anib));
  CHECK(q.out[2] == w + r256(anib) + r256(asc));
  CHECK(q.out[3] == w + r256(anib) + r256(asc) + r256(bnib));
  CHECK(need == r256(anib) + r256(asc) + r256(bnib) + r256(bsc));
  CHECK(g.src == q.out[0] && g.out[0] == q.out[1] && g.out[1] == q.out[2] &&
        g.out[2] == q.out[3]);
  // a failed first launch stops the product
  stub::reset(hipErrorInvalidValue);
  CHECK(fn(P, Q, T, N, K, 16, 0, ws, need, Y, 0, nullptr) == MXFP4_ERR_HIP);
  CHECK(stub::g_ncalls == 1);
}

}  // namespace

int main() {
  quantize_cases();
  gemm_cases();
  fused_case(MXFP4_OP_FPROP, 96, 160, 224);
  fused_case(MXFP4_OP_DGRAD, 96, 160, 224);
  fused_case(MXFP4_OP_WGRAD, 96, 160, 224);
  fused_case(MXFP4_OP_FPROP, 33, 7, 64);
  fused_case(MXFP4_OP_WGRAD, 64, 5, 9);
  CHECK(mxfp4_workspace_bytes(MXFP4_OP_DGRAD, 10, 33, 10) == 0);
  CHECK(mxfp4_workspace_bytes(7, 32, 32, 32) == 0);
  CHECK(strcmp(mxfp4_status_string(MXFP4_ERR_HIP), "MXFP4_ERR_HIP") == 0);
  CHECK(strcmp(mxfp4_status_string(-3), "MXFP4_ERR_UNKNOWN") == 0);
  printf("host_check: %d checks passed\n", g_cases);
  return 0;
}
