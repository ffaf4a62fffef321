// Tensor-level MXFP4 error decomposition for gfx950 (MI355X).
//
// Page cited: [P3] "Decomposing MXFP4 quantization error" blog
// (arXiv:2605.20402): core-insight section (ideal scale s* = m_b / 6, the
// error of a block split as e = e_scale + e_DZ + e_grid with the deadzone
// D = {i : |x_i| < m_b / 24}), Property 1 (orthogonality of e_DZ, the MSE
// identity with one cross term) and the deadzone share it reports for
// weights. The quantized values are those of [P1] "Pretraining Large
// Language Models with MXFP4 on Native FP4 Hardware" (arXiv:2605.09825
// summary), sections A.1/A.2: the operand is rotated, then blocked.
//
// One pass over the bf16 source. Each thread takes whole 32-element blocks
// (1x32 along cols or 32x1 down rows), rotates them with the same fp32
// butterfly as the quantizer, takes E8M0 and the E2M1 codes from the same
// instructions, and then, per element in fp64:
//   Q  = code value * 2^E                      (what the packed operand holds)
//   s* = m_b / 6,  Q* = s* * grid(x / s*)      (ideal scale, nearest grid value,
//                                                ties to the even code, clamp 6)
//   deadzone: 24 |x| < m_b
//   e_scale = Q - Q*,  e_DZ = (Q* - x) in the deadzone, e_grid = (Q* - x) outside
// and accumulates ten sums (see mxfp4_error_stats in include/mxfp4.h).
// Blocks holding a non-finite rotated value are skipped and counted.
// Partial sums per work-group go to a workspace; a second one-work-group
// kernel adds them in a fixed order, so the result is deterministic.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "internal.h"
#include "mxfp4_device.h"

namespace mx {
namespace {

constexpr int kStats = 10;
constexpr int kThreads = 256;

// Nearest E2M1 grid value of t (ties to the even code, clamp at 6) as a
// chain of selects on |t|; the grid values differ only in their upper
// dword, so each select is one 32-bit move. The sign is t's.
__device__ __forceinline__ double grid_of(double t) {
  const double a = fabs(t);
  double g = 0.0;
  g = a > 0.25 ? 0.5 : g;
  g = a >= 0.75 ? 1.0 : g;
  g = a > 1.25 ? 1.5 : g;
  g = a >= 1.75 ? 2.0 : g;
  g = a > 2.5 ? 3.0 : g;
  g = a >= 3.5 ? 4.0 : g;
  g = a > 5.0 ? 6.0 : g;
  return copysign(g, t);
}

typedef float st_f32x2 __attribute__((ext_vector_type(2)));

// Per element, in fp64: Q from the code (the scaled FP4-to-fp32 convert at
// scale 1 gives the E2M1 value exactly; times 2^E in fp64), t = x / s*
// (one correctly rounded fp64 division), Q* = s* grid(t), the
// deadzone test and the terms; each sum takes one fused multiply-add per
// element. Every branch depends only on the block (non-finite, s* = 0), so
// the per-element work is straight-line code.
template <int MODE>
__device__ __forceinline__ void block_stats(const float (&v)[32], double (&acc)[kStats]) {
  const uint32_t am = amax_bits_n<32>(v);
  if (am >= 0x7f800000u) {
    acc[9] += 1.0;
    return;
  }
  const uint32_t sb = e8m0_byte<MODE>(am);
  const uint4 nib = encode32(v, scale_of_byte(sb));
  // 2^(sb - 127) as fp64 (sb - 127 >= -127 is a normal fp64 exponent)
  const double p2 = __longlong_as_double((long long)((int64_t)(sb + 896u) << 52));
  const double mb = (double)__uint_as_float(am);
  const double ss = mb / 6.0;
  // s* = 0 only for an all-zero block, whose t is 0 (x / 1)
  const double sd = ss > 0.0 ? ss : 1.0;
  const uint32_t w[4] = {nib.x, nib.y, nib.z, nib.w};
  double nd = 0.0;
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    st_f32x2 cvs[4];
    cvs[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 0);
    cvs[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 1);
    cvs[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 2);
    cvs[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], 1.0f, 3);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const st_f32x2 cv = cvs[k];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int i = 8 * d + 2 * k + h;
        const double x = (double)v[i];
        const double q = (double)(h ? cv.y : cv.x) * p2;
        const double qs = ss * grid_of(x / sd);
        const bool dz = 24.0 * fabs(x) < mb;
        const double es = q - qs, r = qs - x, e = q - x;
        const double edz = dz ? r : 0.0, eg = dz ? 0.0 : r;
        acc[0] = fma(es, es, acc[0]);
        acc[1] = fma(edz, edz, acc[1]);
        acc[2] = fma(eg, eg, acc[2]);
        acc[3] = fma(es, eg, acc[3]);
        acc[4] = fma(es, edz, acc[4]);
        acc[5] = fma(e, e, acc[5]);
        acc[6] = fma(x, x, acc[6]);
        nd += dz ? 1.0 : 0.0;
      }
    }
  }
  acc[7] += nd;
  acc[8] += 32.0;
}

// AXIS 0: block b = elements [32 b, 32 b + 32) of the flat row-major array.
// AXIS 1: block b = column b % cols, rows [32 (b / cols), +32).
template <int H, int MODE, int AXIS>
__global__ __launch_bounds__(kThreads) void error_stats_kernel(const uint16_t* __restrict__ src,
                                                               int64_t rows, int64_t cols,
                                                               double* __restrict__ part) {
  double acc[kStats];
#pragma unroll
  for (int k = 0; k < kStats; ++k) acc[k] = 0.0;
  const int64_t nblk = rows * cols / 32;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x; b < nblk; b += stride) {
    float v[32];
    if (AXIS == 0) {
      const uint4* p = reinterpret_cast<const uint4*>(src) + b * 4;
      uint4 q[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) q[j] = p[j];
      unpack64B(q, v);
    } else {
      const int64_t c = b % cols, band = b / cols;
      const uint16_t* p = src + band * 32 * cols + c;
#pragma unroll
      for (int r = 0; r < 32; ++r) v[r] = __uint_as_float((uint32_t)p[r * cols] << 16);
    }
    hadamard32<H>(v);
    block_stats<MODE>(v, acc);
  }
  // fixed-order reduction: lanes (xor tree), then the four waves in order
  __shared__ double red[kThreads / 64][kStats];
#pragma unroll
  for (int k = 0; k < kStats; ++k) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) acc[k] += __shfl_xor(acc[k], o);
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (lane == 0) {
#pragma unroll
    for (int k = 0; k < kStats; ++k) red[wave][k] = acc[k];
  }
  __syncthreads();
  if (threadIdx.x < kStats) {
    double s = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) s += red[w][threadIdx.x];
    part[(int64_t)blockIdx.x * kStats + threadIdx.x] = s;
  }
}

// One work-group: thread t adds partials t, t + 256, ... in order, then a
// fixed pairwise tree over the 256 threads.
__global__ __launch_bounds__(kThreads) void error_stats_final(const double* __restrict__ part,
                                                              int nparts, double* __restrict__ out) {
  __shared__ double red[kThreads][kStats];
  double acc[kStats];
#pragma unroll
  for (int k = 0; k < kStats; ++k) acc[k] = 0.0;
  for (int i = threadIdx.x; i < nparts; i += kThreads) {
#pragma unroll
    for (int k = 0; k < kStats; ++k) acc[k] += part[(int64_t)i * kStats + k];
  }
#pragma unroll
  for (int k = 0; k < kStats; ++k) red[threadIdx.x][k] = acc[k];
  __syncthreads();
  for (int s = kThreads / 2; s >= 1; s >>= 1) {
    if ((int)threadIdx.x < s) {
#pragma unroll
      for (int k = 0; k < kStats; ++k) red[threadIdx.x][k] += red[threadIdx.x + s][k];
    }
    __syncthreads();
  }
  if (threadIdx.x < kStats) out[threadIdx.x] = red[0][threadIdx.x];
}

template <int H, int MODE>
hipError_t dispatch_stats(const void* src, int64_t rows, int64_t cols, int axis, double* part,
                          double* out, hipStream_t st) {
  const int64_t nblk = rows * cols / 32;
  const int64_t want = (nblk + kThreads - 1) / kThreads;
  const int grid = (int)(want < kStatsMaxGroups ? want : kStatsMaxGroups);
  if (grid == 0) {  // empty input: the final pass writes zeros
    hipLaunchKernelGGL(error_stats_final, dim3(1), dim3(kThreads), 0, st, part, 0, out);
    return hipGetLastError();
  }
  if (axis == 0)
    hipLaunchKernelGGL((error_stats_kernel<H, MODE, 0>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(src), rows, cols, part);
  else
    hipLaunchKernelGGL((error_stats_kernel<H, MODE, 1>), dim3(grid), dim3(kThreads), 0, st,
                       static_cast<const uint16_t*>(src), rows, cols, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(error_stats_final, dim3(1), dim3(kThreads), 0, st, part, grid, out);
  return hipGetLastError();
}

template <int H>
hipError_t dispatch_stats_mode(const void* src, int64_t rows, int64_t cols, int axis, int mode,
                               double* part, double* out, hipStream_t st) {
  return mode == kCeil ? dispatch_stats<H, kCeil>(src, rows, cols, axis, part, out, st)
                       : dispatch_stats<H, kOcpFloor>(src, rows, cols, axis, part, out, st);
}

// Partial sums of mxfp4_error_stats_noalloc: one row of kStats doubles per
// work-group of the first pass, whose grid never exceeds kStatsMaxGroups.
// Every GPU holds its own copy for the life of the process. Host code never
// uses this name as an address (on the host it is only a stand-in for the
// symbol): it looks the device address up once per device.
static __device__ __align__(256) double scratch[kStatsMaxGroups * kStats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
double* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the current device, looked up on the first
// call on that device and kept.
hipError_t scratch_of_current_device(double** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = static_cast<double*>(p);
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace

hipError_t launch_error_stats_noalloc(const void* src, int64_t rows, int64_t cols, int axis,
                                      int hadamard, int scale_mode, void* out,
                                      hipStream_t stream) {
  double* part = nullptr;
  const hipError_t e = scratch_of_current_device(&part);
  if (e != hipSuccess) return e;
  return launch_error_stats(src, rows, cols, axis, hadamard, scale_mode, part, out, stream);
}

hipError_t launch_error_stats(const void* src, int64_t rows, int64_t cols, int axis,
                              int hadamard, int scale_mode, void* ws, void* out,
                              hipStream_t stream) {
  auto* part = static_cast<double*>(ws);
  auto* o = static_cast<double*>(out);
  switch (hadamard) {
    case 16: return dispatch_stats_mode<16>(src, rows, cols, axis, scale_mode, part, o, stream);
    case 32: return dispatch_stats_mode<32>(src, rows, cols, axis, scale_mode, part, o, stream);
    default: return dispatch_stats_mode<0>(src, rows, cols, axis, scale_mode, part, o, stream);
  }
}

}  // namespace mx
