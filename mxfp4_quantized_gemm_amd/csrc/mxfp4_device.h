// Device-side building blocks shared by the quantizer (quant.hip) and the
// error-statistics kernels (stats.hip): bf16 widening, the fixed fp32
// Hadamard butterfly, the block amax, the E8M0 rules and the E2M1 encode.
// Pages: [P1] "Pretraining Large Language Models with MXFP4 on Native FP4
// Hardware" (arXiv:2605.09825 summary), sections A.1 and A.2; [P3]
// "Decomposing MXFP4 quantization error" blog (arXiv:2605.20402),
// pain-point and core-insight sections.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mx {
namespace {

constexpr int kOcpFloor = 0;
constexpr int kCeil = 1;

__device__ __forceinline__ float bf16lo(uint32_t d) { return __uint_as_float(d << 16); }
__device__ __forceinline__ float bf16hi(uint32_t d) { return __uint_as_float(d & 0xffff0000u); }

// fp32 Walsh-Hadamard butterfly on every aligned group of H values of v[32]:
// for s = 1, 2, 4, ... H/2 each pair (i, i+s) with (i & s) == 0 becomes
// (a + b, a - b); then one multiply by 1/4 (H16) or RN(2^-2.5) (H32).
// The order of operations is part of the definition; every add is one
// fp32 round-to-nearest-even step (no reassociation, no contraction).
template <int H>
__device__ __forceinline__ void hadamard32(float (&v)[32]) {
  if constexpr (H != 0) {
#pragma unroll
    for (int s = 1; s < H; s <<= 1) {
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        if ((i & s) == 0) {
          const float a = v[i], b = v[i + s];
          v[i] = a + b;
          v[i + s] = a - b;
        }
      }
    }
    const float c = (H == 16) ? 0.25f : __uint_as_float(0x3E3504F3u);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] *= c;
  }
}

// Largest |v| as fp32 bits. Integer max over the sign-cleared patterns is
// exact and orders NaN (> 0x7f800000) above +Inf above every finite value.
__device__ __forceinline__ uint32_t amax_bits32(const float (&v)[32]) {
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 32; ++i) m = max(m, __float_as_uint(v[i]) & 0x7fffffffu);
  return m;
}

// E8M0 byte (E + 127) of a block whose amax has fp32 bits `a`; 0xFF when the
// block holds a non-finite value. amax = m * 2^e, m in [1, 2):
// ocp_floor E = e - 2; ceil E = e - 2 + (m > 1.5). A zero or subnormal amax
// (e <= -127) lands below the clamp, so E = -127. E never exceeds 126.
template <int MODE>
__device__ __forceinline__ uint32_t e8m0_byte(uint32_t a) {
  if (a >= 0x7f800000u) return 255u;
  const int be = (int)(a >> 23);
  int E = be - 129;
  if (MODE == kCeil && (a & 0x7fffffu) > 0x400000u) E += 1;
  if (be == 0) E = -127;
  E = max(E, -127);
  return (uint32_t)(E + 127);
}

// 2^(byte - 127) as fp32 (byte 0 is the subnormal 2^-127).
__device__ __forceinline__ float scale_of_byte(uint32_t s) {
  return s ? __uint_as_float(s << 23) : __uint_as_float(0x00400000u);
}

// 32 rotated values -> 16 bytes of packed E2M1 (element 2j in the low
// nibble of byte j). The convert returns code(x / scale) with RNE ties
// and saturation; its op_sel picks the destination byte.
__device__ __forceinline__ uint4 encode32(const float (&v)[32], float scale) {
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t r = 0;
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 0], v[8 * d + 1], scale, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 2], v[8 * d + 3], scale, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 4], v[8 * d + 5], scale, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * d + 6], v[8 * d + 7], scale, 3);
    w[d] = r;
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void unpack64B(const uint4 (&q)[4], float (&v)[32]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t d[4] = {q[j].x, q[j].y, q[j].z, q[j].w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * j + 2 * k] = bf16lo(d[k]);
      v[8 * j + 2 * k + 1] = bf16hi(d[k]);
    }
  }
}

template <int MODE>
__device__ __forceinline__ void encode_block(const float (&v)[32], uint4& nib, uint32_t& s) {
  s = e8m0_byte<MODE>(amax_bits32(v));
  nib = (s == 255u) ? make_uint4(0, 0, 0, 0) : encode32(v, scale_of_byte(s));
}

}  // namespace
}  // namespace mx
