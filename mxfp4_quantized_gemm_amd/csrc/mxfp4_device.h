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

// ------------------------------------------ H16 with the 1/4 folded into E
// The H16 normalisation 1/4 is a power of two, so it can move from the
// values into the scale: with u the unnormalised butterfly output and
// y = u / 4, every finite |u| is a multiple of 2^-133 (a bf16 quantum)
// and below 2^128, so y is exact (a non-finite u gives the same 0xFF block
// either way), amax(y) = amax(u) / 4 exactly, and
// code(y / 2^E) = code(u / 2^(E+2)). Kernels that quantize without keeping
// y therefore skip the multiply (one VALU op per element) and use the
// helpers below with SH = 2 (SH = 0 for H32 and H0, whose values are the
// rotated values themselves). The result is bit-identical to the
// normalise-then-quantize order.
template <int H>
constexpr int kScaleShift = (H == 16) ? 2 : 0;

// E8M0 byte of a block whose stored values are 2^SH times the rotated
// values and whose stored amax has fp32 bits `a`. With SH = 2 the amax of
// the rotated values is a / 4: its exponent is two lower (or it is
// subnormal and lands on the clamp, as does every e <= -127 here) and its
// mantissa is unchanged, so the e8m0_byte rules apply to the shifted
// exponent.
template <int MODE, int SH>
__device__ __forceinline__ uint32_t e8m0_byte_sh(uint32_t a) {
  if (a >= 0x7f800000u) return 255u;
  int E = (int)(a >> 23) - 129 - SH;
  if (MODE == kCeil && (a & 0x7fffffu) > 0x400000u) E += 1;
  E = max(E, -127);
  return (uint32_t)(E + 127);
}

// The convert's divisor for byte s of values stored at 2^SH times their
// rotated value: 2^(s - 127 + SH). With SH = 2 and finite stored values the
// byte is at most 251, so the divisor is a normal fp32 power of two.
template <int SH>
__device__ __forceinline__ float cvt_scale(uint32_t s) {
  if constexpr (SH == 0)
    return scale_of_byte(s);
  else
    return __uint_as_float((s + SH) << 23);
}

// Butterfly of hadamard32 with H32's multiply but without H16's 1/4.
template <int H>
__device__ __forceinline__ void butterfly32(float (&v)[32]) {
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
    if constexpr (H == 32) {
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] *= __uint_as_float(0x3E3504F3u);
    }
  }
}

// Largest |v| of N values as fp32 bits, ordered as amax_bits32 (NaN above
// +Inf above every finite value) with one three-input max per two values
// and no sign masking per value: the unsigned max of the raw bits is the
// largest negative magnitude (sign bit set) whenever a value is negative,
// the signed max (floored at 0) the largest non-negative one.
template <int N>
__device__ __forceinline__ uint32_t amax_bits_n(const float* v) {
  uint32_t mu = 0;
  int32_t mi = 0;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    mu = max(mu, __float_as_uint(v[i]));
    mi = max(mi, (int32_t)__float_as_uint(v[i]));
  }
  return max(mu & 0x7fffffffu, (uint32_t)mi);
}

// encode_block for values stored at 2^SH times their rotated value.
template <int MODE, int SH>
__device__ __forceinline__ void encode_block_sh(const float (&v)[32], uint4& nib, uint32_t& s) {
  s = e8m0_byte_sh<MODE, SH>(amax_bits_n<32>(v));
  nib = (s == 255u) ? make_uint4(0, 0, 0, 0) : encode32(v, cvt_scale<SH>(s));
}

}  // namespace
}  // namespace mx
