// Rotate + MXFP4-quantize kernels for gfx950 (MI355X).
//
// Pages cited: [P1] "Pretraining Large Language Models with MXFP4 on Native
// FP4 Hardware" (arXiv:2605.09825 summary), section A.1 (MX reconstruction,
// shared exponent from the block maximum, nearest FP4 value), A.2
// (deterministic tiled Hadamard before the GEMM), D (1x32 / 32x1 / 32x32
// scale layouts); [P3] "Decomposing MXFP4 quantization error" blog
// (arXiv:2605.20402), pain-point and core-insight sections (32-element OCP
// MX block, E8M0 scale, E2M1 grid, ceiling-rounded scale of max|x| / 6).
//
// Every kernel is HBM-bound: it reads 2 B/element of bf16 and writes
// 0.5 B/element of packed E2M1 plus one E8M0 byte per block. Per element the
// ALU work is the widening shift, the fp32 butterfly (log2 h add/sub), one
// multiply by the Hadamard normalisation (H32 only: H16's 1/4 is folded into
// the convert's power-of-two divisor, bit-identically), an integer max for
// the block amax and half of one v_cvt_scalef32_pk_fp4_f32 (gfx950's scaled
// FP4 convert, which rounds x / 2^E to nearest-even E2M1 and saturates at
// 6).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "internal.h"
#include "mxfp4_device.h"

namespace mx {
namespace {

// Non-temporal loads of a lane's 8 or 16 consecutive source bytes. Every
// kernel reads its source once; where the 64 lanes of a load read one
// contiguous row segment, the non-temporal hint is 10-16% faster (measured on
// the column kernels: 8192 x 4096 20.1 -> 17.1 us, 8192 x 14336 68.5 -> 57.8
// us), while on a lane-strided pattern it is slower, so only contiguous
// loads use it.
typedef unsigned int nt_u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int nt_u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint2 ld_nt8(const uint16_t* p) {
  const nt_u32x2 w = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x2*>(p));
  return make_uint2(w.x, w.y);
}
__device__ __forceinline__ uint4 ld_nt16(const uint16_t* p) {
  const nt_u32x4 w = __builtin_nontemporal_load(reinterpret_cast<const nt_u32x4*>(p));
  return make_uint4(w.x, w.y, w.z, w.w);
}

// ---------------------------------------------------------------- row (1x32)
// One thread per 32-element block of a row-major matrix whose rows are a
// multiple of 32 long, so block b covers elements [32b, 32b + 32) of the
// flat array and owns nibble bytes [16b, 16b + 16) and scale byte b.
template <int H, int MODE>
__device__ __forceinline__ void row_block(const uint4* __restrict__ src, int64_t nblocks,
                                          uint4* __restrict__ nib, uint8_t* __restrict__ sc,
                                          int64_t b) {
  if (b >= nblocks) return;
  uint4 q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = src[b * 4 + j];
  float v[32];
  unpack64B(q, v);
  butterfly32<H>(v);
  uint4 out;
  uint32_t s;
  encode_block_sh<MODE, kScaleShift<H>>(v, out, s);
  nib[b] = out;
  sc[b] = (uint8_t)s;
}

template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_row_kernel(const uint4* __restrict__ src,
                                                        int64_t nblocks,
                                                        uint4* __restrict__ nib,
                                                        uint8_t* __restrict__ sc) {
  row_block<H, MODE>(src, nblocks, nib, sc, (int64_t)blockIdx.x * 256 + threadIdx.x);
}

// Lane-contiguous variant (nblocks % 64 == 0): a wave owns 64 consecutive
// blocks (4 KiB of bf16) and reads them with four 1 KiB instructions, lane l
// of instruction j taking 16-byte chunk 64 j + l (block 16 j + l / 4,
// quarter l % 4), so that every instruction covers whole cache lines once.
// A 4 x 4 transpose inside each lane quad (two DPP exchange stages, per
// dword) then gives lane 4 Q + p the four quarters of block 16 p + Q. The
// loads are non-temporal: the source is read once. Measured against the
// one-block-per-thread kernel (each load of which touches every line of a
// 4 KiB span a quarter at a time): 8192 x 28672 104 -> 89 us (6.7 TB/s),
// 32768 x 8192 119 -> 115 us, 8192 x 4096 16.7 -> 17.5 us; used above
// 2^20 blocks.
template <int CTRL>
__device__ __forceinline__ uint32_t quad_swap(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

__device__ __forceinline__ void quad_transpose(uint32_t (&x)[4], int p) {
  const bool b1 = (p & 2) != 0, b0 = (p & 1) != 0;
  // stage 1: lanes p and p ^ 2 trade a pair of values (quad_perm [2,3,0,1])
  const uint32_t r0 = quad_swap<0x4e>(b1 ? x[0] : x[2]), r1 = quad_swap<0x4e>(b1 ? x[1] : x[3]);
  if (b1) { x[0] = r0; x[1] = r1; } else { x[2] = r0; x[3] = r1; }
  // stage 2: lanes p and p ^ 1 trade one value of each pair (quad_perm [1,0,3,2])
  const uint32_t u0 = quad_swap<0xb1>(b0 ? x[0] : x[1]), u1 = quad_swap<0xb1>(b0 ? x[2] : x[3]);
  if (b0) { x[0] = u0; x[2] = u1; } else { x[1] = u0; x[3] = u1; }
}

// Blocks b0 .. b0 + 63 by one wave.
template <int H, int MODE>
__device__ __forceinline__ void row_lc_wave(const uint4* __restrict__ src, uint4* __restrict__ nib,
                                            uint8_t* __restrict__ sc, int64_t b0, int lane) {
  const nt_u32x4* s4 = reinterpret_cast<const nt_u32x4*>(src);
  uint4 q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const nt_u32x4 w = __builtin_nontemporal_load(s4 + b0 * 4 + 64 * j + lane);
    q[j] = make_uint4(w.x, w.y, w.z, w.w);
  }
  const int p = lane & 3;
  uint32_t x[4];
  x[0] = q[0].x; x[1] = q[1].x; x[2] = q[2].x; x[3] = q[3].x;
  quad_transpose(x, p);
  q[0].x = x[0]; q[1].x = x[1]; q[2].x = x[2]; q[3].x = x[3];
  x[0] = q[0].y; x[1] = q[1].y; x[2] = q[2].y; x[3] = q[3].y;
  quad_transpose(x, p);
  q[0].y = x[0]; q[1].y = x[1]; q[2].y = x[2]; q[3].y = x[3];
  x[0] = q[0].z; x[1] = q[1].z; x[2] = q[2].z; x[3] = q[3].z;
  quad_transpose(x, p);
  q[0].z = x[0]; q[1].z = x[1]; q[2].z = x[2]; q[3].z = x[3];
  x[0] = q[0].w; x[1] = q[1].w; x[2] = q[2].w; x[3] = q[3].w;
  quad_transpose(x, p);
  q[0].w = x[0]; q[1].w = x[1]; q[2].w = x[2]; q[3].w = x[3];
  const int64_t b = b0 + 16 * p + (lane >> 2);
  float v[32];
  unpack64B(q, v);
  butterfly32<H>(v);
  uint4 out;
  uint32_t s;
  encode_block_sh<MODE, kScaleShift<H>>(v, out, s);
  nib[b] = out;
  sc[b] = (uint8_t)s;
}

template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_row_lc_kernel(const uint4* __restrict__ src,
                                                           uint4* __restrict__ nib,
                                                           uint8_t* __restrict__ sc) {
  row_lc_wave<H, MODE>(src, nib, sc, ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * 64,
                       threadIdx.x & 63);
}

// ----------------------------------------------------------- 2D (32x32 tile)
// Any cols % 32 == 0 (the lane-contiguous form below takes cols % 256 == 0).
// Work-group = 32 rows x 8 column blocks (256 threads, one 1x32 block each);
// thread t: column block t & 7, row t >> 3. The tile amax is reduced across
// the 32 rows with lane shuffles (xor 8, 16, 32) and then across the four
// waves through LDS. Grid is flat: tile-row major over (rows/32, ceil(ncb/8)).
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_2d_kernel(const uint16_t* __restrict__ src,
                                                       int64_t rows, int64_t cols,
                                                       uint8_t* __restrict__ nib,
                                                       uint8_t* __restrict__ sc) {
  __shared__ uint32_t red[4][8];
  const int t = threadIdx.x;
  const int cbl = t & 7, r = t >> 3;
  const int64_t ncb = cols / 32;
  const int64_t ngrp = (ncb + 7) / 8;
  const int64_t tile_row = (int64_t)blockIdx.x / ngrp;
  const int64_t cb = ((int64_t)blockIdx.x % ngrp) * 8 + cbl;
  const int64_t row = tile_row * 32 + r;
  const bool active = cb < ncb;
  float v[32];
  if (active) {
    const uint4* p = reinterpret_cast<const uint4*>(src + row * cols + cb * 32);
    uint4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = p[j];
    unpack64B(q, v);
    butterfly32<H>(v);
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = 0.f;
  }
  uint32_t am = amax_bits_n<32>(v);
  am = max(am, (uint32_t)__shfl_xor((int)am, 8));
  am = max(am, (uint32_t)__shfl_xor((int)am, 16));
  am = max(am, (uint32_t)__shfl_xor((int)am, 32));
  const int wave = t >> 6;
  if ((t & 63) < 8) red[wave][cbl] = am;
  __syncthreads();
  am = max(max(red[0][cbl], red[1][cbl]), max(red[2][cbl], red[3][cbl]));
  if (!active) return;
  const uint32_t s = e8m0_byte_sh<MODE, kScaleShift<H>>(am);
  const uint4 out = (s == 255u) ? make_uint4(0, 0, 0, 0) : encode32(v, cvt_scale<kScaleShift<H>>(s));
  reinterpret_cast<uint4*>(nib + row * (cols / 2))[cb] = out;
  if (r == 0) sc[tile_row * ncb + cb] = (uint8_t)s;
}

// 2D with lane-contiguous loads, cols % 256 == 0: work-group = 4 waves over
// 32 rows x 256 columns (8 tiles). Lane l of wave w holds columns
// [8 (l % 32), 8 (l % 32) + 8) of rows 8 i + 2 w + l / 32, i = 0..3: each
// load instruction reads two whole 512-byte row segments. Within a lane the
// butterfly's stages 1, 2, 4 run in registers; stage 8 (and 16 for H32)
// pairs lanes l ^ 1 (l ^ 2), exchanged by DPP: the lower lane keeps a + b,
// the upper one a - b, each as one fma(own, +-1, partner), which rounds
// once like the add or subtract. Tile amax: the lane's 32 values, then
// lanes l ^ 1, l ^ 2, l ^ 32 and the four waves through LDS. Against the
// one-thread-per-block kernel above (lane-strided 16-byte loads) on the
// 8192 x 4096 workload: 15.9 against 16.4-16.5 us, identical bytes. A form
// with one wave per 32 x 64 strip (no LDS, amax over lanes ^ 8, 16, 32)
// was slower, 17.6 us.
template <int S>
__device__ __forceinline__ void cross_stage(float (&v)[8], int lane) {
  constexpr int ctl = S == 8 ? 0xb1 : 0x4e;  // quad_perm [1,0,3,2] / [2,3,0,1]
  const float sg = (lane & (S == 8 ? 1 : 2)) ? -1.0f : 1.0f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float p = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v[i]), ctl, 0xf, 0xf, false));
    v[i] = fmaf(v[i], sg, p);
  }
}

template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_2d_lc_kernel(const uint16_t* __restrict__ src,
                                                          int64_t rows, int64_t cols,
                                                          uint8_t* __restrict__ nib,
                                                          uint8_t* __restrict__ sc) {
  __shared__ uint32_t red[4][8];
  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int c8 = lane & 31, rh = lane >> 5;
  const int64_t ncg = cols / 256;
  const int64_t tile_row = (int64_t)blockIdx.x / ncg;
  const int64_t c0 = ((int64_t)blockIdx.x % ncg) * 256;
  float v[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t row = tile_row * 32 + 8 * i + 2 * w + rh;
    const uint4 q = ld_nt16(src + row * cols + c0 + 8 * c8);
    const uint32_t d[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[i][2 * k] = bf16lo(d[k]);
      v[i][2 * k + 1] = bf16hi(d[k]);
    }
  }
  uint32_t am = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (H != 0) {
#pragma unroll
      for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if ((e & s) == 0) {
            const float a = v[i][e], b = v[i][e + s];
            v[i][e] = a + b;
            v[i][e + s] = a - b;
          }
      cross_stage<8>(v[i], lane);
      if constexpr (H == 32) {
        cross_stage<16>(v[i], lane);
#pragma unroll
        for (int e = 0; e < 8; ++e) v[i][e] *= __uint_as_float(0x3E3504F3u);
      }
    }
    am = max(am, amax_bits_n<8>(v[i]));
  }
  am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0xb1, 0xf, 0xf, false));
  am = max(am, (uint32_t)__builtin_amdgcn_mov_dpp((int)am, 0x4e, 0xf, 0xf, false));
  am = max(am, (uint32_t)__shfl_xor((int)am, 32));
  if (rh == 0 && (c8 & 3) == 0) red[w][c8 >> 2] = am;
  __syncthreads();
  const int bc = c8 >> 2;
  am = max(max(red[0][bc], red[1][bc]), max(red[2][bc], red[3][bc]));
  const uint32_t s = e8m0_byte_sh<MODE, kScaleShift<H>>(am);
  const float scale = cvt_scale<kScaleShift<H>>(s);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t r = 0;
    if (s != 255u) {
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[i][0], v[i][1], scale, 0);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[i][2], v[i][3], scale, 1);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[i][4], v[i][5], scale, 2);
      r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[i][6], v[i][7], scale, 3);
    }
    const int64_t row = tile_row * 32 + 8 * i + 2 * w + rh;
    *reinterpret_cast<uint32_t*>(nib + row * (cols / 2) + c0 / 2 + 4 * c8) = r;
  }
  if (w == 0 && rh == 0 && (c8 & 3) == 0) sc[tile_row * (cols / 32) + c0 / 32 + bc] = (uint8_t)s;
}

// ------------------------------------------------------ column (32x1, transposed)
// Three paths: staged (below, rows % 128 == 0), vector (cols % 8 == 0) and
// scalar (any cols).
// Vector path (cols % 8 == 0). Work-group = 4 waves; the flat grid walks
// (row group of 128, column group of 512) with the column group fastest.
// Lane l of wave w owns columns [c0, c0 + 8), c0 = group*512 + 8l, for the
// 32-row band 4*rowgroup + w: it loads the band with 32 coalesced 16-byte
// loads (a wave reads 1 KB contiguous per row), so each of its 8 columns'
// 32x1 block sits in its own registers and the rotation down the rows needs
// no data exchange. Output row c of the transposed operand receives the
// band's 16 nibble bytes at offset 16*band and its scale byte at `band`.
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_col_kernel(const uint16_t* __restrict__ src,
                                                        int64_t rows, int64_t cols,
                                                        uint8_t* __restrict__ nib,
                                                        uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ncg = (cols + 511) / 512;
  const int64_t cg = (int64_t)blockIdx.x % ncg;
  const int64_t rg = (int64_t)blockIdx.x / ncg;
  const int64_t band = rg * 4 + wave;
  const int64_t c0 = cg * 512 + (int64_t)lane * 8;
  if (band * 32 >= rows || c0 >= cols) return;
  const uint16_t* p = src + band * 32 * cols + c0;
  uint4 raw[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) raw[r] = ld_nt16(p + r * cols);
  const int64_t nib_pitch = rows / 2, sc_pitch = rows / 32;
#pragma unroll
  for (int pr = 0; pr < 4; ++pr) {
    float a[32], b[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t d = pr == 0 ? raw[r].x : pr == 1 ? raw[r].y : pr == 2 ? raw[r].z : raw[r].w;
      a[r] = bf16lo(d);
      b[r] = bf16hi(d);
    }
    butterfly32<H>(a);
    butterfly32<H>(b);
    uint4 na, nb;
    uint32_t sa, sb;
    encode_block_sh<MODE, kScaleShift<H>>(a, na, sa);
    encode_block_sh<MODE, kScaleShift<H>>(b, nb, sb);
    const int64_t ca = c0 + 2 * pr, cb = ca + 1;
    *reinterpret_cast<uint4*>(nib + ca * nib_pitch + band * 16) = na;
    *reinterpret_cast<uint4*>(nib + cb * nib_pitch + band * 16) = nb;
    sc[ca * sc_pitch + band] = (uint8_t)sa;
    sc[cb * sc_pitch + band] = (uint8_t)sb;
  }
}

// Staged path (rows % (32 NB) == 0, cols % 4 == 0, scale pointer aligned to
// NB bytes): work-group = NB waves = NB bands of 32 rows x 256 columns, NB = 8
// (or 4). Lane l of wave w owns columns [c0, c0 + 4), c0 = group*256 + 4l, of
// band NB*rowgroup + w and loads them with 32 8-byte loads (a wave reads 512
// contiguous bytes per row). The quantized bands go to LDS; the work-group
// then writes each column's NB bands as 16 NB contiguous nibble bytes (with
// NB = 8 a whole 128-byte line) and one NB-byte scale word, instead of
// scattered 16-byte and 1-byte stores. Four columns per lane keep the
// register count low enough for several waves per SIMD, so the loads of one
// wave overlap the arithmetic of another.
template <int H, int MODE, int NB, bool RS>
__device__ __forceinline__ void col_staged_wg(const uint16_t* __restrict__ src, int64_t rows,
                                              int64_t cols, uint8_t* __restrict__ nib,
                                              uint8_t* __restrict__ sc,
                                              const uint8_t* __restrict__ signs, int64_t wg) {
  __shared__ __attribute__((aligned(16))) uint8_t onib[256 * NB * 16];
  __shared__ __attribute__((aligned(16))) uint8_t osc[256 * NB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ncg = (cols + 255) / 256;
  const int64_t cg = wg % ncg;
  const int64_t rg = wg / ncg;
  const int64_t band = rg * NB + wave;
  const int64_t c0 = cg * 256 + (int64_t)lane * 4;
  if (c0 < cols) {
    const uint16_t* p = src + band * 32 * cols + c0;
    uint2 raw[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) raw[r] = ld_nt8(p + r * cols);
    if constexpr (RS) {  // random-sign arm: one sign per row, the same for the whole wave
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const uint32_t f = (signs[band * 32 + r] & 1u) ? 0x80008000u : 0u;
        raw[r].x ^= f;
        raw[r].y ^= f;
      }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {  // one column at a time keeps the register count low
      float a[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const uint32_t d = j < 2 ? raw[r].x : raw[r].y;
        a[r] = (j & 1) ? bf16hi(d) : bf16lo(d);
      }
      butterfly32<H>(a);
      uint4 na;
      uint32_t sa;
      encode_block_sh<MODE, kScaleShift<H>>(a, na, sa);
      const int ca = lane * 4 + j;
      *reinterpret_cast<uint4*>(onib + (ca * NB + wave) * 16) = na;
      osc[ca * NB + wave] = (uint8_t)sa;
    }
  }
  __syncthreads();
  const int64_t npitch = rows / 2, spitch = rows / 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = threadIdx.x + 64 * NB * i;  // 16-byte chunk: column q / NB, band q % NB
    const int64_t col = cg * 256 + q / NB;
    if (col < cols)
      *reinterpret_cast<uint4*>(nib + col * npitch + rg * 16 * NB + (q % NB) * 16) =
          *reinterpret_cast<const uint4*>(onib + q * 16);
  }
  if (threadIdx.x < 256) {
    const int64_t col = cg * 256 + threadIdx.x;
    if (col < cols) {
      if constexpr (NB == 8)
        *reinterpret_cast<uint2*>(sc + col * spitch + rg * 8) =
            *reinterpret_cast<const uint2*>(osc + threadIdx.x * 8);
      else
        *reinterpret_cast<uint32_t*>(sc + col * spitch + rg * 4) =
            *reinterpret_cast<const uint32_t*>(osc + threadIdx.x * 4);
    }
  }
}

template <int H, int MODE, int NB, bool RS = false>
__global__ __launch_bounds__(64 * NB) void quant_col_staged_kernel(const uint16_t* __restrict__ src,
                                                                   int64_t rows, int64_t cols,
                                                                   uint8_t* __restrict__ nib,
                                                                   uint8_t* __restrict__ sc,
                                                                   const uint8_t* __restrict__ signs) {
  col_staged_wg<H, MODE, NB, RS>(src, rows, cols, nib, sc, signs, blockIdx.x);
}

// Scalar path for any cols: one thread per (column, 32-row band); loads are
// 2-byte, coalesced across the threads of a row.
template <int H, int MODE, bool RS = false>
__global__ __launch_bounds__(256) void quant_col_scalar_kernel(const uint16_t* __restrict__ src,
                                                               int64_t rows, int64_t cols,
                                                               uint8_t* __restrict__ nib,
                                                               uint8_t* __restrict__ sc,
                                                               const uint8_t* __restrict__ signs) {
  const int64_t ncg = (cols + 255) / 256;
  const int64_t c = ((int64_t)blockIdx.x % ncg) * 256 + threadIdx.x;
  const int64_t band = (int64_t)blockIdx.x / ncg;
  if (c >= cols || band * 32 >= rows) return;
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    uint32_t b = (uint32_t)src[(band * 32 + r) * cols + c] << 16;
    if constexpr (RS) b ^= (signs[band * 32 + r] & 1u) << 31;
    v[r] = __uint_as_float(b);
  }
  butterfly32<H>(v);
  uint4 out;
  uint32_t s;
  encode_block_sh<MODE, kScaleShift<H>>(v, out, s);
  *reinterpret_cast<uint4*>(nib + c * (rows / 2) + band * 16) = out;
  sc[c * (rows / 32) + band] = (uint8_t)s;
}

// ------------------------------------------------ dual (row + column, one read)
// Training needs an activation both along its feature axis (Fprop, Dgrad:
// 1x32 blocks, rotation along cols) and along the token axis (Wgrad: 32x1
// blocks, rotation down rows, transposed output); [P1] A.2 and D quantize
// both from the same tensor. This kernel reads the bf16 tile once and emits
// both packed operands, each exactly as mxfp4_quantize would.
//
// Tiling as the staged column path (4 bands of 32 rows; here also
// cols % 256 == 0): lane l of wave w holds columns [4l, 4l + 4) of its
// 256-column group for the 32 rows of band 4*rowgroup + w. Column
// direction: unchanged. Row direction, per group of 4 rows: a 4x4 transpose
// inside each quad of lanes (DPP quad permutations) gives lane 4q + p the 16
// consecutive columns [16q, 16q + 16) of row 4g + p, so the H16 butterfly
// runs in registers; the two 16-column halves of a 32-block sit in lanes l
// and l ^ 4, which exchange once for the block amax (and, for H32, for the
// butterfly's last stage). The kernel is VALU-bound (two rotations and two
// encodes per element loaded), so the H16 1/4 moves into the scale
// (kScaleShift) and the amax uses amax_bits_n. Both outputs are staged in
// LDS and written with 16-byte nibble stores (whole 128-byte lines per row)
// and 4- or 8-byte scale stores. Measured against the previous layout, in
// which each row's 32-block stayed spread over 8 lanes (two cross-lane
// butterfly stages and three cross-lane amax steps per row, 144 VGPRs, 3
// waves per SIMD): 8192 x 4096 32.2 -> 23.7 us, 8192 x 14336 88.0 -> 75.1
// us, bit-identical outputs.
//
// Lane exchange inside groups of 8 lanes: partner lane l ^ M. M = 1, 2 use a
// DPP quad permutation (lane i of a quad reads lane sel[i]); M = 4 uses
// ds_swizzle in bit mode (lane i reads lane ((i & 0x1f) | 0) ^ 4).
template <int M>
__device__ __forceinline__ uint32_t xchg(uint32_t v) {
  if constexpr (M == 1)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);  // [1,0,3,2]
  else if constexpr (M == 2)
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, false);  // [2,3,0,1]
  else
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x101F);               // xor 4
}

template <int M>
__device__ __forceinline__ float xchgf(float v) {
  return __uint_as_float(xchg<M>(__float_as_uint(v)));
}

// Quad transpose with every partner value fetched unconditionally and then
// selected (x[j] of lane p becomes x[p] of lane j). Same result as
// quad_transpose; selecting what to send first, as there, lets the compiler
// turn the DPP moves into branches around single lanes, which costs more
// here where the transpose runs 16 times per wave.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_quad(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, 0xf, 0xf, true);
}

__device__ __forceinline__ void quad_transpose_sel(uint32_t (&x)[4], bool b1, bool b0) {
  const uint32_t d0 = dpp_quad<0x4e>(x[0]), d1 = dpp_quad<0x4e>(x[1]);
  const uint32_t d2 = dpp_quad<0x4e>(x[2]), d3 = dpp_quad<0x4e>(x[3]);
  const uint32_t y0 = b1 ? d2 : x[0], y1 = b1 ? d3 : x[1];
  const uint32_t y2 = b1 ? x[2] : d0, y3 = b1 ? x[3] : d1;
  const uint32_t e0 = dpp_quad<0xb1>(y0), e1 = dpp_quad<0xb1>(y1);
  const uint32_t e2 = dpp_quad<0xb1>(y2), e3 = dpp_quad<0xb1>(y3);
  x[0] = b0 ? e1 : y0;
  x[1] = b0 ? y1 : e0;
  x[2] = b0 ? e3 : y2;
  x[3] = b0 ? y3 : e2;
}

template <int H, int MODE, int NB>
__global__ __launch_bounds__(64 * NB) void quant_dual_kernel(const uint16_t* __restrict__ src,
                                                             int64_t rows, int64_t cols,
                                                             uint8_t* __restrict__ rnib,
                                                             uint8_t* __restrict__ rsc,
                                                             uint8_t* __restrict__ cnib,
                                                             uint8_t* __restrict__ csc) {
  constexpr int SH = kScaleShift<H>;
  __shared__ __attribute__((aligned(16))) uint8_t onib[256 * NB * 16];  // column output
  __shared__ __attribute__((aligned(16))) uint8_t osc[256 * NB];
  __shared__ __attribute__((aligned(16))) uint8_t lrn[32 * NB * 128];   // row output
  __shared__ __attribute__((aligned(16))) uint8_t lrs[32 * NB * 8];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ncg = cols / 256;
  const int64_t cg = (int64_t)blockIdx.x % ncg;
  const int64_t rg = (int64_t)blockIdx.x / ncg;
  const int64_t band = rg * NB + wave;
  const int64_t c0 = cg * 256 + (int64_t)lane * 4;
  const uint16_t* p = src + band * 32 * cols + c0;
  uint2 raw[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) raw[r] = ld_nt8(p + r * cols);
  // row direction
  const int q = lane >> 2, pq = lane & 3;
  const bool b1 = (pq & 2) != 0, b0 = (pq & 1) != 0;
#pragma unroll
  for (int g = 0; g < 8; ++g) {
    uint32_t xs[4], ys[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      xs[i] = raw[4 * g + i].x;
      ys[i] = raw[4 * g + i].y;
    }
    quad_transpose_sel(xs, b1, b0);
    quad_transpose_sel(ys, b1, b0);
    float v[16];  // columns 16q + k of row 4g + pq
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 * i] = bf16lo(xs[i]);
      v[4 * i + 1] = bf16hi(xs[i]);
      v[4 * i + 2] = bf16lo(ys[i]);
      v[4 * i + 3] = bf16hi(ys[i]);
    }
    if constexpr (H != 0) {
#pragma unroll
      for (int s = 1; s < 16; s <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          if ((i & s) == 0) {
            const float a = v[i], b = v[i + s];
            v[i] = a + b;
            v[i + s] = a - b;
          }
        }
      }
    }
    if constexpr (H == 32) {
      // stage 16: the lane with the lower half forms own + partner (a + b),
      // its partner partner + (-own) (a - b, the same fp32 operation)
      const uint32_t flip = (lane & 4) ? 0x80000000u : 0u;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float y = xchgf<4>(v[i]);
        v[i] = y + __uint_as_float(__float_as_uint(v[i]) ^ flip);
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] *= __uint_as_float(0x3E3504F3u);
    }
    uint32_t am = amax_bits_n<16>(v);
    am = max(am, xchg<4>(am));
    const uint32_t s = e8m0_byte_sh<MODE, SH>(am);
    uint32_t w0 = 0, w1 = 0;
    if (s != 255u) {
      const float scale = cvt_scale<SH>(s);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[0], v[1], scale, 0);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[2], v[3], scale, 1);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[4], v[5], scale, 2);
      w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, v[6], v[7], scale, 3);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[8], v[9], scale, 0);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[10], v[11], scale, 1);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[12], v[13], scale, 2);
      w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, v[14], v[15], scale, 3);
    }
    const int lr = wave * 32 + 4 * g + pq;
    *reinterpret_cast<uint2*>(lrn + lr * 128 + 8 * q) = make_uint2(w0, w1);
    if ((q & 1) == 0) lrs[lr * 8 + (q >> 1)] = (uint8_t)s;
  }
  // column direction
#pragma unroll
  for (int j = 0; j < 4; ++j) {  // one column at a time keeps the register count low
    float a[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) {
      const uint32_t d = j < 2 ? raw[r].x : raw[r].y;
      a[r] = (j & 1) ? bf16hi(d) : bf16lo(d);
    }
    butterfly32<H>(a);
    uint4 na;
    uint32_t sa;
    encode_block_sh<MODE, SH>(a, na, sa);
    const int ca = lane * 4 + j;
    *reinterpret_cast<uint4*>(onib + (ca * NB + wave) * 16) = na;
    osc[ca * NB + wave] = (uint8_t)sa;
  }
  __syncthreads();
  const int t = threadIdx.x;
  const int64_t npitch = rows / 2, spitch = rows / 32;
  const int64_t rpitch = cols / 2, rspitch = cols / 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = t + 64 * NB * i;
    // column output: 16-byte chunk k = (column k / NB, band k % NB)
    *reinterpret_cast<uint4*>(cnib + (cg * 256 + k / NB) * npitch + rg * 16 * NB + (k % NB) * 16) =
        *reinterpret_cast<const uint4*>(onib + k * 16);
    // row output: 16-byte chunk k = (row k / 8, chunk k % 8)
    *reinterpret_cast<uint4*>(rnib + (rg * 32 * NB + (k >> 3)) * rpitch + cg * 128 + (k & 7) * 16) =
        *reinterpret_cast<const uint4*>(lrn + k * 16);
  }
  if (t < 256) {
    if constexpr (NB == 8)
      *reinterpret_cast<uint2*>(csc + (cg * 256 + t) * spitch + rg * 8) =
          *reinterpret_cast<const uint2*>(osc + t * 8);
    else
      *reinterpret_cast<uint32_t*>(csc + (cg * 256 + t) * spitch + rg * 4) =
          *reinterpret_cast<const uint32_t*>(osc + t * 4);
  }
  if (t < 32 * NB)
    *reinterpret_cast<uint2*>(rsc + (rg * 32 * NB + t) * rspitch + cg * 8) =
        *reinterpret_cast<const uint2*>(lrs + t * 8);
}

// -------------------------------------------------- outlier fallback (OF)
// [P3] "three targeted fixes" section, OF: x_OF = Q(x) + alpha Q(x - Q(x)),
// alpha = 1/2, here applied as a prescale of the residual, Q(r / 2) (equal to
// Q(r) / 2 unless the residual block sits at the E8M0 floor). Per 32-block:
// quantize, decode the codes back to fp32 (an E2M1 value times 2^E, exact
// unless it overflows), r = y - q1 and h = r / 2 in fp32 (one rounding
// each), quantize h. The values stay normalised here (no folded H16 scale):
// near the fp32 maximum the decode of 4 q1 can overflow where that of q1
// does not.
// The output is one K-concatenated operand: row i = q1's row, then q2's
// row; a GEMM of depth 2 Kb against the other operand repeated along K
// computes sum (q1 + q2) b. A non-finite block is 0xFF in both halves.
// The first pass is decoded with gfx950's scaled FP4-to-fp32 convert, which
// returns the E2M1 value times the fp32 scale as one IEEE multiply (an
// in-bounds probe over all 16 codes and all 255 scale bytes matched fp32
// products bit for bit, subnormal results and overflow to +-Inf included).
typedef float of_f32x2 __attribute__((ext_vector_type(2)));

template <int MODE>
__device__ __forceinline__ void of_block(float (&v)[32], uint4& n1, uint32_t& s1, uint4& n2,
                                         uint32_t& s2) {
  s1 = e8m0_byte<MODE>(amax_bits_n<32>(v));
  if (s1 == 255u) {
    n1 = make_uint4(0, 0, 0, 0);
    n2 = make_uint4(0, 0, 0, 0);
    s2 = 255u;
    return;
  }
  const float sc = scale_of_byte(s1);
  n1 = encode32(v, sc);
  const uint32_t w[4] = {n1.x, n1.y, n1.z, n1.w};
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    of_f32x2 q[4];
    q[0] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], sc, 0);
    q[1] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], sc, 1);
    q[2] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], sc, 2);
    q[3] = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[d], sc, 3);
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      v[8 * d + 2 * k] = 0.5f * (v[8 * d + 2 * k] - q[k].x);
      v[8 * d + 2 * k + 1] = 0.5f * (v[8 * d + 2 * k + 1] - q[k].y);
    }
  }
  s2 = e8m0_byte<MODE>(amax_bits_n<32>(v));
  n2 = (s2 == 255u) ? make_uint4(0, 0, 0, 0) : encode32(v, scale_of_byte(s2));
}

// Row axis: one thread per 32-block (block b of row b / ncb).
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_of_row_kernel(const uint4* __restrict__ src,
                                                           int64_t nblocks, int64_t ncb,
                                                           uint8_t* __restrict__ nib,
                                                           uint8_t* __restrict__ sc) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint4 q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = src[b * 4 + j];
  float v[32];
  unpack64B(q, v);
  hadamard32<H>(v);
  uint4 n1, n2;
  uint32_t s1, s2;
  of_block<MODE>(v, n1, s1, n2, s2);
  const int64_t row = b / ncb, cb = b % ncb;
  uint4* out = reinterpret_cast<uint4*>(nib + row * ncb * 32);  // 2 * ncb * 16 bytes per row
  out[cb] = n1;
  out[ncb + cb] = n2;
  sc[row * 2 * ncb + cb] = (uint8_t)s1;
  sc[row * 2 * ncb + ncb + cb] = (uint8_t)s2;
}

// Column axis: one thread per (column, 32-row band); loads are 2-byte,
// coalesced across the threads of a row. Output row c of the transposed
// operand: the band's q1 block at band, its q2 block at nb + band.
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_of_col_kernel(const uint16_t* __restrict__ src,
                                                           int64_t rows, int64_t cols,
                                                           uint8_t* __restrict__ nib,
                                                           uint8_t* __restrict__ sc) {
  const int64_t ncg = (cols + 255) / 256;
  const int64_t c = ((int64_t)blockIdx.x % ncg) * 256 + threadIdx.x;
  const int64_t band = (int64_t)blockIdx.x / ncg;
  if (c >= cols || band * 32 >= rows) return;
  float v[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) v[r] = __uint_as_float((uint32_t)src[(band * 32 + r) * cols + c] << 16);
  hadamard32<H>(v);
  uint4 n1, n2;
  uint32_t s1, s2;
  of_block<MODE>(v, n1, s1, n2, s2);
  const int64_t nb = rows / 32;
  uint4* out = reinterpret_cast<uint4*>(nib + c * nb * 32);
  out[band] = n1;
  out[nb + band] = n2;
  sc[c * 2 * nb + band] = (uint8_t)s1;
  sc[c * 2 * nb + nb + band] = (uint8_t)s2;
}

// Column axis, staged (rows % 128 == 0, cols % 4 == 0, nibble pointer
// 16-byte and scale pointer 4-byte aligned): the column quantizer's tile
// with 4 bands (128 rows x 256 columns per work-group, 8-byte non-temporal
// loads, a lane's 4 columns of its band in registers); both passes of every
// block are staged in LDS and leave as 64-byte nibble runs and 4-byte scale
// words per column and half.
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_of_col_staged_kernel(const uint16_t* __restrict__ src,
                                                                  int64_t rows, int64_t cols,
                                                                  uint8_t* __restrict__ nib,
                                                                  uint8_t* __restrict__ sc) {
  constexpr int NB = 4;
  __shared__ __attribute__((aligned(16))) uint8_t onib[2][256 * NB * 16];
  __shared__ __attribute__((aligned(16))) uint8_t osc[2][256 * NB];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ncg = (cols + 255) / 256;
  const int64_t cg = (int64_t)blockIdx.x % ncg;
  const int64_t rg = (int64_t)blockIdx.x / ncg;
  const int64_t c0 = cg * 256 + (int64_t)lane * 4;
  if (c0 < cols) {
    const uint16_t* p = src + (rg * NB + wave) * 32 * cols + c0;
    uint2 raw[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) raw[r] = ld_nt8(p + r * cols);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      float a[32];
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const uint32_t d = j < 2 ? raw[r].x : raw[r].y;
        a[r] = (j & 1) ? bf16hi(d) : bf16lo(d);
      }
      hadamard32<H>(a);
      uint4 n1, n2;
      uint32_t s1, s2;
      of_block<MODE>(a, n1, s1, n2, s2);
      const int k = (lane * 4 + j) * NB + wave;
      *reinterpret_cast<uint4*>(onib[0] + k * 16) = n1;
      *reinterpret_cast<uint4*>(onib[1] + k * 16) = n2;
      osc[0][k] = (uint8_t)s1;
      osc[1][k] = (uint8_t)s2;
    }
  }
  __syncthreads();
  // output row c: q1's rows / 2 nibble bytes, then q2's; scales likewise
  const int64_t npitch = rows, spitch = rows / 16, nhalf = rows / 2, shalf = rows / 32;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = threadIdx.x + 64 * NB * i;  // 16-byte chunk: column k / NB, band k % NB
      const int64_t col = cg * 256 + k / NB;
      if (col < cols)
        *reinterpret_cast<uint4*>(nib + col * npitch + h * nhalf + rg * 16 * NB + (k % NB) * 16) =
            *reinterpret_cast<const uint4*>(onib[h] + k * 16);
    }
    const int64_t col = cg * 256 + threadIdx.x;
    if (col < cols)
      *reinterpret_cast<uint32_t*>(sc + col * spitch + h * shalf + rg * NB) =
          *reinterpret_cast<const uint32_t*>(osc[h] + threadIdx.x * NB);
  }
}

template <int H, int MODE>
hipError_t dispatch_of(const void* src, int64_t rows, int64_t cols, int axis, void* nib, void* sc,
                       hipStream_t st) {
  if (axis == 0) {
    const int64_t ncb = cols / 32, nblocks = rows * ncb;
    hipLaunchKernelGGL((quant_of_row_kernel<H, MODE>), dim3((unsigned)((nblocks + 255) / 256)),
                       dim3(256), 0, st, static_cast<const uint4*>(src), nblocks, ncb,
                       static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc));
  } else if (rows % 128 == 0 && cols % 4 == 0 && (uintptr_t)nib % 16 == 0 &&
             (uintptr_t)sc % 4 == 0) {
    const int64_t grid = (rows / 128) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_of_col_staged_kernel<H, MODE>), dim3((unsigned)grid), dim3(256), 0,
                       st, static_cast<const uint16_t*>(src), rows, cols, static_cast<uint8_t*>(nib),
                       static_cast<uint8_t*>(sc));
  } else {
    const int64_t grid = (rows / 32) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_of_col_kernel<H, MODE>), dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const uint16_t*>(src), rows, cols, static_cast<uint8_t*>(nib),
                       static_cast<uint8_t*>(sc));
  }
  return hipGetLastError();
}

// ---------------------------------------------- macro-block scaling (MBS)
// [P3] "three targeted fixes" section, MBS: one 8-bit mantissa (1 + m) per
// macro-block of 128 elements (4 blocks), x_hat = Q((1 + m) x) / (1 + m).
// m is chosen (a reading; the pages fix only the form) as the largest byte
// with (1 + m/256) M <= 6 2^k, M the macro-block amax and k the smallest
// integer with 6 2^k >= M: the prescaled macro maximum then sits at the top
// of its E8M0 bracket, removing that block's scale bias. Evaluated in fp64:
// m = floor(256 (6 2^k / M - 1)); zero or non-finite M gives m = 0.
__device__ __forceinline__ uint32_t mbs_byte(uint32_t am) {
  if (am == 0u || am >= 0x7f800000u) return 0u;
  const double M = (double)__uint_as_float(am);
  int e1;
  const double fr = frexp(M, &e1);  // M = fr 2^e1, fr in [0.5, 1)
  const int e = e1 - 1;
  const int k = (2.0 * fr <= 1.5) ? e - 2 : e - 1;
  const double c = ldexp(6.0, k) / M;
  const double m = floor((c - 1.0) * 256.0);
  return (uint32_t)(m < 0.0 ? 0.0 : (m > 255.0 ? 255.0 : m));
}

// Row axis: one thread per 32-block; the four lanes of a quad hold the four
// blocks of one macro-block (rows are a multiple of 128 long) and share
// their amax through DPP.
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_mbs_row_kernel(const uint4* __restrict__ src,
                                                            int64_t nblocks,
                                                            uint4* __restrict__ nib,
                                                            uint8_t* __restrict__ sc,
                                                            uint8_t* __restrict__ mbs) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;  // nblocks % 4 == 0: whole quads leave together
  uint4 q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = src[b * 4 + j];
  float v[32];
  unpack64B(q, v);
  hadamard32<H>(v);
  uint32_t am = amax_bits32(v);
  am = max(am, xchg<1>(am));
  am = max(am, xchg<2>(am));
  const uint32_t m = mbs_byte(am);
  const float c = 1.0f + (float)m * 0.00390625f;
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = c * v[i];
  uint4 out;
  uint32_t s;
  encode_block<MODE>(v, out, s);
  nib[b] = out;
  sc[b] = (uint8_t)s;
  if ((b & 3) == 0) mbs[b >> 2] = (uint8_t)m;
}

// Column axis: one thread per (column, 128-row macro band); a first pass
// takes the amax of the four rotated 32x1 blocks, a second reloads,
// rotates, prescales and encodes them (2-byte loads, coalesced across the
// threads of a row).
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_mbs_col_kernel(const uint16_t* __restrict__ src,
                                                            int64_t rows, int64_t cols,
                                                            uint8_t* __restrict__ nib,
                                                            uint8_t* __restrict__ sc,
                                                            uint8_t* __restrict__ mbs) {
  const int64_t ncg = (cols + 255) / 256;
  const int64_t c = ((int64_t)blockIdx.x % ncg) * 256 + threadIdx.x;
  const int64_t mb = (int64_t)blockIdx.x / ncg;
  if (c >= cols) return;
  const uint16_t* p = src + mb * 128 * cols + c;
  uint32_t am = 0;
  for (int j = 0; j < 4; ++j) {
    float v[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = __uint_as_float((uint32_t)p[(32 * j + r) * cols] << 16);
    hadamard32<H>(v);
    am = max(am, amax_bits32(v));
  }
  const uint32_t m = mbs_byte(am);
  const float cf = 1.0f + (float)m * 0.00390625f;
  for (int j = 0; j < 4; ++j) {
    float v[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) v[r] = __uint_as_float((uint32_t)p[(32 * j + r) * cols] << 16);
    hadamard32<H>(v);
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = cf * v[i];
    uint4 out;
    uint32_t s;
    encode_block<MODE>(v, out, s);
    *reinterpret_cast<uint4*>(nib + c * (rows / 2) + (4 * mb + j) * 16) = out;
    sc[c * (rows / 32) + 4 * mb + j] = (uint8_t)s;
  }
  mbs[c * (rows / 128) + mb] = (uint8_t)m;
}

// Column axis, staged (rows % 128 == 0, cols % 4 == 0, nibble and scale
// pointers 16- and 4-byte aligned): a work-group of 4 waves covers one
// 128-row macro band x 256 columns, the column quantizer's tile with 4
// bands. Lane l of wave w loads its 4 columns of band w (32 rows, 8-byte
// non-temporal loads), rotates them and keeps the 128 rotated values in
// registers; the block amaxes meet in LDS, where each lane takes the
// macro-block maximum of its columns over the 4 waves. The prescale needs
// no second pass over the values' maxima: fl32 rounding is monotonic, so the
// amax of fl32(c y) is fl32(c amax(y)). For H16 the values stay
// unnormalised (u = 4 y, exact) and the 1/4 joins the prescale:
// fl32((c / 4) u) is the same single rounding of c y. Outputs are staged in
// LDS and leave as 64-byte nibble runs and 4-byte scale words per column.
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_mbs_col_staged_kernel(
    const uint16_t* __restrict__ src, int64_t rows, int64_t cols, uint8_t* __restrict__ nib,
    uint8_t* __restrict__ sc, uint8_t* __restrict__ mbs) {
  constexpr int NB = 4;
  __shared__ __attribute__((aligned(16))) uint8_t onib[256 * NB * 16];
  __shared__ __attribute__((aligned(16))) uint8_t osc[256 * NB];
  __shared__ __attribute__((aligned(16))) uint32_t lam[NB][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t ncg = (cols + 255) / 256;
  const int64_t cg = (int64_t)blockIdx.x % ncg;
  const int64_t mb = (int64_t)blockIdx.x / ncg;
  const int64_t c0 = cg * 256 + (int64_t)lane * 4;
  const bool live = c0 < cols;
  float u[4][32];
  uint32_t bam[4] = {0u, 0u, 0u, 0u};
  if (live) {
    const uint16_t* p = src + (mb * NB + wave) * 32 * cols + c0;
    uint2 raw[32];
#pragma unroll
    for (int r = 0; r < 32; ++r) raw[r] = ld_nt8(p + r * cols);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const uint32_t d = j < 2 ? raw[r].x : raw[r].y;
        u[j][r] = (j & 1) ? bf16hi(d) : bf16lo(d);
      }
      butterfly32<H>(u[j]);
      bam[j] = amax_bits_n<32>(u[j]);
    }
  }
  *reinterpret_cast<uint4*>(&lam[wave][lane * 4]) = make_uint4(bam[0], bam[1], bam[2], bam[3]);
  __syncthreads();
  if (live) {
    uint32_t mcol[4];
    {
      const uint4 a0 = *reinterpret_cast<const uint4*>(&lam[0][lane * 4]);
      const uint4 a1 = *reinterpret_cast<const uint4*>(&lam[1][lane * 4]);
      const uint4 a2 = *reinterpret_cast<const uint4*>(&lam[2][lane * 4]);
      const uint4 a3 = *reinterpret_cast<const uint4*>(&lam[3][lane * 4]);
      mcol[0] = max(max(a0.x, a1.x), max(a2.x, a3.x));
      mcol[1] = max(max(a0.y, a1.y), max(a2.y, a3.y));
      mcol[2] = max(max(a0.z, a1.z), max(a2.z, a3.z));
      mcol[3] = max(max(a0.w, a1.w), max(a2.w, a3.w));
    }
    const int64_t mpitch = rows / 128;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // macro amax of the rotated values (H16: u / 4, exact in fp32)
      const uint32_t M = (H == 16) ? __float_as_uint(__uint_as_float(mcol[j]) * 0.25f) : mcol[j];
      const uint32_t m = mbs_byte(M);
      const float cf = 1.0f + (float)m * 0.00390625f;
      const float ck = (H == 16) ? cf * 0.25f : cf;
#pragma unroll
      for (int r = 0; r < 32; ++r) u[j][r] = ck * u[j][r];
      const uint32_t s = e8m0_byte<MODE>(__float_as_uint(ck * __uint_as_float(bam[j])));
      const uint4 na = (s == 255u) ? make_uint4(0, 0, 0, 0) : encode32(u[j], scale_of_byte(s));
      const int ca = lane * 4 + j;
      *reinterpret_cast<uint4*>(onib + (ca * NB + wave) * 16) = na;
      osc[ca * NB + wave] = (uint8_t)s;
      if (wave == 0) mbs[(c0 + j) * mpitch + mb] = (uint8_t)m;
    }
  }
  __syncthreads();
  const int64_t npitch = rows / 2, spitch = rows / 32;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + 64 * NB * i;  // 16-byte chunk: column k / NB, band k % NB
    const int64_t col = cg * 256 + k / NB;
    if (col < cols)
      *reinterpret_cast<uint4*>(nib + col * npitch + mb * 16 * NB + (k % NB) * 16) =
          *reinterpret_cast<const uint4*>(onib + k * 16);
  }
  const int64_t col = cg * 256 + threadIdx.x;
  if (col < cols)
    *reinterpret_cast<uint32_t*>(sc + col * spitch + mb * 4) =
        *reinterpret_cast<const uint32_t*>(osc + threadIdx.x * 4);
}

template <int H, int MODE>
hipError_t dispatch_mbs(const void* src, int64_t rows, int64_t cols, int axis, void* nib,
                        void* sc, void* mbs, hipStream_t st) {
  if (axis == 0) {
    const int64_t nblocks = rows * (cols / 32);
    hipLaunchKernelGGL((quant_mbs_row_kernel<H, MODE>), dim3((unsigned)((nblocks + 255) / 256)),
                       dim3(256), 0, st, static_cast<const uint4*>(src), nblocks,
                       static_cast<uint4*>(nib), static_cast<uint8_t*>(sc),
                       static_cast<uint8_t*>(mbs));
  } else if (cols % 4 == 0 && (uintptr_t)nib % 16 == 0 && (uintptr_t)sc % 4 == 0) {
    const int64_t grid = (rows / 128) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_mbs_col_staged_kernel<H, MODE>), dim3((unsigned)grid), dim3(256), 0,
                       st, static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc),
                       static_cast<uint8_t*>(mbs));
  } else {
    const int64_t grid = (rows / 128) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_mbs_col_kernel<H, MODE>), dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const uint16_t*>(src), rows, cols, static_cast<uint8_t*>(nib),
                       static_cast<uint8_t*>(sc), static_cast<uint8_t*>(mbs));
  }
  return hipGetLastError();
}

template <int H, int MODE>
hipError_t dispatch_axis(const void* src, int64_t rows, int64_t cols, int axis, void* nib,
                         void* sc, hipStream_t st) {
  const dim3 blk(256);
  if (axis == 0) {
    const int64_t nblocks = rows * (cols / 32);
    const int64_t grid = (nblocks + 255) / 256;
    // Launched on its own, the lane-contiguous kernel is as fast or faster at
    // every size measured (back to back over six buffer sets: 8192 x 4096
    // 15.3 against 16.8 us, 6144 x 4096 12.1 against 12.9 us, 28672 x 4096
    // equal). Inside the Llama step, right after a GEMM, the one-block-per-
    // thread body is faster below 2^20 blocks; the two-operand launch
    // (launch_quantize_pair) keeps that choice.
    if (nblocks % 256 == 0)
      hipLaunchKernelGGL((quant_row_lc_kernel<H, MODE>), dim3((unsigned)grid), blk, 0, st,
                         static_cast<const uint4*>(src), static_cast<uint4*>(nib),
                         static_cast<uint8_t*>(sc));
    else
      hipLaunchKernelGGL((quant_row_kernel<H, MODE>), dim3((unsigned)grid), blk, 0, st,
                         static_cast<const uint4*>(src), nblocks, static_cast<uint4*>(nib),
                         static_cast<uint8_t*>(sc));
  } else if (axis == 1) {
    if (rows % 256 == 0 && cols % 4 == 0 && ((uintptr_t)sc % 8 == 0)) {
      const int64_t grid = (rows / 256) * ((cols + 255) / 256);
      hipLaunchKernelGGL((quant_col_staged_kernel<H, MODE, 8>), dim3((unsigned)grid), dim3(512),
                         0, st, static_cast<const uint16_t*>(src), rows, cols,
                         static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc), nullptr);
    } else if (rows % 128 == 0 && cols % 4 == 0 && ((uintptr_t)sc % 4 == 0)) {
      const int64_t grid = (rows / 128) * ((cols + 255) / 256);
      hipLaunchKernelGGL((quant_col_staged_kernel<H, MODE, 4>), dim3((unsigned)grid), blk, 0, st,
                         static_cast<const uint16_t*>(src), rows, cols,
                         static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc), nullptr);
    } else if (cols % 8 == 0) {
      const int64_t grid = ((rows / 32 + 3) / 4) * ((cols + 511) / 512);
      hipLaunchKernelGGL((quant_col_kernel<H, MODE>), dim3((unsigned)grid), blk, 0, st,
                         static_cast<const uint16_t*>(src), rows, cols,
                         static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc));
    } else {
      const int64_t grid = (rows / 32) * ((cols + 255) / 256);
      hipLaunchKernelGGL((quant_col_scalar_kernel<H, MODE>), dim3((unsigned)grid), blk, 0, st,
                         static_cast<const uint16_t*>(src), rows, cols,
                         static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc), nullptr);
    }
  } else if (cols % 256 == 0) {
    const int64_t grid = (rows / 32) * (cols / 256);
    hipLaunchKernelGGL((quant_2d_lc_kernel<H, MODE>), dim3((unsigned)grid), blk, 0, st,
                       static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc));
  } else {
    const int64_t grid = (rows / 32) * ((cols / 32 + 7) / 8);
    hipLaunchKernelGGL((quant_2d_kernel<H, MODE>), dim3((unsigned)grid), blk, 0, st,
                       static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc));
  }
  return hipGetLastError();
}

template <int H>
hipError_t dispatch_mode(const void* src, int64_t rows, int64_t cols, int axis, int mode,
                         void* nib, void* sc, hipStream_t st) {
  return mode == kCeil ? dispatch_axis<H, kCeil>(src, rows, cols, axis, nib, sc, st)
                       : dispatch_axis<H, kOcpFloor>(src, rows, cols, axis, nib, sc, st);
}

template <int H, int MODE>
hipError_t dispatch_dual(const void* src, int64_t rows, int64_t cols, void* rnib, void* rsc,
                         void* cnib, void* csc, hipStream_t st) {
  const bool fast = rows % 128 == 0 && cols % 256 == 0 && ((uintptr_t)rsc % 8 == 0) &&
                    ((uintptr_t)csc % 4 == 0);
  if (!fast) {
    hipError_t e = dispatch_axis<H, MODE>(src, rows, cols, 0, rnib, rsc, st);
    if (e != hipSuccess) return e;
    return dispatch_axis<H, MODE>(src, rows, cols, 1, cnib, csc, st);
  }
  const auto* s16 = static_cast<const uint16_t*>(src);
  auto* rn = static_cast<uint8_t*>(rnib);
  auto* rs = static_cast<uint8_t*>(rsc);
  auto* cn = static_cast<uint8_t*>(cnib);
  auto* cs = static_cast<uint8_t*>(csc);
  // Four bands per work-group: with both outputs staged, eight bands would
  // take 68 KB of LDS per work-group and leave too few waves per CU.
  hipLaunchKernelGGL((quant_dual_kernel<H, MODE, 4>), dim3((unsigned)((rows / 128) * (cols / 256))),
                     dim3(256), 0, st, s16, rows, cols, rn, rs, cn, cs);
  return hipGetLastError();
}

// ------------------------------------------------ comparison arms
// [P1] reports that random Hadamard transforms and stochastic rounding
// diverge under full MXFP4 training (quick-read block, section A.2,
// hypothesis H2); these arms quantize with them so their error can be
// measured beside the deterministic H16 + round-to-nearest operand. The
// random numbers are inputs.
//
// Random signs (RS): the operand of diag(s) x, s_i = -1 where bit 0 of
// signs[i] is set, i along the blocked axis; a bf16 sign flip is exact, so
// the kernels flip the loaded bits and then run the plain rotation and
// encode. Row blocks: one thread per 32-block (the block's 32 sign bytes
// come from L2; every row shares them). Column blocks: the column kernels
// with their RS flag (one sign per row, the same for a whole wave).
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_rs_row_kernel(const uint4* __restrict__ src,
                                                           int64_t nblocks, int64_t ncb,
                                                           const uint4* __restrict__ signs,
                                                           uint4* __restrict__ nib,
                                                           uint8_t* __restrict__ sc) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  const int64_t cb = b % ncb;
  const uint4 s0 = signs[cb * 2], s1 = signs[cb * 2 + 1];
  const uint32_t sw[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
  uint4 q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    q[j] = src[b * 4 + j];
    // bf16 dword k of the block holds elements 2k, 2k + 1; sign byte i sits
    // in sw[i / 4] at bit 8 (i % 4)
    uint32_t* d = reinterpret_cast<uint32_t*>(&q[j]);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int k = 4 * j + t;
      const uint32_t w = sw[k >> 1] >> (16 * (k & 1));
      d[t] ^= ((w & 1u) << 15) | (((w >> 8) & 1u) << 31);
    }
  }
  float v[32];
  unpack64B(q, v);
  butterfly32<H>(v);
  uint4 out;
  uint32_t s;
  encode_block_sh<MODE, kScaleShift<H>>(v, out, s);
  nib[b] = out;
  sc[b] = (uint8_t)s;
}

// Stochastic rounding (SR) of one rotated value y in a finite block with
// E8M0 byte s (E = s - 127), with one uniform 32-bit integer u:
// a = |y| 2^-E; below 6, between the neighbouring grid values
// g_lo <= a < g_hi, round up exactly when u < p 2^32 with
// p = (a - g_lo) / (g_hi - g_lo), i.e. with probability p; a >= 6 gives 6.
// In fp32 and exact: the multiply by 2^-E is exact unless its result falls
// below 2^-126 with bits lost, a - g_lo is exact (g_lo = 0, or
// g_hi <= 2 g_lo), the gap is 0.5, 1 or 2, and for an fp32 p < 1 the
// threshold t = p 2^32 <= 2^32 - 2^8, so u < t is u < ceil(t) as integers.
// Where the multiply loses bits, the exact threshold 2^33 a is below 2^-93:
// only u = 0 rounds up, and it does whenever y != 0, which the limit of at
// least 1 for a non-zero y in the lowest interval gives also when the
// product rounds to 0.
// Returns the 4-bit code (sign of y kept).
__device__ __forceinline__ uint32_t sr_code(float y, uint32_t s, uint32_t u) {
  const float inv = s == 254u ? __uint_as_float(0x00400000u) : __uint_as_float((254u - s) << 23);
  const float a = fabsf(y * inv);
  const int lo = (a >= 0.5f) + (a >= 1.0f) + (a >= 1.5f) + (a >= 2.0f) + (a >= 3.0f) +
                 (a >= 4.0f) + (a >= 6.0f);
  const float glo = lo < 4 ? 0.5f * (float)lo : (lo == 4 ? 2.0f : (lo == 5 ? 3.0f : 4.0f));
  const float k = lo < 4 ? 8589934592.0f : (lo < 6 ? 4294967296.0f : 2147483648.0f);
  const float t = lo >= 7 ? 0.0f : (a - glo) * k;
  const uint32_t nz = (lo == 0 && (__float_as_uint(y) & 0x7FFFFFFFu) != 0u) ? 1u : 0u;
  const uint32_t lim = max((uint32_t)ceilf(t), nz);
  const uint32_t mag = lo >= 7 ? 7u : (uint32_t)lo + (u < lim ? 1u : 0u);
  return mag | ((__float_as_uint(y) >> 28) & 8u);
}

// 32 rotated values and their 32 random integers -> (nibbles, scale byte),
// with the E8M0 rule of the round-to-nearest operand.
template <int MODE>
__device__ __forceinline__ void sr_block(const float (&v)[32], const uint32_t (&u)[32], uint4& nib,
                                         uint32_t& s) {
  s = e8m0_byte<MODE>(amax_bits_n<32>(v));
  if (s == 255u) {
    nib = make_uint4(0, 0, 0, 0);
    return;
  }
  uint32_t w[4];
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 8; ++k) r |= sr_code(v[8 * d + k], s, u[8 * d + k]) << (4 * k);
    w[d] = r;
  }
  nib = make_uint4(w[0], w[1], w[2], w[3]);
}

// SR, row blocks: one thread per 32-block (64 source bytes, 128 random bytes).
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_sr_row_kernel(const uint4* __restrict__ src,
                                                           int64_t nblocks,
                                                           const uint4* __restrict__ rnd,
                                                           uint4* __restrict__ nib,
                                                           uint8_t* __restrict__ sc) {
  const int64_t b = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (b >= nblocks) return;
  uint4 q[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) q[j] = src[b * 4 + j];
  uint32_t u[32];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint4 t = rnd[b * 8 + j];
    u[4 * j] = t.x; u[4 * j + 1] = t.y; u[4 * j + 2] = t.z; u[4 * j + 3] = t.w;
  }
  float v[32];
  unpack64B(q, v);
  hadamard32<H>(v);
  uint4 out;
  uint32_t s;
  sr_block<MODE>(v, u, out, s);
  nib[b] = out;
  sc[b] = (uint8_t)s;
}

// SR, column blocks: one thread per (column, 32-row band); source and random
// loads are coalesced across the threads of a row.
template <int H, int MODE>
__global__ __launch_bounds__(256) void quant_sr_col_kernel(const uint16_t* __restrict__ src,
                                                           int64_t rows, int64_t cols,
                                                           const uint32_t* __restrict__ rnd,
                                                           uint8_t* __restrict__ nib,
                                                           uint8_t* __restrict__ sc) {
  const int64_t ncg = (cols + 255) / 256;
  const int64_t c = ((int64_t)blockIdx.x % ncg) * 256 + threadIdx.x;
  const int64_t band = (int64_t)blockIdx.x / ncg;
  if (c >= cols || band * 32 >= rows) return;
  float v[32];
  uint32_t u[32];
#pragma unroll
  for (int r = 0; r < 32; ++r) {
    const int64_t e = (band * 32 + r) * cols + c;
    v[r] = __uint_as_float((uint32_t)src[e] << 16);
    u[r] = rnd[e];
  }
  hadamard32<H>(v);
  uint4 out;
  uint32_t s;
  sr_block<MODE>(v, u, out, s);
  *reinterpret_cast<uint4*>(nib + c * (rows / 2) + band * 16) = out;
  sc[c * (rows / 32) + band] = (uint8_t)s;
}

template <int H, int MODE>
hipError_t dispatch_rs(const void* src, int64_t rows, int64_t cols, int axis, const void* signs,
                       void* nib, void* sc, hipStream_t st) {
  const auto* sg = static_cast<const uint8_t*>(signs);
  if (axis == 0) {
    const int64_t ncb = cols / 32, nblocks = rows * ncb;
    hipLaunchKernelGGL((quant_rs_row_kernel<H, MODE>), dim3((unsigned)((nblocks + 255) / 256)),
                       dim3(256), 0, st, static_cast<const uint4*>(src), nblocks, ncb,
                       static_cast<const uint4*>(signs), static_cast<uint4*>(nib),
                       static_cast<uint8_t*>(sc));
  } else if (rows % 128 == 0 && cols % 4 == 0 && (uintptr_t)sc % 4 == 0) {
    const int64_t grid = (rows / 128) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_col_staged_kernel<H, MODE, 4, true>), dim3((unsigned)grid),
                       dim3(256), 0, st, static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc), sg);
  } else {
    const int64_t grid = (rows / 32) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_col_scalar_kernel<H, MODE, true>), dim3((unsigned)grid), dim3(256),
                       0, st, static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<uint8_t*>(nib), static_cast<uint8_t*>(sc), sg);
  }
  return hipGetLastError();
}

template <int H, int MODE>
hipError_t dispatch_sr(const void* src, int64_t rows, int64_t cols, int axis, const void* rnd,
                       void* nib, void* sc, hipStream_t st) {
  if (axis == 0) {
    const int64_t nblocks = rows * (cols / 32);
    hipLaunchKernelGGL((quant_sr_row_kernel<H, MODE>), dim3((unsigned)((nblocks + 255) / 256)),
                       dim3(256), 0, st, static_cast<const uint4*>(src), nblocks,
                       static_cast<const uint4*>(rnd), static_cast<uint4*>(nib),
                       static_cast<uint8_t*>(sc));
  } else {
    const int64_t grid = (rows / 32) * ((cols + 255) / 256);
    hipLaunchKernelGGL((quant_sr_col_kernel<H, MODE>), dim3((unsigned)grid), dim3(256), 0, st,
                       static_cast<const uint16_t*>(src), rows, cols,
                       static_cast<const uint32_t*>(rnd), static_cast<uint8_t*>(nib),
                       static_cast<uint8_t*>(sc));
  }
  return hipGetLastError();
}

// ------------------------------------------------ two operands in one launch
// A product quantizes two operands; one launch over both grids saves a
// launch's ramp and tail. Work-groups [0, ga) run the first job's kernel
// body, the rest the second's (the column operand first when the pair mixes
// a row and a column operand). Both bodies run with 512-thread work-groups: the
// row kernels take 512 blocks per work-group (one per thread, or 64 per
// wave in the lane-contiguous form), the column kernel its 8-band staged
// form. Each body and its results are exactly those of its own launch.
struct QJob {
  const void* src;
  int64_t rows, cols;
  void* nib;
  void* sc;
};

template <int H, int MODE>
struct RowBody {
  static int64_t groups(const QJob& j) { return (j.rows * (j.cols / 32) + 511) / 512; }
  __device__ static void run(const QJob& j, int64_t wg) {
    row_block<H, MODE>(static_cast<const uint4*>(j.src), j.rows * (j.cols / 32),
                       static_cast<uint4*>(j.nib), static_cast<uint8_t*>(j.sc),
                       wg * 512 + threadIdx.x);
  }
};

template <int H, int MODE>
struct RowLcBody {  // blocks % 512 == 0
  static int64_t groups(const QJob& j) { return j.rows * (j.cols / 32) / 512; }
  __device__ static void run(const QJob& j, int64_t wg) {
    row_lc_wave<H, MODE>(static_cast<const uint4*>(j.src), static_cast<uint4*>(j.nib),
                         static_cast<uint8_t*>(j.sc), (wg * 8 + (threadIdx.x >> 6)) * 64,
                         threadIdx.x & 63);
  }
};

template <int H, int MODE>
struct ColBody {  // rows % 256 == 0, cols % 4 == 0, scales 8-byte aligned
  static int64_t groups(const QJob& j) { return (j.rows / 256) * ((j.cols + 255) / 256); }
  __device__ static void run(const QJob& j, int64_t wg) {
    col_staged_wg<H, MODE, 8, false>(static_cast<const uint16_t*>(j.src), j.rows, j.cols,
                                     static_cast<uint8_t*>(j.nib), static_cast<uint8_t*>(j.sc),
                                     nullptr, wg);
  }
};

template <class BA, class BB>
__global__ __launch_bounds__(512) void quant_pair_kernel(QJob a, QJob b, int64_t ga) {
  const int64_t wg = blockIdx.x;
  if (wg < ga)
    BA::run(a, wg);
  else
    BB::run(b, wg - ga);
}

// Which body serves an operand in a pair launch: 0 row, 1 row lane-
// contiguous, 2 column; -1 when its shape needs a kernel of its own. Rows:
// lane-contiguous above 2^20 blocks only; in the Llama step (after a GEMM)
// it made the qkv pair of 8192 x 4096 and 6144 x 4096 slower (34.8 against
// 29.2 us), unlike a launch on its own (dispatch_axis).
int pair_kind(int64_t rows, int64_t cols, int axis, const void* sc) {
  if (axis == 0) {
    const int64_t nblocks = rows * (cols / 32);
    return (nblocks % 512 == 0 && nblocks > (int64_t(1) << 20)) ? 1 : 0;
  }
  if (axis == 1 && rows % 256 == 0 && cols % 4 == 0 && ((uintptr_t)sc % 8 == 0)) return 2;
  return -1;
}

template <int H, int MODE, class BA>
hipError_t pair_b(const QJob& a, const QJob& b, int kb, hipStream_t st) {
  const int64_t ga = BA::groups(a);
  const auto go = [&](auto bb) {
    using BB = decltype(bb);
    hipLaunchKernelGGL((quant_pair_kernel<BA, BB>), dim3((unsigned)(ga + BB::groups(b))),
                       dim3(512), 0, st, a, b, ga);
    return hipGetLastError();
  };
  if (kb == 0) return go(RowBody<H, MODE>{});
  if (kb == 1) return go(RowLcBody<H, MODE>{});
  return go(ColBody<H, MODE>{});
}

template <int H, int MODE>
hipError_t dispatch_pair(const QJob& a, int axa, const QJob& b, int axb, hipStream_t st) {
  const int ka = pair_kind(a.rows, a.cols, axa, a.sc), kb = pair_kind(b.rows, b.cols, axb, b.sc);
  if (ka < 0 || kb < 0) {
    hipError_t e = dispatch_axis<H, MODE>(a.src, a.rows, a.cols, axa, a.nib, a.sc, st);
    if (e != hipSuccess) return e;
    return dispatch_axis<H, MODE>(b.src, b.rows, b.cols, axb, b.nib, b.sc, st);
  }
  if (ka != 2 && kb == 2) {
    // A row operand with a column one: the column body's work-groups (128
    // KiB of source each, against 32 KiB for a row work-group) go first, so
    // the launch ends on the short ones. On the down-projection Dgrad pair
    // (8192 x 4096 row, 4096 x 14336 column) 47.6 -> 42.0 us.
    if (ka == 0) return pair_b<H, MODE, ColBody<H, MODE>>(b, a, 0, st);
    return pair_b<H, MODE, ColBody<H, MODE>>(b, a, 1, st);
  }
  if (ka == 0) return pair_b<H, MODE, RowBody<H, MODE>>(a, b, kb, st);
  if (ka == 1) return pair_b<H, MODE, RowLcBody<H, MODE>>(a, b, kb, st);
  return pair_b<H, MODE, ColBody<H, MODE>>(a, b, kb, st);
}

template <int H>
hipError_t dispatch_pair_mode(const QJob& a, int axa, const QJob& b, int axb, int mode,
                              hipStream_t st) {
  return mode == kCeil ? dispatch_pair<H, kCeil>(a, axa, b, axb, st)
                       : dispatch_pair<H, kOcpFloor>(a, axa, b, axb, st);
}

}  // namespace

hipError_t launch_quantize_pair(const void* src_a, int64_t rows_a, int64_t cols_a, int axis_a,
                                void* nib_a, void* sc_a, const void* src_b, int64_t rows_b,
                                int64_t cols_b, int axis_b, void* nib_b, void* sc_b,
                                int hadamard, int scale_mode, hipStream_t stream) {
  const QJob a{src_a, rows_a, cols_a, nib_a, sc_a}, b{src_b, rows_b, cols_b, nib_b, sc_b};
  switch (hadamard) {
    case 16: return dispatch_pair_mode<16>(a, axis_a, b, axis_b, scale_mode, stream);
    case 32: return dispatch_pair_mode<32>(a, axis_a, b, axis_b, scale_mode, stream);
    default: return dispatch_pair_mode<0>(a, axis_a, b, axis_b, scale_mode, stream);
  }
}

hipError_t launch_quantize(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                           int scale_mode, void* nib, void* sc, hipStream_t stream) {
  switch (hadamard) {
    case 16: return dispatch_mode<16>(src, rows, cols, axis, scale_mode, nib, sc, stream);
    case 32: return dispatch_mode<32>(src, rows, cols, axis, scale_mode, nib, sc, stream);
    default: return dispatch_mode<0>(src, rows, cols, axis, scale_mode, nib, sc, stream);
  }
}

hipError_t launch_quantize_dual(const void* src, int64_t rows, int64_t cols, int hadamard,
                                int scale_mode, void* rnib, void* rsc, void* cnib, void* csc,
                                hipStream_t stream) {
  const bool ceil = scale_mode == kCeil;
  switch (hadamard) {
    case 16: return ceil ? dispatch_dual<16, kCeil>(src, rows, cols, rnib, rsc, cnib, csc, stream)
                         : dispatch_dual<16, kOcpFloor>(src, rows, cols, rnib, rsc, cnib, csc, stream);
    case 32: return ceil ? dispatch_dual<32, kCeil>(src, rows, cols, rnib, rsc, cnib, csc, stream)
                         : dispatch_dual<32, kOcpFloor>(src, rows, cols, rnib, rsc, cnib, csc, stream);
    default: return ceil ? dispatch_dual<0, kCeil>(src, rows, cols, rnib, rsc, cnib, csc, stream)
                         : dispatch_dual<0, kOcpFloor>(src, rows, cols, rnib, rsc, cnib, csc, stream);
  }
}

hipError_t launch_quantize_of(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, void* nib, void* sc, hipStream_t stream) {
  const bool ceil = scale_mode == kCeil;
  switch (hadamard) {
    case 16: return ceil ? dispatch_of<16, kCeil>(src, rows, cols, axis, nib, sc, stream)
                         : dispatch_of<16, kOcpFloor>(src, rows, cols, axis, nib, sc, stream);
    case 32: return ceil ? dispatch_of<32, kCeil>(src, rows, cols, axis, nib, sc, stream)
                         : dispatch_of<32, kOcpFloor>(src, rows, cols, axis, nib, sc, stream);
    default: return ceil ? dispatch_of<0, kCeil>(src, rows, cols, axis, nib, sc, stream)
                         : dispatch_of<0, kOcpFloor>(src, rows, cols, axis, nib, sc, stream);
  }
}

hipError_t launch_quantize_mbs(const void* src, int64_t rows, int64_t cols, int axis,
                               int hadamard, int scale_mode, void* nib, void* sc, void* mbs,
                               hipStream_t stream) {
  const bool ceil = scale_mode == kCeil;
  switch (hadamard) {
    case 16: return ceil ? dispatch_mbs<16, kCeil>(src, rows, cols, axis, nib, sc, mbs, stream)
                         : dispatch_mbs<16, kOcpFloor>(src, rows, cols, axis, nib, sc, mbs, stream);
    case 32: return ceil ? dispatch_mbs<32, kCeil>(src, rows, cols, axis, nib, sc, mbs, stream)
                         : dispatch_mbs<32, kOcpFloor>(src, rows, cols, axis, nib, sc, mbs, stream);
    default: return ceil ? dispatch_mbs<0, kCeil>(src, rows, cols, axis, nib, sc, mbs, stream)
                         : dispatch_mbs<0, kOcpFloor>(src, rows, cols, axis, nib, sc, mbs, stream);
  }
}

hipError_t launch_quantize_rs(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, const void* signs, void* nib, void* sc,
                              hipStream_t stream) {
  const bool ceil = scale_mode == kCeil;
  switch (hadamard) {
    case 16: return ceil ? dispatch_rs<16, kCeil>(src, rows, cols, axis, signs, nib, sc, stream)
                         : dispatch_rs<16, kOcpFloor>(src, rows, cols, axis, signs, nib, sc, stream);
    case 32: return ceil ? dispatch_rs<32, kCeil>(src, rows, cols, axis, signs, nib, sc, stream)
                         : dispatch_rs<32, kOcpFloor>(src, rows, cols, axis, signs, nib, sc, stream);
    default: return ceil ? dispatch_rs<0, kCeil>(src, rows, cols, axis, signs, nib, sc, stream)
                         : dispatch_rs<0, kOcpFloor>(src, rows, cols, axis, signs, nib, sc, stream);
  }
}

hipError_t launch_quantize_sr(const void* src, int64_t rows, int64_t cols, int axis, int hadamard,
                              int scale_mode, const void* rnd, void* nib, void* sc,
                              hipStream_t stream) {
  const bool ceil = scale_mode == kCeil;
  switch (hadamard) {
    case 16: return ceil ? dispatch_sr<16, kCeil>(src, rows, cols, axis, rnd, nib, sc, stream)
                         : dispatch_sr<16, kOcpFloor>(src, rows, cols, axis, rnd, nib, sc, stream);
    case 32: return ceil ? dispatch_sr<32, kCeil>(src, rows, cols, axis, rnd, nib, sc, stream)
                         : dispatch_sr<32, kOcpFloor>(src, rows, cols, axis, rnd, nib, sc, stream);
    default: return ceil ? dispatch_sr<0, kCeil>(src, rows, cols, axis, rnd, nib, sc, stream)
                         : dispatch_sr<0, kOcpFloor>(src, rows, cols, axis, rnd, nib, sc, stream);
  }
}

}  // namespace mx
