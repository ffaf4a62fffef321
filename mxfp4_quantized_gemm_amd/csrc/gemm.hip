// MXFP4 GEMM on gfx950's block-scaled FP4 MFMA (MI355X).
//
// C[M][N] = sum_k deqA[m][k] * deqB[n][k], with deq = E2M1 * 2^(E8M0 - 127)
// per 32-element block along k, accumulated in fp32.
// Pages cited: [P1] "Pretraining Large Language Models with MXFP4 on Native
// FP4 Hardware" (arXiv:2605.09825 summary), section A.2 (MXFP4 GEMM kernels
// replace the FP8 GEMMs of the linear layers); [P3] "Decomposing MXFP4
// quantization error" blog (arXiv:2605.20402): native MXFP4 uses the E2M1
// grid, E8M0 block scales and FP32 accumulation.
//
// Instruction: v_mfma_scale_f32_32x32x64_f8f6f4 with both operands in FP4
// (cbsz = blgp = 4). Lane l supplies row (l % 32) and the 32 k-values
// [32 * (l / 32), +32) of a 64-deep k-step as 16 packed bytes (element 2j
// in the low nibble of byte j, exactly the packed operand layout), plus the
// E8M0 byte of that 32-block in the byte of its scale register picked by
// op_sel. Output lane l, register r holds C[8 * (r / 4) + 4 * (l / 32) + r % 4][l % 32].
//
// Three kernels. For K % 2048 == 0 (every Llama-shaped product) the persistent
// LDS-DMA kernel (namespace dm, below) runs 256 x 256 tiles whose operands go
// straight from global memory to LDS; for K % 256 == 0 the register-staged
// large-tile kernel (namespace lt) runs the same tiles with 256- or 128-deep
// k-tiles; both need 32-bit operand offsets. The general kernel here serves
// any K % 32 == 0 and any M, N: a 256-thread work-group (4 waves, 2 x 2)
// computes a 128 x 128 tile of C; each wave a 64 x 64 sub-tile (2 x 2 MFMA
// tiles, 64 fp32 accumulators per lane). The k-loop steps 256 elements (128
// bytes of nibbles per row, 8 scale bytes per row). Tiles of A and B are
// staged in LDS with a 16-byte-chunk XOR swizzle (chunk c of row r stored at
// c ^ (r & 7)) so that the 32 rows read by one ds_read_b128 hit distinct
// banks. LDS is double-buffered: the global loads of tile k+1 are issued
// before the MFMAs of tile k and written to the other buffer after them,
// with one barrier per k-tile.
#include <hip/hip_runtime.h>
#include <atomic>
#include <stdint.h>

#include "internal.h"

namespace mx {
namespace {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));

constexpr int BM = 128, BN = 128;
constexpr int BKB = 128;                  // bytes of nibbles per row per k-tile (256 elements)
constexpr int BKS = 8;                    // scale bytes per row per k-tile
constexpr int TILE_A = BM * BKB;          // 16 KiB
constexpr int TILE_B = BN * BKB;          // 16 KiB
constexpr int STAGE = TILE_A + TILE_B + (BM + BN) * BKS;  // 34 KiB

__device__ __forceinline__ uint32_t bf16_rne(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

struct TileRegs {
  uint4 a[4], b[4];
  uint2 sa, sb;  // thread t < 128: A-row scales; t >= 128: B-row scales (one of the two used)
};

// Global -> registers for k-tile kt. Data chunk q = t + 256 i (i < 4) covers
// row q >> 3, 16-byte chunk q & 7 of the tile. Rows past M/N and chunks past
// K read as zero; scale bytes past M/N/K read as 127 (value 1: times a zero
// nibble gives 0, never 0 * NaN).
template <bool SCALE_VEC>
__device__ __forceinline__ void load_tile(TileRegs& R, const uint8_t* __restrict__ A,
                                          const uint8_t* __restrict__ As,
                                          const uint8_t* __restrict__ B,
                                          const uint8_t* __restrict__ Bs, int64_t m0, int64_t n0,
                                          int64_t M, int64_t N, int64_t kbytes, int64_t kblk,
                                          int kt, int t) {
  const int64_t kb0 = (int64_t)kt * BKB;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 3, c = q & 7;
    const int64_t kb = kb0 + c * 16;
    const bool kin = kb < kbytes;
    R.a[i] = (m0 + row < M && kin)
                 ? *reinterpret_cast<const uint4*>(A + (m0 + row) * kbytes + kb)
                 : make_uint4(0, 0, 0, 0);
    R.b[i] = (n0 + row < N && kin)
                 ? *reinterpret_cast<const uint4*>(B + (n0 + row) * kbytes + kb)
                 : make_uint4(0, 0, 0, 0);
  }
  const int srow = t & 127;
  const bool isA = t < 128;
  const int64_t grow = (isA ? m0 : n0) + srow;
  const int64_t glim = isA ? M : N;
  const uint8_t* S = isA ? As : Bs;
  const int64_t sb0 = (int64_t)kt * BKS;
  uint2 sv = make_uint2(0x7f7f7f7fu, 0x7f7f7f7fu);
  if (grow < glim) {
    if (SCALE_VEC && sb0 + BKS <= kblk) {
      sv = *reinterpret_cast<const uint2*>(S + grow * kblk + sb0);
    } else {
      uint32_t w[2] = {0x7f7f7f7fu, 0x7f7f7f7fu};
#pragma unroll
      for (int j = 0; j < BKS; ++j) {
        if (sb0 + j < kblk) {
          const uint32_t byte = S[grow * kblk + sb0 + j];
          w[j >> 2] = (w[j >> 2] & ~(0xffu << (8 * (j & 3)))) | (byte << (8 * (j & 3)));
        }
      }
      sv = make_uint2(w[0], w[1]);
    }
  }
  R.sa = sv;
}

__device__ __forceinline__ void store_tile(const TileRegs& R, uint8_t* stage, int t) {
  uint8_t* la = stage;
  uint8_t* lb = stage + TILE_A;
  uint8_t* ls = stage + TILE_A + TILE_B;  // [BM + BN][8]: A rows then B rows
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int q = t + 256 * i;
    const int row = q >> 3, c = q & 7;
    const int off = row * BKB + ((c ^ (row & 7)) << 4);
    *reinterpret_cast<uint4*>(la + off) = R.a[i];
    *reinterpret_cast<uint4*>(lb + off) = R.b[i];
  }
  *reinterpret_cast<uint2*>(ls + t * BKS) = R.sa;
}

__device__ __forceinline__ v8i frag(const uint8_t* tile, int row, int chunk) {
  const uint4 q = *reinterpret_cast<const uint4*>(tile + row * BKB + ((chunk ^ (row & 7)) << 4));
  v8i r = {(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  return r;
}

template <int OPSEL>
__device__ __forceinline__ v16f mfma(v8i a, v8i b, v16f c, int sa, int sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 4, 4, OPSEL, sa, OPSEL, sb);
}

__device__ __forceinline__ void compute_tile(const uint8_t* stage, v16f (&acc)[2][2], int wm,
                                             int wn, int lane) {
  const uint8_t* la = stage;
  const uint8_t* lb = stage + TILE_A;
  const uint8_t* ls = stage + TILE_A + TILE_B;
  const int half = lane >> 5;
  // Scale words: the 8 bytes of the row, shifted so that byte 2s (s = k-step)
  // is the byte of this lane's 32-block: blocks 2s + half.
  uint32_t sa[2][2], sb[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ar = wm * 64 + i * 32 + (lane & 31);
    const int br = wn * 64 + i * 32 + (lane & 31);
    const uint64_t va = *reinterpret_cast<const uint64_t*>(ls + ar * BKS) >> (8 * half);
    const uint64_t vb = *reinterpret_cast<const uint64_t*>(ls + (BM + br) * BKS) >> (8 * half);
    sa[i][0] = (uint32_t)va;
    sa[i][1] = (uint32_t)(va >> 32);
    sb[i][0] = (uint32_t)vb;
    sb[i][1] = (uint32_t)(vb >> 32);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    v8i af[2], bf[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      af[i] = frag(la, wm * 64 + i * 32 + (lane & 31), 2 * s + half);
      bf[i] = frag(lb, wn * 64 + i * 32 + (lane & 31), 2 * s + half);
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int wa = (int)sa[i][s >> 1], wb = (int)sb[j][s >> 1];
        acc[i][j] = (s & 1) ? mfma<2>(af[i], bf[j], acc[i][j], wa, wb)
                            : mfma<0>(af[i], bf[j], acc[i][j], wa, wb);
      }
  }
}

template <int OUT, bool SCALE_VEC>
__global__ __launch_bounds__(256) void gemm_kernel(const uint8_t* __restrict__ A,
                                                   const uint8_t* __restrict__ As,
                                                   const uint8_t* __restrict__ B,
                                                   const uint8_t* __restrict__ Bs, int64_t M,
                                                   int64_t N, int64_t K, void* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t ntn = (N + BN - 1) / BN;
  const int64_t tm = (int64_t)blockIdx.x / ntn, tn = (int64_t)blockIdx.x % ntn;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t kbytes = K / 2, kblk = K / 32;
  const int nkt = (int)((kbytes + BKB - 1) / BKB);

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileRegs R;
  load_tile<SCALE_VEC>(R, A, As, B, Bs, m0, n0, M, N, kbytes, kblk, 0, t);
  store_tile(R, lds, t);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) load_tile<SCALE_VEC>(R, A, As, B, Bs, m0, n0, M, N, kbytes, kblk, kt + 1, t);
    compute_tile(lds + (kt & 1) * STAGE, acc, wm, wn, lane);
    if (more) store_tile(R, lds + ((kt + 1) & 1) * STAGE, t);
    __syncthreads();
  }

  // Epilogue: lane holds column (lane & 31) of each 32 x 32 tile, rows
  // 8 * (r / 4) + 4 * (lane / 32) + r % 4.
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) {
          if (OUT == 0)
            static_cast<float*>(C)[row * N + col] = acc[i][j][r];
          else
            static_cast<uint16_t*>(C)[row * N + col] = (uint16_t)bf16_rne(acc[i][j][r]);
        }
      }
    }
}


// ==================================================== macro-block-scaled GEMM
// The product of two MBS operands ([P3] "three targeted fixes" section,
// MBS: x_hat = Q((1 + m) x) / (1 + m) per 128-element macro-block, the
// postscale undoing the prescale): C[m][n] = sum over macro-blocks g of
// P_g[m][n] / (cA[m][g] cB[n][g]), with P_g the MXFP4 product of the
// prescaled operands over the 128 k-values of g and c = 1 + mantissa / 256.
// The factor varies along k, so it cannot join the power-of-two E8M0
// scales: each macro-block is two MFMA k-steps accumulated into a temporary
// set of registers from zero, then added to the result times
// fl32(fl32(1 / cA) fl32(1 / cB)). Tiles and staging are the general
// kernel's (128 x 128, 4 waves of 64 x 64); each stage adds the
// reciprocals 1 / c of its two macro-blocks for the tile's A and B rows, as
// fp32 in LDS ([2][BM + BN]). K % 128 == 0; rows past M or N and a half
// k-tile past K take factor 1 (their products are zero).
constexpr int MBS_R = 2 * (BM + BN) * 4;    // reciprocals of one stage, bytes
constexpr int STAGE_MBS = STAGE + MBS_R;

__device__ __forceinline__ void load_mbs(float (&r)[2], const uint8_t* __restrict__ Am,
                                         const uint8_t* __restrict__ Bm, int64_t m0, int64_t n0,
                                         int64_t M, int64_t N, int64_t kmb, int kt, int t) {
  const int srow = t & 127;
  const bool isA = t < 128;
  const int64_t grow = (isA ? m0 : n0) + srow;
  const uint8_t* Mm = isA ? Am : Bm;
  const bool in = grow < (isA ? M : N);
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const int64_t mb = (int64_t)kt * 2 + g;
    const uint32_t m = (in && mb < kmb) ? Mm[grow * kmb + mb] : 0u;
    r[g] = 1.0f / (1.0f + (float)m * (1.0f / 256.0f));  // c exact in fp32, one rounded division
  }
}

__device__ __forceinline__ void store_mbs(const float (&r)[2], uint8_t* stage, int t) {
  float* lr = reinterpret_cast<float*>(stage + STAGE);
#pragma unroll
  for (int g = 0; g < 2; ++g) lr[g * (BM + BN) + t] = r[g];  // t < 128: A row t, else B row t - 128
}

__device__ __forceinline__ void compute_tile_mbs(const uint8_t* stage, v16f (&acc)[2][2], int wm,
                                                 int wn, int lane) {
  const uint8_t* la = stage;
  const uint8_t* lb = stage + TILE_A;
  const uint8_t* ls = stage + TILE_A + TILE_B;
  const float* lr = reinterpret_cast<const float*>(stage + STAGE);
  const int half = lane >> 5;
  uint32_t sa[2][2], sb[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int ar = wm * 64 + i * 32 + (lane & 31);
    const int br = wn * 64 + i * 32 + (lane & 31);
    const uint64_t va = *reinterpret_cast<const uint64_t*>(ls + ar * BKS) >> (8 * half);
    const uint64_t vb = *reinterpret_cast<const uint64_t*>(ls + (BM + br) * BKS) >> (8 * half);
    sa[i][0] = (uint32_t)va;
    sa[i][1] = (uint32_t)(va >> 32);
    sb[i][0] = (uint32_t)vb;
    sb[i][1] = (uint32_t)(vb >> 32);
  }
  const v16f zero = {};
#pragma unroll
  for (int g = 0; g < 2; ++g) {  // macro-block g: k-steps 2 g and 2 g + 1
    v16f tmp[2][2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int s = 2 * g + u;
      v8i af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        af[i] = frag(la, wm * 64 + i * 32 + (lane & 31), 2 * s + half);
        bf[i] = frag(lb, wn * 64 + i * 32 + (lane & 31), 2 * s + half);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int wa = (int)sa[i][s >> 1], wb = (int)sb[j][s >> 1];
          const v16f c = u == 0 ? zero : tmp[i][j];
          tmp[i][j] = (s & 1) ? mfma<2>(af[i], bf[j], c, wa, wb) : mfma<0>(af[i], bf[j], c, wa, wb);
        }
    }
    // lane: column (lane & 31) of each 32 x 32 tile, rows 8 q + 4 half + e
    float rb[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) rb[j] = lr[g * (BM + BN) + BM + wn * 64 + j * 32 + (lane & 31)];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float4 ra =
            *reinterpret_cast<const float4*>(lr + g * (BM + BN) + wm * 64 + i * 32 + 8 * q + 4 * half);
        const float rv[4] = {ra.x, ra.y, ra.z, ra.w};
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            acc[i][j][4 * q + e] = fmaf(tmp[i][j][4 * q + e], rv[e] * rb[j], acc[i][j][4 * q + e]);
      }
  }
}

template <int OUT, bool SCALE_VEC>
__global__ __launch_bounds__(256) void gemm_mbs_kernel(
    const uint8_t* __restrict__ A, const uint8_t* __restrict__ As, const uint8_t* __restrict__ Am,
    const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, const uint8_t* __restrict__ Bm,
    int64_t M, int64_t N, int64_t K, void* __restrict__ C) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE_MBS];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t ntn = (N + BN - 1) / BN;
  const int64_t tm = (int64_t)blockIdx.x / ntn, tn = (int64_t)blockIdx.x % ntn;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t kbytes = K / 2, kblk = K / 32, kmb = K / 128;
  const int nkt = (int)((kbytes + BKB - 1) / BKB);

  v16f acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  TileRegs R;
  float rm[2];
  load_tile<SCALE_VEC>(R, A, As, B, Bs, m0, n0, M, N, kbytes, kblk, 0, t);
  load_mbs(rm, Am, Bm, m0, n0, M, N, kmb, 0, t);
  store_tile(R, lds, t);
  store_mbs(rm, lds, t);
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const bool more = kt + 1 < nkt;
    if (more) {
      load_tile<SCALE_VEC>(R, A, As, B, Bs, m0, n0, M, N, kbytes, kblk, kt + 1, t);
      load_mbs(rm, Am, Bm, m0, n0, M, N, kmb, kt + 1, t);
    }
    compute_tile_mbs(lds + (kt & 1) * STAGE_MBS, acc, wm, wn, lane);
    if (more) {
      store_tile(R, lds + ((kt + 1) & 1) * STAGE_MBS, t);
      store_mbs(rm, lds + ((kt + 1) & 1) * STAGE_MBS, t);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * 64 + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        if (row < M) {
          if (OUT == 0)
            static_cast<float*>(C)[row * N + col] = acc[i][j][r];
          else
            static_cast<uint16_t*>(C)[row * N + col] = (uint16_t)bf16_rne(acc[i][j][r]);
        }
      }
    }
}

// ====================================================== large-tile kernel
// For K % 256 == 0 (every Llama shape). Templated on the wave layout: WM x WN
// waves per work-group, each computing TM x TN MFMA 32x32x64 tiles, so the
// work-group tile is (32 WM TM) x (32 WN TN); and on the k-tile depth, KB
// bytes of nibbles per operand row (64 or 128, i.e. 128 or 256 elements;
// 128 bytes reads whole cache lines).
//
// Operand roles are swapped in the MFMA (B as the instruction's first
// operand), so a lane's accumulator registers 4q..4q+3 hold four
// consecutive columns of one C row: the epilogue writes 16-byte vectors.
//
// LDS tiles are fragment-major: for each group of 32 rows, chunk column c
// (the rows' 16-byte chunks c) is 512 contiguous bytes padded to 544 (576 for
// 64-byte k-tiles). An MFMA fragment read is then 32 lanes x 16 contiguous
// bytes per half-wave and the staging writes are 16 lanes x 16 contiguous
// bytes; with the padding both run near the LDS peak (measured 188 and 245
// B/clk per CU, where row-major 16-byte writes ran at 76).
namespace lt {

// Output tiles are walked in groups of GROUP_M tile-rows (see tile_of).
constexpr int GROUP_M = 4;

// Staging registers use the native vector type: HIP's uint4 is a class
// whose copies lower to memcpy, which keeps the struct in scratch memory.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Work-group barrier that orders LDS only: global loads in flight (the
// prefetch of later k-tiles) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Per-thread global offsets (32-bit, relative to the operand base; the k-tile
// offset is added to the uniform base): chunk c = t % CPR of rows
// t / CPR + RSTEP i, clamped to the last row (results of clamped rows are
// never stored), and the scale rows d = t + NT i (A rows, then B rows; a d
// past the tile reloads a valid B row whose words go to a trash slot).
template <class G>
struct Offs {
  uint32_t a[G::CA], b[G::CB], s[G::SC];
};

// Buffer resources of the operands. Loads go through them with a 32-bit
// per-lane offset and the k-tile offset in a scalar register, so the
// per-lane offsets stay 32-bit and no 64-bit address arithmetic is needed
// per load. The record count is the operand's size: a load past it returns
// zero instead of touching memory (the clamped offsets never get there).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)(uint32_t)bytes,
                                           0x00020000);
}

// Scale rows d = t + NT i are rows of A for d < BM and rows of B after;
// BM is a multiple of 64, so the choice is uniform over a wave.
template <class G>
struct Src {
  rsrc_t a, b, s[G::SC];
};

template <class G>
__device__ __forceinline__ void make_src(Src<G>& S, const uint8_t* A, const uint8_t* As,
                                         const uint8_t* B, const uint8_t* Bs, int64_t M,
                                         int64_t N, int64_t kbytes, int64_t kblk, int wave) {
  S.a = make_rsrc(A, M * kbytes);
  S.b = make_rsrc(B, N * kbytes);
#pragma unroll
  for (int i = 0; i < G::SC; ++i) {
    const bool isA = 64 * wave + G::NT * i < G::BM;
    S.s[i] = isA ? make_rsrc(As, M * kblk) : make_rsrc(Bs, N * kblk);
  }
}

template <class G>
__device__ __forceinline__ void make_offsets(Offs<G>& O, int64_t m0, int64_t n0, int64_t M,
                                             int64_t N, int64_t kbytes, int64_t kblk, int t) {
  const int r0 = t / G::CPR, c = t % G::CPR;
#pragma unroll
  for (int i = 0; i < G::CA; ++i)
    O.a[i] = (uint32_t)(min(m0 + r0 + G::RSTEP * i, M - 1) * kbytes + c * 16);
#pragma unroll
  for (int i = 0; i < G::CB; ++i)
    O.b[i] = (uint32_t)(min(n0 + r0 + G::RSTEP * i, N - 1) * kbytes + c * 16);
#pragma unroll
  for (int i = 0; i < G::SC; ++i) {
    const int d = t + G::NT * i;
    O.s[i] = (uint32_t)(d < G::BM ? min(m0 + d, M - 1) * kblk
                                  : min(n0 + min(d - G::BM, G::BN - 1), N - 1) * kblk);
  }
}

template <int SB> struct ScalePair;
template <> struct ScalePair<8> { typedef u32x4 type; };
template <> struct ScalePair<4> { typedef u32x2 type; };

// Staging registers of one k-tile of A and B rows, and the scale bytes of
// the scale row for two consecutive k-tiles (even tile in the low half).
template <class G>
struct Regs {
  u32x4 a[G::CA], b[G::CB];
  typename ScalePair<G::SB>::type s[G::SC];
};

template <class G>
__device__ __forceinline__ void gload_data(Regs<G>& R, const Offs<G>& O, const Src<G>& S, int kt) {
  constexpr int KB = G::CPR * 16;
  const int ko = kt * KB;
#pragma unroll
  for (int i = 0; i < G::CA; ++i) R.a[i] = __builtin_amdgcn_raw_buffer_load_b128(S.a, O.a[i], ko, 0);
#pragma unroll
  for (int i = 0; i < G::CB; ++i) R.b[i] = __builtin_amdgcn_raw_buffer_load_b128(S.b, O.b[i], ko, 0);
}

// Scale bytes of the even k-tile kt and of kt + 1 in one load per scale row:
// a scale row holds SB bytes per k-tile, so a load of 2 SB bytes per lane
// touches half as many cache lines per byte as one k-tile's SB bytes would.
template <class G>
__device__ __forceinline__ void gload_scales(Regs<G>& R, const Offs<G>& O, const Src<G>& S,
                                             int kt) {
  const int so = kt * G::SB;
#pragma unroll
  for (int i = 0; i < G::SC; ++i) {
    if constexpr (G::SB == 8)
      R.s[i] = __builtin_amdgcn_raw_buffer_load_b128(S.s[i], O.s[i], so, 0);
    else
      R.s[i] = __builtin_amdgcn_raw_buffer_load_b64(S.s[i], O.s[i], so, 0);
  }
}

// Work-group id -> output tile. Consecutive work-group ids are dispatched
// round-robin over the 8 XCDs; the remap gives each XCD a contiguous range
// of logical tiles, walked in groups of GROUP_M tile-rows so that the tiles
// resident at once on one XCD share rows of A and columns of B in its L2.
template <int GM>
__device__ __forceinline__ void tile_of(int64_t wg, int64_t nwg, int64_t ntm, int64_t ntn,
                                        int64_t& tm, int64_t& tn) {
  const int64_t per = nwg / 8;
  int64_t lg = wg;
  if (wg < per * 8) lg = (wg % 8) * per + wg / 8;
  const int64_t width = (int64_t)GM * ntn;
  const int64_t g = lg / width;
  const int64_t first = g * GM;
  const int64_t gs = min(ntm - first, (int64_t)GM);
  const int64_t r = lg % width;
  tm = first + r % gs;
  tn = r / gs;
}

// Large-tile kernel, software pipelined. A 512-thread work-group (8 waves,
// 2 x 4) computes a 256 x 256 tile of C, each wave 128 x 64 (4 x 2 MFMA
// tiles, 128 fp32 accumulators per lane, in AGPRs). k-tiles are KB = 128
// (256-deep) or 64 (128-deep) bytes of every operand row; A and B rows are
// staged in LDS in the fragment-major layout above, double-buffered, loaded
// through buffer resources into staging registers. Within a k-tile:
//  * scale bytes are stored in LDS pre-split into an "even blocks" word and
//    an "odd blocks" word per row, laid out so that a lane's TM (TN) rows are
//    consecutive: one vector LDS read per operand per k-tile, and byte s of
//    the lane's word is its block for k-step s, so op_sel is the k-step;
//  * the fragment reads of k-step s+1, the LDS writes of the next k-tile and
//    the global loads of a later k-tile are interleaved one by one with the
//    MFMAs of k-step s (scheduling groups), instead of being left to the
//    scheduler, which bunches the reads behind the MFMAs;
//  * the barrier comes before the last k-step: its MFMAs (operands already
//    in registers) are issued after it, together with the first reads of the
//    next k-tile, so neither the barrier nor that read latency idles the
//    matrix cores;
//  * the next k-tile's staging registers are written to LDS early in the
//    k-tile (the other LDS buffer is free once the previous barrier passed),
//    then reloaded with a later k-tile (NS = 2 staging sets would run the
//    loads two k-tiles ahead; the 8-wave shape has registers for one).
template <int WM, int WN, int TM, int TN, int KB>
struct Cfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BM = 32 * WM * TM, BN = 32 * WN * TN;
  static constexpr int CPR = KB / 16;                    // 16-byte chunks per row
  static constexpr int SB = KB / 16;                     // scale bytes per row per k-tile
  static constexpr int KSTEPS = KB / 32;                 // MFMA k-steps (64 elements each)
  // Fragment-major tiles: per group of 32 rows, chunk column c holds the 32
  // rows' 16-byte chunk c back to back, padded to CP bytes. A 16-byte LDS
  // write serves 8 lanes per cycle over 32 four-byte banks; the 8 lanes hold
  // chunks c = 0..CPR-1 of 8 / CPR consecutive rows, at bank offsets
  // (CP / 4) c + 4 r mod 32, which are all distinct for a pitch of 512 + 16
  // bytes with 8 chunks per row and 512 + 32 with 4. Fragment reads take 16
  // consecutive rows of one chunk column and do not depend on the pitch.
  static constexpr int CP = KB == 128 ? 528 : 544;       // chunk-column pitch
  static constexpr int GP = (KB / 16) * CP;              // 32-row group pitch
  static constexpr int TA = (BM / 32) * GP, TB = (BN / 32) * GP;
  static constexpr int SOFF = TA + TB;                   // A scale words, then B scale words
  static constexpr int SBOFF = SOFF + BM * 8;
  static constexpr int TRASH = SBOFF + BN * 8;           // sink for surplus scale rows
  static constexpr int STAGE = TRASH + 16;
  static constexpr int RSTEP = NT / CPR;                 // rows between a thread's chunks
  static constexpr int CA = BM / RSTEP, CB = BN / RSTEP; // chunks per thread
  static constexpr int SC = (BM + BN + NT - 1) / NT;     // scale rows per thread
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0 && RSTEP % 32 == 0, "bad tiling");
  static_assert(KB == 64 || KB == 128, "k-tiles of 128 or 256 elements");
};

// LDS byte offsets (within a stage) of the even and odd scale words of the
// thread's scale rows. Row r = 32 (T g + i) + l of the A tile (T = TM rows
// per wave row g) goes to word ((32 g + l) 2 + h) T + i for parity h, so the
// lane (l, h) of wave row g finds its T words side by side; B likewise after
// the A words.
template <class G, int TM, int TN>
struct SPos {
  uint32_t e[G::SC], o[G::SC];
};

template <class G, int TM, int TN>
__device__ __forceinline__ void make_spos(SPos<G, TM, TN>& P, int t) {
#pragma unroll
  for (int i = 0; i < G::SC; ++i) {
    const int d = t + G::NT * i;
    if (d >= G::BM + G::BN) {
      // No row: the (redundant, clamped) load of this slot is written to the
      // trash words, so loads and stores stay unconditional.
      P.e[i] = P.o[i] = G::TRASH;
    } else if (d < G::BM) {
      const int g = d / (32 * TM), ii = (d / 32) % TM, l = d % 32;
      P.e[i] = G::SOFF + 4 * ((g * 32 + l) * 2 * TM + ii);
      P.o[i] = P.e[i] + 4 * TM;
    } else {
      const int e = d - G::BM;
      const int g = e / (32 * TN), jj = (e / 32) % TN, l = e % 32;
      P.e[i] = G::SBOFF + 4 * ((g * 32 + l) * 2 * TN + jj);
      P.o[i] = P.e[i] + 4 * TN;
    }
  }
}

// Part P of NP of the staging registers -> LDS stage st (chunks in the
// fragment-major layout; the scale words, from half H of the scale pair, go
// with the last part). Thread t holds chunk c = t % CPR of rows
// r0 + RSTEP i: group (r0 >> 5) + i RSTEP/32, slot r0 & 31 of chunk column c.
template <class G, int TM, int TN, int P, int NP, int H>
__device__ __forceinline__ void lstore_part(const Regs<G>& R, const SPos<G, TM, TN>& SP,
                                            uint8_t* st, int t) {
  const int r0 = t / G::CPR, c = t % G::CPR;
  uint8_t* pa = st + (r0 >> 5) * G::GP + c * G::CP + (r0 & 31) * 16;
  constexpr int STEP = (G::RSTEP / 32) * G::GP;
#pragma unroll
  for (int i = G::CA * P / NP; i < G::CA * (P + 1) / NP; ++i)
    *reinterpret_cast<u32x4*>(pa + i * STEP) = R.a[i];
#pragma unroll
  for (int i = G::CB * P / NP; i < G::CB * (P + 1) / NP; ++i)
    *reinterpret_cast<u32x4*>(pa + G::TA + i * STEP) = R.b[i];
  if (P == NP - 1) {
#pragma unroll
    for (int i = 0; i < G::SC; ++i) {
      uint32_t lo, hi = 0;
      if constexpr (G::SB == 8) {
        lo = H ? R.s[i].z : R.s[i].x;
        hi = H ? R.s[i].w : R.s[i].y;
      } else {
        lo = H ? R.s[i].y : R.s[i].x;
      }
      uint32_t ev, od;
      if (G::SB == 8) {
        ev = (lo & 0xffu) | ((lo >> 8) & 0xff00u) | ((hi & 0xffu) << 16) | ((hi << 8) & 0xff000000u);
        od = ((lo >> 8) & 0xffu) | ((lo >> 16) & 0xff00u) | (((hi >> 8) & 0xffu) << 16) |
             (hi & 0xff000000u);
      } else {
        ev = (lo & 0xffu) | ((lo >> 8) & 0xff00u);
        od = ((lo >> 8) & 0xffu) | ((lo >> 16) & 0xff00u);
      }
      *reinterpret_cast<uint32_t*>(st + SP.e[i]) = ev;
      *reinterpret_cast<uint32_t*>(st + SP.o[i]) = od;
    }
  }
}

template <int T>
__device__ __forceinline__ void lds_words(const uint8_t* p, int (&w)[T]) {
  if constexpr (T == 4) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(p);
    w[0] = (int)q.x; w[1] = (int)q.y; w[2] = (int)q.z; w[3] = (int)q.w;
  } else if constexpr (T == 2) {
    const u32x2 q = *reinterpret_cast<const u32x2*>(p);
    w[0] = (int)q.x; w[1] = (int)q.y;
  } else {
#pragma unroll
    for (int i = 0; i < T; ++i) w[i] = *reinterpret_cast<const int*>(p + 4 * i);
  }
}

template <int TM, int TN>
struct Frag {
  v8i a[TM], b[TN];
};

template <int TM, int TN>
struct Scl {
  int a[TM], b[TN];
};

// Per-lane LDS read addresses, relative to a stage.
struct RAddr {
  uint32_t fa, fb, sa, sb;
  int half;
};

// Fragment of k-step s for lane (l32, half): chunk 2 s + half of row
// row0 + 32 i + l32 = group row0/32 + i, slot l32.
template <class G, int TM, int TN>
__device__ __forceinline__ RAddr make_raddr(int wm, int wn, int lane) {
  RAddr r;
  const int l32 = lane & 31;
  r.half = lane >> 5;
  r.fa = (uint32_t)(wm * TM * G::GP + r.half * G::CP + l32 * 16);
  r.fb = (uint32_t)(G::TA + wn * TN * G::GP + r.half * G::CP + l32 * 16);
  r.sa = (uint32_t)(G::SOFF + 4 * ((wm * 32 + l32) * 2 + r.half) * TM);
  r.sb = (uint32_t)(G::SBOFF + 4 * ((wn * 32 + l32) * 2 + r.half) * TN);
  return r;
}

template <class G, int TM, int TN, int S>
__device__ __forceinline__ void read_frags(const uint8_t* st, const RAddr& ra, Frag<TM, TN>& F) {
  constexpr int co = 2 * S * G::CP;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(st + ra.fa + co + i * G::GP);
    F.a[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(st + ra.fb + co + j * G::GP);
    F.b[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
}

template <int TM, int TN>
__device__ __forceinline__ void read_scales(const uint8_t* st, const RAddr& ra, Scl<TM, TN>& S) {
  lds_words<TM>(st + ra.sa, S.a);
  lds_words<TN>(st + ra.sb, S.b);
}

// MFMAs of k-step S. Operand roles are swapped (B fragment first) so that
// accumulator register 4q + e of a lane holds four consecutive C columns.
template <int TM, int TN, int S>
__device__ __forceinline__ void mfma_step(const Frag<TM, TN>& F, const Scl<TM, TN>& sc,
                                          v16f (&acc)[TN][TM]) {
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.b[j], F.a[i], acc[j][i], 4, 4,
                                                                  S, sc.b[j], S, sc.a[i]);
}

// Scheduling groups for one k-step: NM MFMAs, each followed by its share of
// NR LDS reads (front-loaded, one per MFMA), NW LDS writes and NL global loads
// (spread evenly).
template <int R, int NM, int NR, int NW, int NL>
__device__ __forceinline__ void interleave() {
  if constexpr (R < NM) {
    constexpr int r = (R < NR) ? ((R == NM - 1) ? NR - R : 1) : 0;
    constexpr int w = NW * (R + 1) / NM - NW * R / NM;
    constexpr int l = NL * (R + 1) / NM - NL * R / NM;
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);
    if constexpr (w > 0) __builtin_amdgcn_sched_group_barrier(0x200, w, 0);
    if constexpr (l > 0) __builtin_amdgcn_sched_group_barrier(0x020, l, 0);
    interleave<R + 1, NM, NR, NW, NL>();
  }
}

template <class G, int TM, int TN, int NS, int C>
struct Pipe {
  static constexpr int NM = TM * TN, NR = TM + TN;
  static constexpr int NWR = G::CA + G::CB + 2 * G::SC;   // LDS writes per k-tile
  static constexpr int NLD = G::CA + G::CB + (C == 0 ? G::SC : 0);  // global loads
};

// One k-tile (stage C holds it, C = k % 2; F0 / SCc hold its k-step-0
// fragments and its scales). Leaves the next k-tile's k-step-0 fragments in
// F0 and its scales in SCn, the next k-tile written to stage C ^ 1, and tile
// k + 2 loading into the staging set just written; an even k also loads the
// scale pair of tiles k + 2 and k + 3 (the pair of k + 1 was used up here).
template <class G, int TM, int TN, int NS, int C>
__device__ __forceinline__ void ktile(uint8_t* lds, const RAddr& ra, Regs<G> (&R)[NS],
                                      const SPos<G, TM, TN>& SP, const Offs<G>& O,
                                      const Src<G>& S, Frag<TM, TN>& F0, Frag<TM, TN>& F1,
                                      const Scl<TM, TN>& SCc, Scl<TM, TN>& SCn,
                                      v16f (&acc)[TN][TM], int k, int nkt, int t) {
  static_assert(NS == 1, "one staging set");
  using PP = Pipe<G, TM, TN, NS, C>;
  uint8_t* cur = lds + C * G::STAGE;
  uint8_t* nxt = lds + (C ^ 1) * G::STAGE;
  constexpr int X = 0;
  // Prefetch indices clamp to the last k-tile (the last even one for the
  // scale pair); the redundant loads land in a stage nobody reads again.
  const int kl = min(k + 2, nkt - 1), kp = min(k + 2, nkt - 2);
  if constexpr (G::KSTEPS == 4) {
    read_frags<G, TM, TN, 1>(cur, ra, F1);
    lstore_part<G, TM, TN, 0, 2, C ^ 1>(R[X], SP, nxt, t);
    mfma_step<TM, TN, 0>(F0, SCc, acc);
    interleave<0, PP::NM, PP::NR, (G::CA + G::CB) / 2, 0>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags<G, TM, TN, 2>(cur, ra, F0);
    lstore_part<G, TM, TN, 1, 2, C ^ 1>(R[X], SP, nxt, t);
    gload_data<G>(R[X], O, S, kl);
    if constexpr (C == 0) gload_scales<G>(R[X], O, S, kp);
    mfma_step<TM, TN, 1>(F1, SCc, acc);
    interleave<0, PP::NM, PP::NR, PP::NWR - (G::CA + G::CB) / 2, PP::NLD>();
    __builtin_amdgcn_sched_barrier(0);
    read_frags<G, TM, TN, 3>(cur, ra, F1);
    mfma_step<TM, TN, 2>(F0, SCc, acc);
    interleave<0, PP::NM, PP::NR, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    read_scales<TM, TN>(nxt, ra, SCn);
    read_frags<G, TM, TN, 0>(nxt, ra, F0);
    mfma_step<TM, TN, 3>(F1, SCc, acc);
    interleave<0, PP::NM, PP::NR + 2, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
  } else {
    read_frags<G, TM, TN, 1>(cur, ra, F1);
    lstore_part<G, TM, TN, 0, 1, C ^ 1>(R[X], SP, nxt, t);
    gload_data<G>(R[X], O, S, kl);
    if constexpr (C == 0) gload_scales<G>(R[X], O, S, kp);
    mfma_step<TM, TN, 0>(F0, SCc, acc);
    interleave<0, PP::NM, PP::NR, PP::NWR, PP::NLD>();
    __builtin_amdgcn_sched_barrier(0);
    lds_barrier();
    read_scales<TM, TN>(nxt, ra, SCn);
    read_frags<G, TM, TN, 0>(nxt, ra, F0);
    mfma_step<TM, TN, 1>(F1, SCc, acc);
    interleave<0, PP::NM, PP::NR + 2, 0, 0>();
    __builtin_amdgcn_sched_barrier(0);
  }
}

template <int WM, int WN, int TM, int TN, int KB, int NS, int WPE, int OUT, bool VEC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WM * WN, 64 * WM * WN),
                          amdgpu_waves_per_eu(WPE)))
void gemm_pipe_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                      const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int64_t M,
                      int64_t N, int64_t K, void* __restrict__ C) {
  using G = Cfg<WM, WN, TM, TN, KB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * G::STAGE];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int64_t ntm = (M + G::BM - 1) / G::BM, ntn = (N + G::BN - 1) / G::BN;
  int64_t tm, tn;
  tile_of<GROUP_M>(blockIdx.x, gridDim.x, ntm, ntn, tm, tn);
  const int64_t m0 = tm * G::BM, n0 = tn * G::BN;
  const int64_t kbytes = K / 2, kblk = K / 32;
  const int nkt = (int)(kbytes / KB);
  const int arow0 = wm * TM * 32, brow0 = wn * TN * 32;

  v16f acc[TN][TM];
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;

  Offs<G> O;
  make_offsets<G>(O, m0, n0, M, N, kbytes, kblk, t);
  Src<G> S;
  make_src<G>(S, A, As, B, Bs, M, N, kbytes, kblk, wave);
  SPos<G, TM, TN> SP;
  make_spos<G, TM, TN>(SP, t);
  const RAddr ra = make_raddr<G, TM, TN>(wm, wn, lane);

  // Prologue: k-tile 0 into stage 0; the staging set then holds k-tile 1
  // (nkt is even, so there is one) and the scale pair of tiles 0 and 1.
  Regs<G> R[NS];
  gload_data<G>(R[0], O, S, 0);
  gload_scales<G>(R[0], O, S, 0);
  lstore_part<G, TM, TN, 0, 1, 0>(R[0], SP, lds, t);
  gload_data<G>(R[0], O, S, 1);
  lds_barrier();
  Frag<TM, TN> F0, F1;
  Scl<TM, TN> SCa, SCb;
  read_scales<TM, TN>(lds, ra, SCa);
  read_frags<G, TM, TN, 0>(lds, ra, F0);

  for (int k = 0; k < nkt; k += 2) {
    ktile<G, TM, TN, NS, 0>(lds, ra, R, SP, O, S, F0, F1, SCa, SCb, acc, k, nkt, t);
    ktile<G, TM, TN, NS, 1>(lds, ra, R, SP, O, S, F0, F1, SCb, SCa, acc, k + 1, nkt, t);
  }
  // Epilogue: acc[j][i] register 4q + e holds C[m][n] with
  // m = m0 + arow0 + 32 i + (lane & 31), n = n0 + brow0 + 32 j + 8 q + 4 (lane >> 5) + e.
  const int half = lane >> 5, l32 = lane & 31;
  const bool full = VEC && (m0 + G::BM <= M) && (n0 + G::BN <= N);
  if (full) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int64_t m = m0 + arow0 + i * 32 + l32;
      const int64_t nb = n0 + brow0 + 4 * half;
      if (OUT == 0) {
        float* p = static_cast<float*>(C) + m * N + nb;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q)
            *reinterpret_cast<float4*>(p + j * 32 + 8 * q) =
                make_float4(acc[j][i][4 * q], acc[j][i][4 * q + 1], acc[j][i][4 * q + 2],
                            acc[j][i][4 * q + 3]);
      } else {
        uint16_t* p = static_cast<uint16_t*>(C) + m * N + nb;
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const uint32_t lo = bf16_rne(acc[j][i][4 * q]) | (bf16_rne(acc[j][i][4 * q + 1]) << 16);
            const uint32_t hi = bf16_rne(acc[j][i][4 * q + 2]) | (bf16_rne(acc[j][i][4 * q + 3]) << 16);
            *reinterpret_cast<uint2*>(p + j * 32 + 8 * q) = make_uint2(lo, hi);
          }
      }
      __builtin_amdgcn_sched_barrier(0);  // keep each row group's reads next to its stores
    }
    return;
  }
  // Edge tiles (or unaligned C): element-wise, predicated. (Every index
  // into acc stays a compile-time constant so it remains in registers.)
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t m = m0 + arow0 + i * 32 + l32;
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t n = n0 + brow0 + j * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
        if (m < M && n < N) {
          if (OUT == 0)
            static_cast<float*>(C)[m * N + n] = acc[j][i][r];
          else
            static_cast<uint16_t*>(C)[m * N + n] = (uint16_t)bf16_rne(acc[j][i][r]);
        }
      }
  }
}

template <int WM, int WN, int TM, int TN, int KB, int NS, int WPE>
hipError_t launch(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                  int64_t M, int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  using G = Cfg<WM, WN, TM, TN, KB>;
  const int64_t tiles = ((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN);
  const bool vec = (N % 4 == 0) && ((uintptr_t)C % 16 == 0);
  const dim3 grid((unsigned)tiles), blk(G::NT);
  if (out_dtype == 0) {
    if (vec)
      hipLaunchKernelGGL((gemm_pipe_kernel<WM, WN, TM, TN, KB, NS, WPE, 0, true>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
    else
      hipLaunchKernelGGL((gemm_pipe_kernel<WM, WN, TM, TN, KB, NS, WPE, 0, false>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
  } else {
    if (vec)
      hipLaunchKernelGGL((gemm_pipe_kernel<WM, WN, TM, TN, KB, NS, WPE, 1, true>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
    else
      hipLaunchKernelGGL((gemm_pipe_kernel<WM, WN, TM, TN, KB, NS, WPE, 1, false>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
  }
  return hipGetLastError();
}

}  // namespace lt

// Persistent large-tile kernel fed by LDS DMA (K % 2048 == 0). One 512-thread
// work-group per CU walks output tiles t = blockIdx.x, + gridDim.x, ... (256 x
// 256 tiles, 8 waves of 128 x 64, 4 x 2 MFMA tiles each, 256-deep k-tiles):
//  * buffer_load_dwordx4 ... lds: the 64 lanes of one instruction write 1 KiB
//    of LDS at M0 + 16 lane, with no staging registers and no ds_write issued
//    by the waves that run the MFMAs. A k-tile is 32 such blocks per operand
//    (8 rows of 128 bytes each), 4 per wave, issued in two halves one k-step
//    apart;
//  * the operand stream does not stop at tile boundaries: the last k-tiles of
//    one tile prefetch the first k-tiles (and scale groups) of the next, so
//    no tile starts with an exposed load, and no work-group is relaunched;
//  * buffer resources start at the tile's first operand row and end at the
//    operand's end, so the per-lane offsets are the same for every tile and
//    rows past M or N read as zero (their products are never stored);
//  * tiles are row-major in LDS (128 bytes per row) with 16-byte chunk c of
//    row r at slot c ^ ((r >> 1) & 7). The permutation is applied to which
//    chunk a lane fetches, so a DMA block stays contiguous and 8 lanes fetch a
//    whole 128-byte row; the 16 lanes of a fragment read (rows r .. r + 15 of
//    one chunk) land on 16 distinct 4-bank groups;
//  * scale bytes arrive in groups of 4 k-tiles (32 bytes of every scale row,
//    two lanes per row), double-buffered. The load unit's cost grows with the
//    number of cache lines an instruction touches, not with its bytes, and a
//    scale row holds only 8 bytes per k-tile: fetched per k-tile, the scales
//    touched as many lines as the operand rows themselves (measured: the
//    operand stream of the gate+up product took 273 us with per-k-tile scale
//    rows against 163 us without them). A lane gathers the bytes of its
//    32-element half (even or odd blocks) with one v_perm per row;
//  * the stages and the scale buffers are separate LDS arrays, so the
//    compiler's wait tracking sees that a DMA into one does not feed reads of
//    another; a wave waits for its own DMAs (vmcnt) before the barrier that
//    publishes them;
//  * the MFMA takes A as its first operand, so register r of a lane holds one
//    C column (lane % 32) of row 8 (r / 4) + 4 (lane / 32) + r % 4: a 4-byte
//    store of one register writes two whole 128-byte row segments, straight
//    from the accumulators, non-temporal (C streams past L2 instead of
//    evicting the operand rows that the next tiles re-read). Measured on the
//    gate+up product, these stores cost the load unit about 11 cycles each,
//    cheaper per byte than 8-byte stores of paired rows or 16-byte stores of
//    quad-transposed registers.
namespace dm {

constexpr int BM = 256, BN = 256;
constexpr int KB = 128;                      // bytes per operand row per k-tile
constexpr int TILE = BM * KB;                // 32 KiB per operand
constexpr int STAGE = 2 * TILE;              // A rows then B rows of one k-tile
constexpr int SGB = (BM + BN) * 32;          // scale group: 4 k-tiles x 8 bytes per row

// Wave layout: WM x WN waves of TM x TN MFMA tiles (TM * 32 x TN * 32 each).
template <int WM_, int WN_, int TM_, int TN_>
struct L {
  static constexpr int WM = WM_, WN = WN_, TM = TM_, TN = TN_;
  static constexpr int NW = WM * WN, NT = 64 * NW;
  static constexpr int DA = 32 / NW;         // 1 KiB data DMA blocks per operand per wave
  static constexpr int DS = 8 / NW;          // 1 KiB scale-group blocks per operand per wave
  static constexpr int NDMA = 2 * DA;        // data DMA instructions per wave per k-tile
  static_assert(WM * TM * 32 == BM && WN * TN * 32 == BN, "256 x 256 tile");
  static_assert(NW * DA == 32 && NW * DS == 8, "DMA blocks divide over the waves");
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
using lt::rsrc_t;
using lt::u32x2;
using lt::u32x4;

// Buffer resources of one output tile: operand and scale rows from the
// tile's first row to the operand's last.
struct TileRes {
  rsrc_t a, b, sa, sb;
};

__device__ __forceinline__ rsrc_t rows_rsrc(const uint8_t* p, int64_t r0, int64_t rows,
                                            int64_t pitch) {
  return lt::make_rsrc(p + r0 * pitch, (rows - r0) * pitch);
}

__device__ __forceinline__ void tile_res(TileRes& T, const uint8_t* A, const uint8_t* As,
                                         const uint8_t* B, const uint8_t* Bs, int64_t m0,
                                         int64_t n0, int64_t M, int64_t N, int64_t kbytes,
                                         int64_t kblk) {
  T.a = rows_rsrc(A, m0, M, kbytes);
  T.b = rows_rsrc(B, n0, N, kbytes);
  T.sa = rows_rsrc(As, m0, M, kblk);
  T.sb = rows_rsrc(Bs, n0, N, kblk);
}

// Per-lane DMA offsets within a tile (the same for A and B rows): data block
// u holds rows 8 u .. 8 u + 7, lane l chunk (l % 8) ^ ((row >> 1) & 7) of row
// 8 u + l / 8; scale block v holds 32 rows, 16-byte unit l = 32 (r / 16) +
// 16 s + r % 16 being half s of row r's 32-byte group.
template <class G>
struct Lane {
  uint32_t d[G::DA], s[G::DS];
};

template <class G>
__device__ __forceinline__ void make_lane(Lane<G>& L, int64_t kbytes, int64_t kblk, int wave,
                                          int lane) {
#pragma unroll
  for (int u = 0; u < G::DA; ++u) {
    const int row = 8 * (G::DA * wave + u) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    L.d[u] = (uint32_t)(row * kbytes + c * 16);
  }
#pragma unroll
  for (int v = 0; v < G::DS; ++v) {
    const int srow = 32 * (G::DS * wave + v) + 16 * (lane >> 5) + (lane & 15);
    L.s[v] = (uint32_t)(srow * kblk + 16 * ((lane >> 4) & 1));
  }
}

// One LDS DMA instruction: lane l's 16 bytes at buffer offset voff + soff
// land at lds + 16 l.
__device__ __forceinline__ void dma_b128(rsrc_t r, uint8_t* lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, voff, soff, 0, 0);
}

// k-tile kt of the tile T into stage st. When live is false every lane reads
// out of range (nothing is fetched; that stage is never read again).
template <class G>
__device__ __forceinline__ void dma_data(uint8_t* st, const TileRes& T, const Lane<G>& L, int kt,
                                         bool live, rsrc_t none, int wave) {
  const rsrc_t ra = live ? T.a : none, rb = live ? T.b : none;
  const uint32_t ko = (uint32_t)kt * KB;
#pragma unroll
  for (int u = 0; u < G::DA; ++u) dma_b128(ra, st + (G::DA * wave + u) * 1024, L.d[u], ko);
#pragma unroll
  for (int u = 0; u < G::DA; ++u) dma_b128(rb, st + TILE + (G::DA * wave + u) * 1024, L.d[u], ko);
}

// Half PART (0 or 1) of dma_data: the first or last DA / 2 blocks of each
// operand. The pipeline issues a k-tile's two halves one k-step apart, which
// spreads the TA work of the DMAs over two MFMA groups instead of one (about
// 2 % faster on the Llama products than one burst; thirds or quarters were
// slower).
template <class G, int PART>
__device__ __forceinline__ void dma_data_half(uint8_t* st, const TileRes& T, const Lane<G>& L,
                                              int kt, bool live, rsrc_t none, int wave) {
  static_assert(G::DA % 2 == 0, "DA must split in two halves");
  const rsrc_t ra = live ? T.a : none, rb = live ? T.b : none;
  const uint32_t ko = (uint32_t)kt * KB;
  constexpr int H = G::DA / 2;
#pragma unroll
  for (int u = PART * H; u < (PART + 1) * H; ++u)
    dma_b128(ra, st + (G::DA * wave + u) * 1024, L.d[u], ko);
#pragma unroll
  for (int u = PART * H; u < (PART + 1) * H; ++u)
    dma_b128(rb, st + TILE + (G::DA * wave + u) * 1024, L.d[u], ko);
}

// Scale group g (k-tiles 4 g .. 4 g + 3) of the tile T into sg (A rows, then B rows).
template <class G>
__device__ __forceinline__ void dma_scales(uint8_t* sg, const TileRes& T, const Lane<G>& L, int g,
                                           bool live, rsrc_t none, int wave) {
  const rsrc_t rsa = live ? T.sa : none, rsb = live ? T.sb : none;
  const uint32_t so = (uint32_t)g * 32;
#pragma unroll
  for (int v = 0; v < G::DS; ++v) dma_b128(rsa, sg + 1024 * (G::DS * wave + v), L.s[v], so);
#pragma unroll
  for (int v = 0; v < G::DS; ++v) dma_b128(rsb, sg + 8192 + 1024 * (G::DS * wave + v), L.s[v], so);
}

// Per-lane LDS read offsets: fragment of k-step s (chunk 2 s + half of row
// l32 of each 32-row group) within a stage, and the lane's scale units
// within a scale group.
struct RA {
  uint32_t fa[4], fb[4], sa, sb, psel;
};

template <class G>
__device__ __forceinline__ RA make_ra(int wm, int wn, int lane) {
  RA r;
  const int l32 = lane & 31, h = lane >> 5, key = (l32 >> 1) & 7;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    const uint32_t off = (uint32_t)(l32 * KB + (((2 * s + h) ^ key) * 16));
    r.fa[s] = (uint32_t)(wm * G::TM * 32 * KB) + off;
    r.fb[s] = (uint32_t)(TILE + wn * G::TN * 32 * KB) + off;
  }
  const uint32_t u = (uint32_t)(16 * (32 * (l32 >> 4) + (l32 & 15)));
  r.sa = (uint32_t)(wm * G::TM * 1024) + u;
  r.sb = (uint32_t)(8192 + wn * G::TN * 1024) + u;
  r.psel = h ? 0x07050301u : 0x06040200u;  // bytes 1,3,5,7 or 0,2,4,6 of the row's 8
  return r;
}

template <class G, int S>
__device__ __forceinline__ void read_frags(const uint8_t* st, const RA& ra,
                                           lt::Frag<G::TM, G::TN>& F) {
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(st + ra.fa[S] + i * 32 * KB);
    F.a[i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(st + ra.fb[S] + j * 32 * KB);
    F.b[j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
  }
}

// Scales of k-tile P (0..3) of a scale group: the row's 8 bytes are half
// P / 2, word P % 2; the lane keeps the bytes of its 32-element half.
template <class G, int P>
__device__ __forceinline__ void read_scales(const uint8_t* sg, const RA& ra,
                                            lt::Scl<G::TM, G::TN>& S) {
  constexpr int so = 256 * (P >> 1);
#pragma unroll
  for (int i = 0; i < G::TM; ++i) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(sg + ra.sa + so + i * 1024);
    S.a[i] = (P & 1) ? (int)__builtin_amdgcn_perm(q.w, q.z, ra.psel)
                     : (int)__builtin_amdgcn_perm(q.y, q.x, ra.psel);
  }
#pragma unroll
  for (int j = 0; j < G::TN; ++j) {
    const u32x4 q = *reinterpret_cast<const u32x4*>(sg + ra.sb + so + j * 1024);
    S.b[j] = (P & 1) ? (int)__builtin_amdgcn_perm(q.w, q.z, ra.psel)
                     : (int)__builtin_amdgcn_perm(q.y, q.x, ra.psel);
  }
}

// MFMAs of k-step S, A fragment first: accumulator register r of a lane is
// one C column of one row.
template <int TM, int TN, int S>
__device__ __forceinline__ void mfma_ab(const lt::Frag<TM, TN>& F, const lt::Scl<TM, TN>& sc,
                                          v16f (&acc)[TN][TM]) {
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i)
      acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(F.a[i], F.b[j], acc[j][i], 4, 4,
                                                                  S, sc.a[i], S, sc.b[j]);
}

// s_waitcnt with only vmcnt constrained (expcnt and lgkmcnt at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void tile_at(int64_t vt, int64_t ntiles, int64_t ntm, int64_t ntn,
                                        int64_t& m0, int64_t& n0) {
  int64_t tm, tn;
  lt::tile_of<lt::GROUP_M>(vt, ntiles, ntm, ntn, tm, tn);
  m0 = tm * BM;
  n0 = tn * BN;
}

// One k-tile k (C = k % 8) of the current tile, in stage C % 2; F0 / SCc
// hold its k-step-0 fragments and its scales. The barrier before the last
// k-step publishes k-tile k + 1 (every wave waited for its own DMAs of it)
// and retires stage C % 2, which then receives the first half of k-tile
// k + 2 -- of the next tile (Tn) when k + 2 runs past this tile -- while the
// last MFMAs of k-tile k run; its second half follows with k-step 0 of k-tile
// k + 1. When C % 4 == 3 the scale group buffer of k-tiles k - 3 .. k is
// retired the same way and receives group (k + 5) / 4.
template <class G, int C>
__device__ __forceinline__ void ktile(uint8_t* st0, uint8_t* st1, uint8_t* sg0, uint8_t* sg1,
                                      const RA& ra, const TileRes& Tc, const TileRes& Tn,
                                      bool has_next, rsrc_t none, const Lane<G>& L,
                                      lt::Frag<G::TM, G::TN>& F0, lt::Frag<G::TM, G::TN>& F1,
                                      const lt::Scl<G::TM, G::TN>& SCc, lt::Scl<G::TM, G::TN>& SCn,
                                      v16f (&acc)[G::TN][G::TM], int k, int nkt, int wave) {
  constexpr int TM = G::TM, TN = G::TN, NM = TM * TN, NR = TM + TN;
  constexpr bool SG = (C & 3) == 3;
  uint8_t* cur = (C & 1) ? st1 : st0;
  uint8_t* nxt = (C & 1) ? st0 : st1;
  uint8_t* sgn = (((C + 1) >> 2) & 1) ? sg1 : sg0;  // scale group of k-tile k + 1
  uint8_t* sgw = (((C + 5) >> 2) & 1) ? sg1 : sg0;  // group (k + 5) / 4, written when SG
  read_frags<G, 1>(cur, ra, F1);
  mfma_ab<TM, TN, 0>(F0, SCc, acc);
  {  // second half of k-tile k + 1
    const int kk = k + 1;
    const bool nx = kk >= nkt;
    dma_data_half<G, 1>(nxt, nx ? Tn : Tc, L, nx ? kk - nkt : kk, nx ? has_next : true, none, wave);
  }
  lt::interleave<0, NM, NR, 0, G::NDMA / 2>();
  __builtin_amdgcn_sched_barrier(0);
  read_frags<G, 2>(cur, ra, F0);
  mfma_ab<TM, TN, 1>(F1, SCc, acc);
  lt::interleave<0, NM, NR, 0, 0>();
  __builtin_amdgcn_sched_barrier(0);
  read_frags<G, 3>(cur, ra, F1);
  mfma_ab<TM, TN, 2>(F0, SCc, acc);
  lt::interleave<0, NM, NR, 0, 0>();
  __builtin_amdgcn_sched_barrier(0);
  wait_vm<0>();
  lt::lds_barrier();
  read_scales<G, (C + 1) & 3>(sgn, ra, SCn);
  read_frags<G, 0>(nxt, ra, F0);
  {
    const int kk = k + 2;
    const bool nx = kk >= nkt;
    dma_data_half<G, 0>(cur, nx ? Tn : Tc, L, nx ? kk - nkt : kk, nx ? has_next : true, none, wave);
  }
  if constexpr (SG) {
    const int g = (k + 5) >> 2, ng = nkt >> 2;
    const bool nx = g >= ng;
    dma_scales<G>(sgw, nx ? Tn : Tc, L, nx ? g - ng : g, nx ? has_next : true, none, wave);
  }
  mfma_ab<TM, TN, 3>(F1, SCc, acc);
  lt::interleave<0, NM, 2 * NR, 0, G::NDMA / 2 + (SG ? 2 * G::DS : 0)>();
  // the scale byte gathers (v_perm) wait for their reads: keep them last
  __builtin_amdgcn_sched_group_barrier(0x002, NR, 0);
  __builtin_amdgcn_sched_barrier(0);
}

template <class G, int OUT>
__global__ __attribute__((amdgpu_flat_work_group_size(G::NT, G::NT),
                          amdgpu_waves_per_eu(G::NW == 8 ? 2 : 1)))
void gemm_dma_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int64_t M,
                     int64_t N, int64_t K, void* __restrict__ C) {
  constexpr int TM = G::TM, TN = G::TN;
  constexpr int EB = OUT == 0 ? 4 : 2;  // bytes per C element
  __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
  __shared__ __attribute__((aligned(16))) uint8_t sg0[SGB];
  __shared__ __attribute__((aligned(16))) uint8_t sg1[SGB];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / G::WN, wn = wave % G::WN;
  const int half = lane >> 5, l32 = lane & 31;
  const int64_t ntm = (M + BM - 1) / BM, ntn = (N + BN - 1) / BN, ntiles = ntm * ntn;
  const int64_t P = gridDim.x;
  const int64_t kbytes = K / 2, kblk = K / 32;
  const int nkt = (int)(kbytes / KB);
  const int arow0 = wm * TM * 32, brow0 = wn * TN * 32;
  const rsrc_t none = lt::make_rsrc(A, 0);
  const RA ra = make_ra<G>(wm, wn, lane);
  Lane<G> L;
  make_lane<G>(L, kbytes, kblk, wave, lane);
  // Per-lane part of a full tile's store offsets (the tile's first element
  // is the store resource's base).
  const uint32_t vst = (uint32_t)(((int64_t)(arow0 + 4 * half) * N + brow0 + l32) * EB);

  int64_t vt = blockIdx.x;
  int64_t m0, n0, m0n = 0, n0n = 0;
  tile_at(vt, ntiles, ntm, ntn, m0, n0);
  TileRes Tc, Tn;
  tile_res(Tc, A, As, B, Bs, m0, n0, M, N, kbytes, kblk);
  bool has_next = vt + P < ntiles;
  if (has_next) tile_at(vt + P, ntiles, ntm, ntn, m0n, n0n);
  tile_res(Tn, A, As, B, Bs, m0n, n0n, M, N, kbytes, kblk);

  // Prologue: scale group 0, k-tile 0, the first half of k-tile 1 (k-tile 0
  // issues the second), scale group 1 (nkt % 8 == 0). Loads complete in
  // issue order, so this wave's DMAs of group 0 and k-tile 0 have landed once
  // at most NDMA / 2 + 2 DS are outstanding. No LDS reads precede this
  // barrier, so it needs no release fence (which would also wait for the
  // later DMAs); the acquire fence keeps the reads below it.
  dma_scales<G>(sg0, Tc, L, 0, true, none, wave);
  dma_data<G>(st0, Tc, L, 0, true, none, wave);
  dma_data_half<G, 0>(st1, Tc, L, 1, true, none, wave);
  dma_scales<G>(sg1, Tc, L, 1, true, none, wave);
  wait_vm<G::NDMA / 2 + 2 * G::DS>();
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  lt::Frag<TM, TN> F0, F1;
  lt::Scl<TM, TN> SCa, SCb;
  read_scales<G, 0>(sg0, ra, SCa);
  read_frags<G, 0>(st0, ra, F0);

  v16f acc[TN][TM];
  for (;;) {
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[j][i][r] = 0.f;
    for (int k = 0; k < nkt; k += 8) {
      ktile<G, 0>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCa, SCb, acc, k, nkt, wave);
      ktile<G, 1>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCb, SCa, acc, k + 1, nkt, wave);
      ktile<G, 2>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCa, SCb, acc, k + 2, nkt, wave);
      ktile<G, 3>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCb, SCa, acc, k + 3, nkt, wave);
      ktile<G, 4>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCa, SCb, acc, k + 4, nkt, wave);
      ktile<G, 5>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCb, SCa, acc, k + 5, nkt, wave);
      ktile<G, 6>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCa, SCb, acc, k + 6, nkt, wave);
      ktile<G, 7>(st0, st1, sg0, sg1, ra, Tc, Tn, has_next, none, L, F0, F1, SCb, SCa, acc, k + 7, nkt, wave);
    }
    // Store the tile: acc[j][i] register r holds
    // C[m0 + arow0 + 32 i + 8 (r / 4) + 4 half + r % 4][n0 + brow0 + 32 j + l32].
    if (m0 + BM <= M && n0 + BN <= N) {
      const rsrc_t rc = lt::make_rsrc(static_cast<uint8_t*>(C) + (m0 * N + n0) * EB,
                                      min((M - m0) * N * EB, (int64_t)0xffffffff));
      if constexpr (OUT == 0) {
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t so = (uint32_t)((32 * i + 8 * (r >> 2) + (r & 3)) * N * EB);
#pragma unroll
            for (int j = 0; j < TN; ++j)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[j][i][r]), rc,
                                                    vst + 128 * j, so, 2);
          }
      } else {
        // bf16: v_permlane32_swap of the two 32-column blocks gives each
        // register 64 consecutive columns of one row (lane = column); two
        // such rows R, R + 1 then trade one value between neighbouring
        // lanes, so an even lane holds row R at columns l, l + 1 and an odd
        // lane row R + 1 at columns l - 1, l: one 4-byte store per two rows.
        static_assert(TN == 2, "two 32-column blocks per wave");
        const int odd = lane & 1;
        const uint32_t vb = (uint32_t)(((int64_t)(arow0 + odd) * N + brow0 + lane - odd) * 2);
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
          for (int q = 0; q < 4; ++q)
#pragma unroll
            for (int e = 0; e < 4; e += 2) {
              const auto s0 = __builtin_amdgcn_permlane32_swap(
                  __float_as_uint(acc[0][i][4 * q + e]), __float_as_uint(acc[1][i][4 * q + e]), false,
                  false);
              const auto s1 = __builtin_amdgcn_permlane32_swap(
                  __float_as_uint(acc[0][i][4 * q + e + 1]),
                  __float_as_uint(acc[1][i][4 * q + e + 1]), false, false);
#pragma unroll
              for (int t = 0; t < 2; ++t) {  // rows 8 q + e + 4 t and the next one
                const uint32_t a = s0[t], b = s1[t];
                const uint32_t rcv = (uint32_t)__builtin_amdgcn_mov_dpp((int)(odd ? a : b), 0xb1, 0xf,
                                                                        0xf, false);
                const float lo = __uint_as_float(odd ? rcv : a), hi = __uint_as_float(odd ? b : rcv);
                const uint32_t so = (uint32_t)((32 * i + 8 * q + e + 4 * t) * N * 2);
                const bf16x2 pk = {(__bf16)lo, (__bf16)hi};  // v_cvt_pk_bf16_f32 (RNE)
                __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, pk), rc, vb, so,
                                                      2);
              }
            }
      }
    } else {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int64_t m = m0 + arow0 + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int64_t n = n0 + brow0 + 32 * j + l32;
            if (m < M && n < N) {
              if (OUT == 0)
                static_cast<float*>(C)[m * N + n] = acc[j][i][r];
              else
                static_cast<uint16_t*>(C)[m * N + n] = (uint16_t)bf16_rne(acc[j][i][r]);
            }
          }
        }
    }
    if (!has_next) break;
    vt += P;
    m0 = m0n;
    n0 = n0n;
    Tc = Tn;
    has_next = vt + P < ntiles;
    if (has_next) {
      tile_at(vt + P, ntiles, ntm, ntn, m0n, n0n);
      tile_res(Tn, A, As, B, Bs, m0n, n0n, M, N, kbytes, kblk);
    }
  }
  // The last k-tiles' DMAs (out of range) still write LDS: let them land.
  wait_vm<0>();
}

// Compute units of the current device (the persistent grid), queried once
// per device; calls from several host threads are safe.
int cu_count() {
  constexpr int kMaxDevices = 64;
  static std::atomic<int> cache[kMaxDevices];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n == 0) {
    int c = 0;
    n = (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess &&
         c > 0)
            ? c
            : 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

template <class G>
hipError_t launch(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                  int64_t M, int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const int64_t ncu = cu_count();
  const dim3 grid((unsigned)(tiles < ncu ? tiles : ncu)), blk(G::NT);
  if (out_dtype == 0)
    hipLaunchKernelGGL((gemm_dma_kernel<G, 0>), grid, blk, 0, stream, a, as, b, bs, M, N, K, C);
  else
    hipLaunchKernelGGL((gemm_dma_kernel<G, 1>), grid, blk, 0, stream, a, as, b, bs, M, N, K, C);
  return hipGetLastError();
}

}  // namespace dm

}  // namespace

hipError_t launch_gemm_mbs(const void* Aq, const void* As, const void* Am, const void* Bq,
                           const void* Bs, const void* Bm, int64_t M, int64_t N, int64_t K,
                           void* C, int out_dtype, hipStream_t stream) {
  const auto* a = static_cast<const uint8_t*>(Aq);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* am = static_cast<const uint8_t*>(Am);
  const auto* b = static_cast<const uint8_t*>(Bq);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  const auto* bm = static_cast<const uint8_t*>(Bm);
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const bool svec = (K % 256 == 0) && ((uintptr_t)As % 8 == 0) && ((uintptr_t)Bs % 8 == 0);
  const dim3 grid((unsigned)tiles), blk(256);
  if (out_dtype == 0) {
    if (svec)
      hipLaunchKernelGGL((gemm_mbs_kernel<0, true>), grid, blk, 0, stream, a, as, am, b, bs, bm, M,
                         N, K, C);
    else
      hipLaunchKernelGGL((gemm_mbs_kernel<0, false>), grid, blk, 0, stream, a, as, am, b, bs, bm,
                         M, N, K, C);
  } else {
    if (svec)
      hipLaunchKernelGGL((gemm_mbs_kernel<1, true>), grid, blk, 0, stream, a, as, am, b, bs, bm, M,
                         N, K, C);
    else
      hipLaunchKernelGGL((gemm_mbs_kernel<1, false>), grid, blk, 0, stream, a, as, am, b, bs, bm,
                         M, N, K, C);
  }
  return hipGetLastError();
}

hipError_t launch_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs, int64_t M,
                       int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  const auto* a = static_cast<const uint8_t*>(Aq);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(Bq);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  const dim3 blk(256);
  // Large-tile paths (32-bit per-lane operand offsets): 256 x 256 tiles, 8
  // waves of 128 x 64. The persistent LDS-DMA kernel runs its main loop over
  // 8 k-tiles of 256 (two scale groups), so it needs K % 2048 == 0 and
  // 16-byte aligned scale arrays (scale groups are 16-byte loads), and its
  // 32-bit store offsets span 256 rows of C (N < 2^22); the register-staged kernel
  // runs k-tiles in pairs, 256-deep when K % 512 == 0 (16-byte scale pairs)
  // and 128-deep when only K % 256 == 0 (8-byte pairs).
  const bool off32 = (M * (K / 2) < (int64_t(1) << 32)) && (N * (K / 2) < (int64_t(1) << 32));
  const bool sc_al = ((uintptr_t)As % 8 == 0) && ((uintptr_t)Bs % 8 == 0);
  const bool sc_al16 = ((uintptr_t)As % 16 == 0) && ((uintptr_t)Bs % 16 == 0);
  if (off32 && sc_al16 && K % 2048 == 0 && N < (int64_t(1) << 22))
    return dm::launch<dm::L<2, 4, 4, 2>>(a, as, b, bs, M, N, K, C, out_dtype, stream);
  if (off32 && sc_al16 && K % 512 == 0)
    return lt::launch<2, 4, 4, 2, 128, 1, 2>(a, as, b, bs, M, N, K, C, out_dtype, stream);
  if (off32 && sc_al && K % 256 == 0)
    return lt::launch<2, 4, 4, 2, 64, 1, 2>(a, as, b, bs, M, N, K, C, out_dtype, stream);
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const bool svec = (K % 256 == 0) && ((uintptr_t)As % 8 == 0) && ((uintptr_t)Bs % 8 == 0);
  const dim3 grid((unsigned)tiles);
  if (out_dtype == 0) {
    if (svec)
      hipLaunchKernelGGL((gemm_kernel<0, true>), grid, blk, 0, stream, a, as, b, bs, M, N, K, C);
    else
      hipLaunchKernelGGL((gemm_kernel<0, false>), grid, blk, 0, stream, a, as, b, bs, M, N, K, C);
  } else {
    if (svec)
      hipLaunchKernelGGL((gemm_kernel<1, true>), grid, blk, 0, stream, a, as, b, bs, M, N, K, C);
    else
      hipLaunchKernelGGL((gemm_kernel<1, false>), grid, blk, 0, stream, a, as, b, bs, M, N, K, C);
  }
  return hipGetLastError();
}

}  // namespace mx
