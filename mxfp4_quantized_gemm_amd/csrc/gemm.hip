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
// Tiling: a 256-thread work-group (4 waves, 2 x 2) computes a 128 x 128
// tile of C; each wave a 64 x 64 sub-tile (2 x 2 MFMA tiles, 64 fp32
// accumulators per lane). The k-loop steps 256 elements (128 bytes of
// nibbles per row, 8 scale bytes per row). Tiles of A and B are staged in
// LDS with a 16-byte-chunk XOR swizzle (chunk c of row r stored at c ^ (r & 7))
// so that the 32 rows read by one ds_read_b128 hit distinct banks. LDS is
// double-buffered: the global loads of tile k+1 are issued before the MFMAs
// of tile k and written to the other buffer after them, with one barrier
// per k-tile.
#include <hip/hip_runtime.h>
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

}  // namespace

hipError_t launch_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs, int64_t M,
                       int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
  const bool svec = (K % 256 == 0) && ((uintptr_t)As % 8 == 0) && ((uintptr_t)Bs % 8 == 0);
  const auto* a = static_cast<const uint8_t*>(Aq);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(Bq);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  const dim3 grid((unsigned)tiles), blk(256);
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
