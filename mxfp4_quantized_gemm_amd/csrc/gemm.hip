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
// Two kernel families. The large-tile kernels (namespace big, below) serve
// K % 256 == 0. The general kernel here serves any K % 32 == 0 and any M, N:
// a 256-thread work-group (4 waves, 2 x 2) computes a 128 x 128
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


// ===================================================================== big
// Large-tile kernels for K % 256 == 0 (every Llama shape), templated on the
// wave layout: WM x WN waves per work-group, each computing TM x TN MFMA
// 32x32x64 tiles, so the work-group tile is (32 WM TM) x (32 WN TN); on the
// k-tile depth, KB bytes of nibbles per operand row (64 or 128, i.e. 128 or
// 256 elements; 128 bytes reads whole cache lines); and on NS, the number of
// k-tiles staged in registers ahead of the MFMAs (1 or 2). Global loads of
// later k-tiles are issued into registers before the MFMAs of tile t and
// written to the free LDS buffer after them; two LDS buffers, one LDS-only
// barrier per k-tile, so the prefetch stays in flight across it.
//
// Operand roles are swapped in the MFMA (B as the instruction's first
// operand), so a lane's accumulator registers 4q..4q+3 hold four
// consecutive columns of one C row: the epilogue writes 16-byte vectors.
//
// LDS tile rows are KB bytes of 16-byte chunks; chunk c of row r is stored
// at c ^ g(r), which spreads the rows read together by one ds_read_b128
// over distinct banks for both 8- and 16-lane service groups:
// g(r) = ((r >> 1) ^ (r >> 3)) & 3 for 4 chunks, (r ^ (r >> 3)) & 7 for 8.
namespace big {

constexpr int GROUP_M = 4;

// Staging registers use the native vector type: HIP's uint4 is a class
// whose copies lower to memcpy, which keeps the struct in scratch memory.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Swizzle of the 16-byte chunks of an LDS row. It depends on row bits 0-4
// only: every row a lane touches is congruent to the lane's row modulo 32,
// so the swizzle is a per-lane constant and tile offsets become immediates.
template <int KB>
__device__ __forceinline__ int swz(int r) {
  return KB == 64 ? (((r >> 1) ^ (r >> 3)) & 3) : ((r & 7) ^ ((r >> 3) & 3));
}

// Work-group barrier that orders LDS only: global loads in flight (the
// prefetch of later k-tiles) stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

template <int WM, int WN, int TM, int TN, int KB>
struct Cfg {
  static constexpr int NT = 64 * WM * WN;
  static constexpr int BM = 32 * WM * TM, BN = 32 * WN * TN;
  static constexpr int CPR = KB / 16;                    // 16-byte chunks per row
  static constexpr int SB = KB / 16;                     // scale bytes per row per k-tile
  static constexpr int KSTEPS = KB / 32;                 // MFMA k-steps (64 elements each)
  static constexpr int TA = BM * KB, TB = BN * KB;
  static constexpr int SOFF = TA + TB;                   // scales: A rows then B rows
  static constexpr int STAGE = TA + TB + (BM + BN) * SB;
  static constexpr int RSTEP = NT / CPR;                 // rows between a thread's chunks
  static constexpr int CA = BM / RSTEP, CB = BN / RSTEP; // chunks per thread
  static constexpr int SC = (BM + BN + NT - 1) / NT;     // scale rows per thread
  static_assert(BM % RSTEP == 0 && BN % RSTEP == 0 && RSTEP % 32 == 0, "bad tiling");
};

// Per-thread global offsets (32-bit, relative to the operand base; the k-tile
// offset is added to the uniform base): chunk c = t % CPR of rows
// t / CPR + RSTEP i, clamped to the last row (results of clamped rows are
// never stored), and the scale rows d = t + NT i (A rows, then B rows; a d
// past the tile reloads a valid B row that lstore drops).
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

// Staging registers use the native vector type: HIP's uint4 is a class
// whose copies lower to memcpy, which keeps the struct in scratch memory.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

template <class G>
struct Regs {
  u32x4 a[G::CA], b[G::CB];
  u32x2 s[G::SC];  // SB bytes used (4 or 8)
};

template <class G>
__device__ __forceinline__ void gload(Regs<G>& R, const Offs<G>& O, const Src<G>& S, int kt) {
  constexpr int KB = G::CPR * 16;
  const int ko = kt * KB, so = kt * G::SB;
#pragma unroll
  for (int i = 0; i < G::CA; ++i) R.a[i] = __builtin_amdgcn_raw_buffer_load_b128(S.a, O.a[i], ko, 0);
#pragma unroll
  for (int i = 0; i < G::CB; ++i) R.b[i] = __builtin_amdgcn_raw_buffer_load_b128(S.b, O.b[i], ko, 0);
#pragma unroll
  for (int i = 0; i < G::SC; ++i) {
    if (G::SB == 8) {
      R.s[i] = __builtin_amdgcn_raw_buffer_load_b64(S.s[i], O.s[i], so, 0);
    } else {
      const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(S.s[i], O.s[i], so, 0);
      R.s[i] = u32x2{w, w};
    }
  }
}

template <class G>
__device__ __forceinline__ void lstore(const Regs<G>& R, uint8_t* st, int t) {
  constexpr int KB = G::CPR * 16;
  const int r0 = t / G::CPR, c = t % G::CPR;
  uint8_t* pa = st + r0 * KB + ((c ^ swz<KB>(r0 & 31)) << 4);
#pragma unroll
  for (int i = 0; i < G::CA; ++i) *reinterpret_cast<u32x4*>(pa + i * G::RSTEP * KB) = R.a[i];
#pragma unroll
  for (int i = 0; i < G::CB; ++i) *reinterpret_cast<u32x4*>(pa + G::TA + i * G::RSTEP * KB) = R.b[i];
#pragma unroll
  for (int i = 0; i < G::SC; ++i) {
    const int d = t + G::NT * i;
    // When the block's threads cover the scale rows exactly the test is
    // static: a run-time one lets the compiler sink the scale load of gload
    // into the guarded block, right before its use, exposing its latency.
    if (G::SC * G::NT == G::BM + G::BN || d < G::BM + G::BN) {
      if (G::SB == 8)
        *reinterpret_cast<u32x2*>(st + G::SOFF + d * 8) = R.s[i];
      else
        *reinterpret_cast<uint32_t*>(st + G::SOFF + d * 4) = R.s[i].x;
    }
  }
}

// One k-tile: KSTEPS k-steps of TM x TN MFMAs. The fragments of k-step s+1
// are read from LDS while the MFMAs of k-step s run (two fragment sets);
// scheduling barriers keep the compiler from hoisting every k-step's reads
// at once. Lane l reads rows (row0 + 32 i + l % 32), chunk (2s + l / 32)
// ^ swz(l % 32): one base address per k-step, tile offsets immediate.
// Scale word of a row for k-step pair p: the row's scale bytes shifted by
// 8 * (l / 32), so byte 2s' of the word is this lane's block for k-step
// 2p + s'; op_sel 0 / 2 picks it.
template <class G, int TM, int TN>
__device__ __forceinline__ void compute(const uint8_t* st, v16f (&acc)[TN][TM], int arow0,
                                        int brow0, int lane) {
  constexpr int KB = G::CPR * 16;
  const int half = lane >> 5, l32 = lane & 31;
  const int g = swz<KB>(l32);
  const uint8_t* pa = st + (arow0 + l32) * KB;
  const uint8_t* pb = st + G::TA + (brow0 + l32) * KB;
  int sa[TM][2], sb[TN][2];
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const uint8_t* ps = st + G::SOFF + (arow0 + l32 + 32 * i) * G::SB;
    if (G::SB == 8) {
      const uint64_t v = *reinterpret_cast<const uint64_t*>(ps) >> (8 * half);
      sa[i][0] = (int)(uint32_t)v;
      sa[i][1] = (int)(uint32_t)(v >> 32);
    } else {
      sa[i][0] = (int)(*reinterpret_cast<const uint32_t*>(ps) >> (8 * half));
      sa[i][1] = 0;
    }
  }
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const uint8_t* ps = st + G::SOFF + (G::BM + brow0 + l32 + 32 * j) * G::SB;
    if (G::SB == 8) {
      const uint64_t v = *reinterpret_cast<const uint64_t*>(ps) >> (8 * half);
      sb[j][0] = (int)(uint32_t)v;
      sb[j][1] = (int)(uint32_t)(v >> 32);
    } else {
      sb[j][0] = (int)(*reinterpret_cast<const uint32_t*>(ps) >> (8 * half));
      sb[j][1] = 0;
    }
  }
  v8i af[2][TM], bf[2][TN];
#pragma unroll
  for (int s = 0; s <= G::KSTEPS; ++s) {
    if (s < G::KSTEPS) {
      const int co = ((2 * s + half) ^ g) << 4;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(pa + co + i * 32 * KB);
        af[s & 1][i] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const u32x4 q = *reinterpret_cast<const u32x4*>(pb + co + j * 32 * KB);
        bf[s & 1][j] = v8i{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      }
    }
    if (s > 0) {
      const int u = s - 1, x = u & 1;
#pragma unroll
      for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          if ((u & 1) == 0)
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[x][j], af[x][i], acc[j][i], 4, 4, 0, sb[j][u >> 1], 0, sa[i][u >> 1]);
          else
            acc[j][i] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                bf[x][j], af[x][i], acc[j][i], 4, 4, 2, sb[j][u >> 1], 2, sa[i][u >> 1]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Ordering point: every MFMA issued so far must have been issued before any
// later memory operation. MFMAs touch no memory, so without this the
// compiler may sink a k-tile's MFMAs below the next LDS stores and barrier,
// which leaves the global-load latency of the prefetch uncovered. The empty
// asm reads the accumulators (in AGPRs) and clobbers memory.
template <int TM, int TN>
__device__ __forceinline__ void order_after_mfma(v16f (&acc)[TN][TM]) {
#pragma unroll
  for (int j = 0; j < TN; ++j)
#pragma unroll
    for (int i = 0; i < TM; ++i) asm volatile("" ::"a"(acc[j][i]) : "memory");
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

template <int WM, int WN, int TM, int TN, int KB, int NS, int WPE, int OUT, bool VEC,
          int GM = GROUP_M>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * WM * WN, 64 * WM * WN),
                          amdgpu_waves_per_eu(WPE)))
void gemm_big_kernel(const uint8_t* __restrict__ A, const uint8_t* __restrict__ As,
                     const uint8_t* __restrict__ B, const uint8_t* __restrict__ Bs, int64_t M,
                     int64_t N, int64_t K, void* __restrict__ C) {
  using G = Cfg<WM, WN, TM, TN, KB>;
  __shared__ __attribute__((aligned(16))) uint8_t lds[2 * G::STAGE];
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int64_t ntm = (M + G::BM - 1) / G::BM, ntn = (N + G::BN - 1) / G::BN;
  int64_t tm, tn;
  tile_of<GM>(blockIdx.x, gridDim.x, ntm, ntn, tm, tn);
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

  // Buffer 0 holds even k-tiles, buffer 1 odd ones. Prefetch indices are
  // clamped to the last tile so the loop body is branch-free; the clamped
  // (redundant) loads at the end land in a buffer nobody reads again.
  Offs<G> O;
  make_offsets<G>(O, m0, n0, M, N, kbytes, kblk, t);
  Src<G> S;
  make_src<G>(S, A, As, B, Bs, M, N, kbytes, kblk, wave);
  if (NS == 2) {
    Regs<G> R0, R1;
    gload<G>(R0, O, S, 0);
    gload<G>(R1, O, S, min(1, nkt - 1));
    lstore<G>(R0, lds, t);
    lds_barrier();
    for (int kt = 0; kt < nkt; kt += 2) {
      gload<G>(R0, O, S, min(kt + 2, nkt - 1));
      compute<G, TM, TN>(lds, acc, arow0, brow0, lane);
      order_after_mfma<TM, TN>(acc);
      lstore<G>(R1, lds + G::STAGE, t);
      lds_barrier();
      gload<G>(R1, O, S, min(kt + 3, nkt - 1));
      compute<G, TM, TN>(lds + G::STAGE, acc, arow0, brow0, lane);
      order_after_mfma<TM, TN>(acc);
      lstore<G>(R0, lds, t);
      lds_barrier();
    }
  } else {
    Regs<G> R;
    gload<G>(R, O, S, 0);
    lstore<G>(R, lds, t);
    lds_barrier();
    for (int kt = 0; kt < nkt; kt += 2) {
      gload<G>(R, O, S, min(kt + 1, nkt - 1));
      compute<G, TM, TN>(lds, acc, arow0, brow0, lane);
      order_after_mfma<TM, TN>(acc);
      lstore<G>(R, lds + G::STAGE, t);
      lds_barrier();
      gload<G>(R, O, S, min(kt + 2, nkt - 1));
      compute<G, TM, TN>(lds + G::STAGE, acc, arow0, brow0, lane);
      order_after_mfma<TM, TN>(acc);
      lstore<G>(R, lds, t);
      lds_barrier();
    }
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

// K must be a multiple of 2 * KB * 2 (an even number of k-tiles).
template <int WM, int WN, int TM, int TN, int KB, int NS, int WPE>
hipError_t launch(const uint8_t* a, const uint8_t* as, const uint8_t* b, const uint8_t* bs,
                  int64_t M, int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  using G = Cfg<WM, WN, TM, TN, KB>;
  const int64_t tiles = ((M + G::BM - 1) / G::BM) * ((N + G::BN - 1) / G::BN);
  const bool vec = (N % 4 == 0) && ((uintptr_t)C % 16 == 0);
  const dim3 grid((unsigned)tiles), blk(G::NT);
  if (out_dtype == 0) {
    if (vec)
      hipLaunchKernelGGL((gemm_big_kernel<WM, WN, TM, TN, KB, NS, WPE, 0, true>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
    else
      hipLaunchKernelGGL((gemm_big_kernel<WM, WN, TM, TN, KB, NS, WPE, 0, false>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
  } else {
    if (vec)
      hipLaunchKernelGGL((gemm_big_kernel<WM, WN, TM, TN, KB, NS, WPE, 1, true>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
    else
      hipLaunchKernelGGL((gemm_big_kernel<WM, WN, TM, TN, KB, NS, WPE, 1, false>), grid, blk, 0,
                         stream, a, as, b, bs, M, N, K, C);
  }
  return hipGetLastError();
}

}  // namespace big

}  // namespace

hipError_t launch_gemm(const void* Aq, const void* As, const void* Bq, const void* Bs, int64_t M,
                       int64_t N, int64_t K, void* C, int out_dtype, hipStream_t stream) {
  const auto* a = static_cast<const uint8_t*>(Aq);
  const auto* as = static_cast<const uint8_t*>(As);
  const auto* b = static_cast<const uint8_t*>(Bq);
  const auto* bs = static_cast<const uint8_t*>(Bs);
  const dim3 blk(256);
  // Large-tile paths (the main loop runs k-tiles in pairs, so K must hold
  // an even number of them; 32-bit per-lane operand offsets):
  //  K % 512 == 0: 256 x 256 tile, 8 waves of 128 x 64, 256-deep k-tiles
  //                (whole 128-byte operand rows per k-tile);
  //  K % 256 == 0: 256 x 256 tile, 4 waves of 128 x 128, 128-deep k-tiles.
  const bool off32 = (M * (K / 2) < (int64_t(1) << 32)) && (N * (K / 2) < (int64_t(1) << 32));
  const bool sc_al = ((uintptr_t)As % 8 == 0) && ((uintptr_t)Bs % 8 == 0);
  if (off32 && sc_al && K % 512 == 0)
    return big::launch<2, 4, 4, 2, 128, 1, 2>(a, as, b, bs, M, N, K, C, out_dtype, stream);
  if (off32 && sc_al && K % 256 == 0)
    return big::launch<2, 2, 4, 4, 64, 2, 1>(a, as, b, bs, M, N, K, C, out_dtype, stream);
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
