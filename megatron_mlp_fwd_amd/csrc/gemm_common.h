// Device-side pieces shared by the bf16 MFMA GEMM kernels: vector types, bf16
// packing, the exact-erf GELU and its derivative, the block -> tile mapping and
// the epilogue (staged through LDS so that stores are row-contiguous).
#pragma once

#include "common.h"

namespace tpr {
namespace gemm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Block tile 256 x 256 computed by 4 waves in a 2 x 2 grid; each wave owns a
// 128 x 128 sub-tile = 8 x 8 MFMA 16x16 blocks.
constexpr int BM = 256, BN = 256;
constexpr int NT = 256;
constexpr int WTM = 128, WTN = 128;
constexpr int FM = WTM / 16, FN = WTN / 16;
constexpr int GROUP_M = 8;  // tile rows per raster group (L2 reuse of the B panel)

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  const uint32_t x = __builtin_bit_cast(uint16_t, (__bf16)a);
  const uint32_t y = __builtin_bit_cast(uint16_t, (__bf16)b);
  return x | (y << 16);
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Exact-erf GELU and its derivative (fp32).  Phi(x) = erfc(-x/sqrt2)/2.
__device__ __forceinline__ float gelu_f(float x) { return 0.5f * x * erfcf(-0.70710678118654752f * x); }
__device__ __forceinline__ float gelu_prime_f(float x) {
  return 0.5f * erfcf(-0.70710678118654752f * x) + 0.39894228040143268f * x * expf(-0.5f * x * x);
}

// Workgroups are handed to the 8 XCDs round-robin; renumber so that each XCD
// walks a contiguous range of tiles (neighbouring tiles share its L2).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * per + (x < rem ? x : rem) + slot;
}

// Which problem of the group and which (tm, tn) tile this block computes.
struct TileCoord {
  int g, tm, tn;
};
__device__ __forceinline__ TileCoord locate_tile(const GemmBatch& batch) {
  const int bid = xcd_remap((int)blockIdx.x, batch.total_tiles);
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < batch.count && bid >= batch.p[i].tile_start) g = i;
  const GemmProb& P = batch.p[g];
  int local = bid - P.tile_start;
  const int per_group = GROUP_M * P.tiles_n;
  const int first_m = (local / per_group) * GROUP_M;
  const int gsize = min(P.tiles_m - first_m, GROUP_M);
  local %= per_group;
  return TileCoord{g, first_m + local % gsize, local / gsize};
}

// Apply the epilogue to four consecutive outputs C[m][n .. n+3] (off = m*ldc+n).
template <int EPI>
__device__ __forceinline__ void epilogue_store(const GemmProb& P, floatx4 v, int64_t off, int n, int N, int vec_c) {
  const bool full = vec_c && (n + 3 < N);
  if constexpr (EPI == EPI_F32) {
    float* c = static_cast<float*>(P.C) + off;
    if (full) {
      *reinterpret_cast<floatx4*>(c) = v;
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < N) c[r] = v[r];
    }
  } else if constexpr (EPI == EPI_GELU) {
    uint16_t* c = static_cast<uint16_t*>(P.C) + off;
    uint16_t* h = static_cast<uint16_t*>(P.aux_out) + off;
    floatx4 gv;
    for (int r = 0; r < 4; ++r) gv[r] = gelu_f(v[r]);
    if (full) {
      *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
      *reinterpret_cast<u32x2*>(h) = u32x2{pack_bf16(gv[0], gv[1]), pack_bf16(gv[2], gv[3])};
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < N) {
          c[r] = __builtin_bit_cast(uint16_t, (__bf16)v[r]);
          h[r] = __builtin_bit_cast(uint16_t, (__bf16)gv[r]);
        }
    }
  } else {  // EPI_DGELU: C = acc * gelu'(pre), pre read from aux_in (may alias C)
    const uint16_t* p = static_cast<const uint16_t*>(P.aux_in) + off;
    uint16_t* c = static_cast<uint16_t*>(P.C) + off;
    if (full) {
      const u32x2 pw = *reinterpret_cast<const u32x2*>(p);
      v[0] *= gelu_prime_f(bf_lo(pw[0]));
      v[1] *= gelu_prime_f(bf_hi(pw[0]));
      v[2] *= gelu_prime_f(bf_lo(pw[1]));
      v[3] *= gelu_prime_f(bf_hi(pw[1]));
      *reinterpret_cast<u32x2*>(c) = u32x2{pack_bf16(v[0], v[1]), pack_bf16(v[2], v[3])};
    } else {
      for (int r = 0; r < 4; ++r)
        if (n + r < N) {
          const float pre = __uint_as_float((uint32_t)p[r] << 16);
          c[r] = __builtin_bit_cast(uint16_t, (__bf16)(v[r] * gelu_prime_f(pre)));
        }
    }
  }
}

// Epilogue through LDS (`stage` must be free and hold 32 * (TN_ + 4) floats per
// wave).  Pass q moves MFMA blocks mi = 2q, 2q+1 of every wave (a 32 x TN_
// region per wave) into LDS, then each wave reads its region back
// row-contiguously and applies the epilogue with coalesced stores.  The wave
// (wm, wn) owns rows wm*TM_ .. and columns wn*TN_ .. of the block tile, and
// acc[ni][mi] holds C[m0 + wm*TM_ + mi*16 + lane%16][n0 + wn*TN_ + ni*16 + 4*(lane/16) + r].
template <int EPI, int TM_, int TN_>
__device__ __forceinline__ void epilogue_via_lds(float* stage, const floatx4 (&acc)[TN_ / 16][TM_ / 16],
                                                 const GemmProb& P, int m0, int n0, int wid, int wm, int wn,
                                                 int lane, int vec_c) {
  constexpr int LD = TN_ + 4;
  constexpr int LANES_PER_ROW = TN_ / 4;
  constexpr int ROWS_PER_IT = 64 / LANES_PER_ROW;
  float* ep = stage + wid * (32 * LD);
  const int64_t ldc = P.ldc;
  const int M = P.M, N = P.N;
#pragma unroll
  for (int q = 0; q < TM_ / 32; ++q) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ni = 0; ni < TN_ / 16; ++ni)
        *reinterpret_cast<floatx4*>(ep + (h * 16 + (lane & 15)) * LD + ni * 16 + 4 * (lane >> 4)) =
            acc[ni][2 * q + h];
    __syncthreads();
    const int col = 4 * (lane % LANES_PER_ROW);
    const int n = n0 + wn * TN_ + col;
    for (int it = 0; it < 32 / ROWS_PER_IT; ++it) {
      const int row = ROWS_PER_IT * it + lane / LANES_PER_ROW;
      const int m = m0 + wm * TM_ + 32 * q + row;
      if (m < M && n < N) {
        floatx4 v = *reinterpret_cast<const floatx4*>(ep + row * LD + col);
        epilogue_store<EPI>(P, v, (int64_t)m * ldc + n, n, N, vec_c);
      }
    }
    __syncthreads();
  }
}

}  // namespace gemm
}  // namespace tpr
