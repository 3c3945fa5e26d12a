// Device-side pieces shared by the bf16 MFMA GEMM kernels: vector types, bf16
// packing, the block -> tile mapping and
// the epilogue (staged through LDS so that stores are row-contiguous).
#pragma once

#include <type_traits>

#include "common.h"
#include "activation.h"

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

// Compile-time loop: f(std::integral_constant<int, I>) for I = I0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for<I + 1, N>(f);
  }
}

// One v_cvt_pk_bf16_f32 (round to nearest even) per pair.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Workgroups are handed to the X XCDs round-robin; renumber so that each XCD
// walks a contiguous range of tiles (neighbouring tiles share its L2).
__device__ __forceinline__ int xcd_remap(int bid, int total, int X) {
  const int per = total / X, rem = total % X;
  const int x = bid % X, slot = bid / X;
  return x * per + (x < rem ? x : rem) + slot;
}

// Which problem of the group and which (tm, tn) tile this block computes.
struct TileCoord {
  int g, tm, tn;
};
__device__ __forceinline__ TileCoord locate_tile(const GemmBatch& batch) {
  const int bid = xcd_remap((int)blockIdx.x, batch.total_tiles, batch.nxcd);
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

// The fp32 epilogue on four consecutive outputs C[m][n .. n+3] (off =
// m*ldc+n): one 16-byte store when vec_c allows it and the row has room,
// else element by element.  fp32 results are final outputs, not read again
// by the kernels of the same call: non-temporal stores keep them from
// displacing the operand panels that the running tiles share in L2.
__device__ __forceinline__ void store_f32x4(const GemmProb& P, floatx4 v, int64_t off, int n, int N, int vec_c) {
  float* c = static_cast<float*>(P.C) + off;
  if (vec_c && n + 3 < N) {
    __builtin_nontemporal_store(v, reinterpret_cast<floatx4*>(c));
  } else {
    for (int r = 0; r < 4; ++r)
      if (n + r < N) __builtin_nontemporal_store(v[r], c + r);
  }
}

// The bf16-output epilogues on eight consecutive outputs C[m][n .. n+7]
// (a, b: columns n .. n+3 and n+4 .. n+7).  vec_c bit 1 allows one 16-byte
// store per output (and, for EPI_MUL, `pre` holds the eight sigma'(P)
// values); bit 0 allows 8-byte halves; otherwise element by element.
template <int EPI, int ACT = ACT_GELU>
__device__ __forceinline__ void epilogue_store8(const GemmProb& P, floatx4 a, floatx4 b, int64_t off, int n, int N,
                                                int vec_c, u32x4 pre = u32x4{0u, 0u, 0u, 0u}) {
  float v[8] = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  const bool full16 = (vec_c & 2) && (n + 7 < N);
  uint16_t* c = static_cast<uint16_t*>(P.C) + off;
  float g[8];  // EPI_ACT: the activation (second output)
  if constexpr (EPI == EPI_ACT) {
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      float s, ds;
      act_fast<ACT>(v[r], s, ds);
      g[r] = s;
      v[r] = ds;
    }
  } else if constexpr (EPI == EPI_MUL) {
    if (full16) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        v[2 * q] *= bf_lo(pre[q]);
        v[2 * q + 1] *= bf_hi(pre[q]);
      }
    } else {
      const uint16_t* p = static_cast<const uint16_t*>(P.aux_in) + off;
#pragma unroll
      for (int r = 0; r < 8; ++r)
        if (n + r < N) v[r] *= __uint_as_float((uint32_t)p[r] << 16);
    }
  }
  auto put = [&](uint16_t* dst, const float (&x)[8]) {
    if (full16) {
      *reinterpret_cast<u32x4*>(dst) =
          u32x4{pack_bf16(x[0], x[1]), pack_bf16(x[2], x[3]), pack_bf16(x[4], x[5]), pack_bf16(x[6], x[7])};
      return;
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if ((vec_c & 1) && n + 4 * h + 3 < N) {
        *reinterpret_cast<u32x2*>(dst + 4 * h) =
            u32x2{pack_bf16(x[4 * h], x[4 * h + 1]), pack_bf16(x[4 * h + 2], x[4 * h + 3])};
      } else {
#pragma unroll
        for (int r = 4 * h; r < 4 * h + 4; ++r)
          if (n + r < N) dst[r] = __builtin_bit_cast(uint16_t, (__bf16)x[r]);
      }
    }
  };
  put(c, v);
  if constexpr (EPI == EPI_ACT) put(static_cast<uint16_t*>(P.aux_out) + off, g);
}

// Ordering point between one wave's LDS writes and its own lanes' reads (and
// the next pass's writes): a wave's LDS instructions execute in program
// order, so only the compiler must be kept from moving accesses across it.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// Epilogue through LDS (`stage` must be free and hold 32 * (TN_ + 4) floats per
// wave; each wave writes and reads back only its own region, so the passes
// need no workgroup barrier, only the caller's one before the first pass).  Pass q moves MFMA blocks mi = 2q, 2q+1 of every wave (a 32 x TN_
// region per wave) into LDS, then each wave reads its region back
// row-contiguously and applies the epilogue with coalesced stores.  For
// EPI_MUL the tile's sigma'(P) values are loaded before the first exchange.  The wave (wm, wn) owns rows wm*TM_ .. and
// columns wn*TN_ .. of the block tile, and acc[ni][mi] holds
// C[m0 + wm*TM_ + mi*16 + lane%16][n0 + wn*TN_ + ni*16 + 4*(lane/16) + r].
template <int EPI, int TM_, int TN_, int ACT = ACT_GELU>
__device__ __forceinline__ void epilogue_via_lds(float* stage, const floatx4 (&acc)[TN_ / 16][TM_ / 16],
                                                 const GemmProb& P, int m0, int n0, int wid, int wm, int wn,
                                                 int lane, int vec_c) {
  // fp32 outputs: four columns (one 16-byte store) per lane; bf16 outputs:
  // eight columns per lane, so each output is again one 16-byte store.
  constexpr int CPL = EPI == EPI_F32 ? 4 : 8;
  constexpr int LD = TN_ + 4;
  constexpr int LANES_PER_ROW = TN_ / CPL;
  constexpr int ROWS_PER_IT = 64 / LANES_PER_ROW;
  constexpr int ITS = 32 / ROWS_PER_IT;
  float* ep = stage + wid * (32 * LD);
  const int64_t ldc = P.ldc;
  const int M = P.M, N = P.N;
  const int col = CPL * (lane % LANES_PER_ROW);
  const int n = n0 + wn * TN_ + col;
  // For EPI_MUL the whole tile's sigma'(P) values (TM_/32 passes x ITS
  // loads per lane) are requested before the first pass, so their latency
  // overlaps the LDS exchanges instead of stalling each pass.
  constexpr int NPRE = EPI == EPI_MUL ? (TM_ / 32) * ITS : 1;
  u32x4 pre[NPRE];
  if constexpr (EPI == EPI_MUL) {
    const bool vec16 = (vec_c & 2) && n + 7 < N;
#pragma unroll
    for (int i = 0; i < NPRE; ++i) {
      const int m = m0 + wm * TM_ + 32 * (i / ITS) + lane / LANES_PER_ROW + ROWS_PER_IT * (i % ITS);
      pre[i] = (vec16 && m < M)
                   ? *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(P.aux_in) + (int64_t)m * ldc + n)
                   : u32x4{0u, 0u, 0u, 0u};
    }
  }
  // Passes are unrolled at compile time (static_for), so acc and pre are
  // only ever indexed by constants and stay in registers.
  static_for<0, TM_ / 32>([&](auto q_) {
    constexpr int q = decltype(q_)::value;
    const int mbase = m0 + wm * TM_ + 32 * q + lane / LANES_PER_ROW;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ni = 0; ni < TN_ / 16; ++ni)
        *reinterpret_cast<floatx4*>(ep + (h * 16 + (lane & 15)) * LD + ni * 16 + 4 * (lane >> 4)) =
            acc[ni][2 * q + h];
    wave_sync();
    // All of the pass's LDS reads first (one wait), then the math and stores.
    floatx4 vals[ITS][CPL / 4];
#pragma unroll
    for (int it = 0; it < ITS; ++it)
#pragma unroll
      for (int c4 = 0; c4 < CPL / 4; ++c4)
        vals[it][c4] =
            *reinterpret_cast<const floatx4*>(ep + (ROWS_PER_IT * it + lane / LANES_PER_ROW) * LD + col + 4 * c4);
#pragma unroll
    for (int it = 0; it < ITS; ++it) {
      const int m = mbase + ROWS_PER_IT * it;
      if (m < M && n < N) {
        if constexpr (EPI == EPI_F32)
          store_f32x4(P, vals[it][0], (int64_t)m * ldc + n, n, N, vec_c);
        else if constexpr (EPI == EPI_MUL)
          epilogue_store8<EPI, ACT>(P, vals[it][0], vals[it][1], (int64_t)m * ldc + n, n, N, vec_c, pre[q * ITS + it]);
        else
          epilogue_store8<EPI, ACT>(P, vals[it][0], vals[it][1], (int64_t)m * ldc + n, n, N, vec_c);
      }
    }
    wave_sync();
  });
}

}  // namespace gemm
}  // namespace tpr
