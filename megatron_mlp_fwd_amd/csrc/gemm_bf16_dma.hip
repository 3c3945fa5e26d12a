// bf16 GEMM for gfx950 with direct-to-LDS operand loads (the fast path of
// every aligned bf16 product of the sharded GEMM page's 解题路线 and the TP
// lesson's MLP; the register-staged kernel in gemm_bf16.hip covers the rest).
//
// Block tile 256 x 256, 4 waves (one per SIMD) in a 2 x 2 grid, each owning a
// 128 x 128 sub-tile = 8 x 8 blocks of v_mfma_f32_16x16x32_bf16 whose fp32
// accumulators (256 per lane) stay pinned in AGPRs.  K advances in 64-deep
// slabs through two 64 KB LDS stages.  Operands go global -> LDS with
// buffer_load_dwordx4 ... lds (16 bytes per lane, no registers; the buffer's
// range check zero-fills rows past the edge), so one wave instruction moves
// 1 KB: 8 rows x 128 B of a k-major operand (whole cache lines) or 2 k-rows x
// 512 B of an m/n-major one.  Fragments come out of LDS with ds_read_b128 for
// a k-major operand and with the gfx950 transpose read ds_read_b64_tr_b16 for
// an m/n-major one, so NN, NT and TN all run without register transposes.
//
// Per slab k (stage k % 2): the first half (k 0..31) runs 64 MFMAs while the
// second half's fragments are read; each wave then waits for its own DMA of
// slab k+1, and one barrier makes slab k+1 visible and frees stage k % 2; the
// second half runs 64 MFMAs with slab k+2's 16 DMA issues spread one per 4
// MFMAs (a burst would stall the wave on a full address FIFO) and slab k+1's
// first-half fragment reads one per 2 MFMAs.
//
// LDS layouts (16-byte chunks, XOR-swizzled so every fragment read is free of
// bank conflicts under both a 16-lane/64-bank and an 8-lane/32-bank phase):
//   k-major tile:  256 rows x 128 B; chunk c of row r sits at 8 r + (c ^ kswz(r)).
//   m/n-major tile: 64 k-rows x 512 B; chunk c of k-row k sits at 32 k + (c ^ mswz(k)).
#include <type_traits>

#include "gemm_common.h"

namespace tpr {
namespace {

using namespace gemm;

constexpr int BK = 64;                       // k per LDS stage
constexpr int TILE_BYTES = 256 * BK * 2;     // one operand tile per stage: 32 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // 64 KB; two stages
constexpr int NTH = 256;                     // 4 waves, 2 x 2
constexpr int WT = 128;                      // wave tile 128 x 128
constexpr int FR = WT / 16;                  // fragments per operand per 32-deep half slab
constexpr int NDMA = TILE_BYTES / 1024 / 4;  // DMA instructions per wave per operand per slab
constexpr uint32_t OOB = 0x80000000u;        // voffset beyond every num_records: the load returns zeros
// Tile rows per raster group.  An XCD's 32 resident tiles then span 4 tile
// rows x 8 tile columns; on the 70B-rank MLP launches this ran 1.5-2 % faster
// than 8 rows (3 and 6 rows tied with 4; 1, 16 and 32 rows were slower).
constexpr int RASTER_M = 4;

static_assert(2 * STAGE_BYTES >= 4 * 32 * (WT + 4) * 4, "epilogue staging must fit in the stage ring");

typedef __attribute__((address_space(3))) uint8_t lds_u8;

__device__ __forceinline__ int kswz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int mswz(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }

// s_waitcnt with only a vmcnt limit (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Fragments are read with inline assembly (the builtin forms make the
// compiler wait for every outstanding LDS DMA first, which would drain the
// stage ring each slab).  A k-major fragment is one ds_read_b128; an m/n-major
// one is two ds_read_b64_tr_b16 (k = 8G..8G+3 and 8G+4..8G+7 of the lane's
// column), kept as two halves until the lgkmcnt wait that covers them, so no
// register copy can read a half before its data has landed.
struct FragK {
  u32x4 v;
};
struct FragT {
  u32x2 lo, hi;
};
__device__ __forceinline__ bf16x8 as_operand(const FragK& f) { return __builtin_bit_cast(bf16x8, f.v); }
__device__ __forceinline__ bf16x8 as_operand(const FragT& f) {
  return __builtin_bit_cast(bf16x8, u32x4{f.lo[0], f.lo[1], f.hi[0], f.hi[1]});
}
template <bool KMAJ>
using Frag = typename std::conditional<KMAJ, FragK, FragT>::type;

template <int OFF>
__device__ __forceinline__ void read_frag(FragK& f, uint32_t addr) {
  asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(f.v) : "v"(addr), "i"(OFF));
}
template <int OFF>
__device__ __forceinline__ void read_frag(FragT& f, uint32_t addr) {
  asm volatile("ds_read_b64_tr_b16 %0, %2 offset:%3\n\tds_read_b64_tr_b16 %1, %2 offset:%4"
               : "=&v"(f.lo), "=&v"(f.hi)
               : "v"(addr), "i"(OFF), "i"(OFF + 2048));
}

// Tie every fragment register to a point after an lgkmcnt wait.
__device__ __forceinline__ void tie(FragK (&f)[FR]) {
  asm volatile("" : "+v"(f[0].v), "+v"(f[1].v), "+v"(f[2].v), "+v"(f[3].v), "+v"(f[4].v), "+v"(f[5].v),
               "+v"(f[6].v), "+v"(f[7].v));
}
__device__ __forceinline__ void tie(FragT (&f)[FR]) {
  asm volatile("" : "+v"(f[0].lo), "+v"(f[0].hi), "+v"(f[1].lo), "+v"(f[1].hi), "+v"(f[2].lo), "+v"(f[2].hi),
               "+v"(f[3].lo), "+v"(f[3].hi), "+v"(f[4].lo), "+v"(f[4].hi), "+v"(f[5].lo), "+v"(f[5].hi),
               "+v"(f[6].lo), "+v"(f[6].hi), "+v"(f[7].lo), "+v"(f[7].hi));
}
template <bool AK, bool BKM>
__device__ __forceinline__ void frag_wait(Frag<AK> (&a)[FR], Frag<BKM> (&b)[FR]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  tie(a);
  tie(b);
}

// The accumulators live in AGPRs and are updated in place: inline assembly
// pins each one to its registers (left to itself the compiler shuffles the
// 256 accumulator registers between loop iterations).  The instruction reads
// only its own AGPR accumulator, which nothing else writes, and VGPR operands
// that LDS reads wrote behind an lgkmcnt wait; reading the accumulators after
// the last MFMA is guarded by mfma_drain().
__device__ __forceinline__ void mfma(floatx4& c, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(c) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_drain() {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
}

struct Dma {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[NDMA];  // this lane's byte offsets for the wave's loads of one slab (at k = 0)
  uint32_t kstep;       // bytes between consecutive k slabs
};

// Operand element (r, k): k-major at X[r * ld + k], m/n-major at X[k * ld + r].
// Wave w fills 1 KB blocks NDMA w .. NDMA w + NDMA-1 of the 32 KB tile.
template <bool KMAJ>
__device__ __forceinline__ void dma_setup(Dma& d, const void* X, int64_t ld, int R, int K, int r0, int wid,
                                          int lane) {
  const int64_t bytes = KMAJ ? ((int64_t)(R - 1) * ld + K) * 2 : ((int64_t)(K - 1) * ld + R) * 2;
  d.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(X), (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    const int b = wid * NDMA + j;
    if constexpr (KMAJ) {  // block b: rows 8b .. 8b+7, 8 chunks each
      const int r = 8 * b + (lane >> 3), c = (lane & 7) ^ kswz(r);
      const int gr = r0 + r;
      d.voff[j] = gr < R ? (uint32_t)(((int64_t)gr * ld + 8 * c) * 2) : OOB;
    } else {  // block b: k-rows 2b, 2b+1, 32 chunks each
      const int kl = 2 * b + (lane >> 5), c = (lane & 31) ^ mswz(kl);
      const int gr = r0 + 8 * c;
      d.voff[j] = gr < R ? (uint32_t)(((int64_t)kl * ld + gr) * 2) : OOB;
    }
  }
  d.kstep = KMAJ ? BK * 2 : (uint32_t)(BK * ld * 2);
}

__device__ __forceinline__ void dma_one(const Dma& d, lds_u8* dst, int j, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsrc, (__attribute__((address_space(3))) void*)dst, 16, d.voff[j], soff,
                                           0, 0);
}
__device__ __forceinline__ void dma_all(const Dma& d, lds_u8* tile, int wid, int kt) {
  lds_u8* base = tile + wid * NDMA * 1024;
  const uint32_t soff = (uint32_t)kt * d.kstep;
#pragma unroll
  for (int j = 0; j < NDMA; ++j) dma_one(d, base + j * 1024, j, soff);
}
// The last slab when K % 64 == 32: lanes whose k lies at or past K load
// nothing (zeros), and the slab offset goes into the range-checked vector
// offset, so no load can reach past the operand.
template <bool KMAJ>
__device__ __forceinline__ void dma_tail(const Dma& d, lds_u8* tile, int wid, int kt, int K, int lane) {
  lds_u8* base = tile + wid * NDMA * 1024;
  const uint32_t koff = (uint32_t)kt * d.kstep;
#pragma unroll
  for (int j = 0; j < NDMA; ++j) {
    // k of this lane's chunk: k-major chunk index (lane & 7) ^ kswz(r) with
    // r & 7 = lane >> 3 and (r >> 3) & 1 = j & 1; m/n-major k-row 2b + lane / 32.
    const int kl = KMAJ ? 8 * ((lane & 7) ^ (lane >> 3) ^ (j & 1)) : 2 * (wid * NDMA + j) + (lane >> 5);
    const uint32_t v = (kt * BK + kl < K && d.voff[j] != OOB) ? d.voff[j] + koff : OOB;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsrc, (__attribute__((address_space(3))) void*)(base + j * 1024), 16,
                                             v, 0, 0, 0);
  }
}
template <bool AK, bool BKM>
__device__ __forceinline__ void dma_slab(const Dma& da, const Dma& db, lds_u8* stage, int wid, int kt, bool tail,
                                         int K, int lane) {
  if (tail) {
    dma_tail<AK>(da, stage, wid, kt, K, lane);
    dma_tail<BKM>(db, stage + TILE_BYTES, wid, kt, K, lane);
  } else {
    dma_all(da, stage, wid, kt);
    dma_all(db, stage + TILE_BYTES, wid, kt);
  }
}

// Per-lane LDS byte addresses of the fragments (rows row0 + 16 f ..) of one
// operand; ds offsets are 16-bit immediates, so each stage has its own bases.
// k-major: addr(s, f, h) = base[s][h] + 2048 f;  m/n-major: base[s][f] + 16384 h.
template <bool KMAJ>
struct FragAddr {
  uint32_t base[2][KMAJ ? 2 : FR];
};
template <bool KMAJ>
__device__ __forceinline__ void frag_addr(FragAddr<KMAJ>& fa, uint32_t tile0, int row0, int lane) {
  if constexpr (KMAJ) {
    const int rr = lane & 15, x = lane >> 4;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        fa.base[s][h] = tile0 + s * STAGE_BYTES + (row0 + rr) * 128 + (((4 * h + x) ^ kswz(rr)) * 16);
  } else {
    const int G = lane >> 4, q = lane & 15;
    const int kl = 8 * G + (q >> 2);
#pragma unroll
    for (int f = 0; f < FR; ++f) {
      const int c = row0 / 8 + 2 * f + ((q & 3) >> 1);
      fa.base[0][f] = tile0 + kl * 512 + ((c ^ mswz(kl)) * 16) + (q & 1) * 8;
      fa.base[1][f] = fa.base[0][f] + STAGE_BYTES;
    }
  }
}
// Read fragment F of half H from stage S.
template <bool KMAJ, int S, int H, int F>
__device__ __forceinline__ void read_one(Frag<KMAJ>& fr, const FragAddr<KMAJ>& fa) {
  if constexpr (KMAJ) read_frag<F * 2048>(fr, fa.base[S][H]);
  else read_frag<H * 16384>(fr, fa.base[S][F]);
}

// One 256 x 256 output tile of problem P.
template <bool AK, bool BKM, int EPI, bool ACT_DISPATCH = false>
__device__ __forceinline__ void gemm_tile(const GemmProb& P, int tm, int tn, uint8_t* smem_raw, int vec_c) {
  lds_u8* smem = (lds_u8*)smem_raw;
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 1, wn = wid & 1;
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tm * BM, n0 = tn * BN;

  Dma da, db;
  dma_setup<AK>(da, P.A, AK ? P.sa_m : P.sa_k, M, K, m0, wid, lane);
  dma_setup<BKM>(db, P.B, BKM ? P.sb_n : P.sb_k, N, K, n0, wid, lane);
  FragAddr<AK> aa;
  FragAddr<BKM> ba;
  frag_addr<AK>(aa, lds0, wm * WT, lane);
  frag_addr<BKM>(ba, lds0 + TILE_BYTES, wn * WT, lane);

  floatx4 acc[FR][FR];
#pragma unroll
  for (int ni = 0; ni < FR; ++ni)
#pragma unroll
    for (int mi = 0; mi < FR; ++mi) acc[ni][mi] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;  // 64-deep slabs; the last one is half used when K % 64 == 32
  const bool half_tail = (K % BK) != 0;
  Frag<AK> a0[FR], a1[FR];
  Frag<BKM> b0[FR], b1[FR];
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;

  // All fragments of half H of stage S into (a, b), in program order.
  auto read_half = [&](auto S_, auto H_, Frag<AK>(&a)[FR], Frag<BKM>(&b)[FR]) {
    constexpr int S = decltype(S_)::value, H = decltype(H_)::value;
    static_for<0, FR>([&](auto f_) {
      constexpr int f = decltype(f_)::value;
      read_one<AK, S, H, f>(a[f], aa);
    });
    static_for<0, FR>([&](auto f_) {
      constexpr int f = decltype(f_)::value;
      read_one<BKM, S, H, f>(b[f], ba);
    });
  };
  // The 64 MFMAs of one half slab (acc[ni][mi] += B fragment ni x A fragment mi).
  auto mma_half = [&](const Frag<AK>(&a)[FR], const Frag<BKM>(&b)[FR]) {
#pragma unroll
    for (int ni = 0; ni < FR; ++ni)
#pragma unroll
      for (int mi = 0; mi < FR; ++mi) mfma(acc[ni][mi], as_operand(b[ni]), as_operand(a[mi]));
  };

  if (nk > 0) {
    // Prologue: slabs 0 and 1 in flight, wait for slab 0, read its first half.
    dma_slab<AK, BKM>(da, db, smem, wid, 0, half_tail && nk == 1, K, lane);
    if (nk > 1) {
      dma_slab<AK, BKM>(da, db, smem + STAGE_BYTES, wid, 1, half_tail && nk == 2, K, lane);
      wait_vm<2 * NDMA>();
    } else {
      wait_vm<0>();
    }
    __builtin_amdgcn_s_barrier();
    read_half(I0{}, I0{}, a0, b0);

    // General form of slab k (stage S = k % 2): any position, guarded.
    auto slab = [&](auto S_, int k) {
      constexpr int S = decltype(S_)::value;
      const bool full = !(half_tail && k == nk - 1);
      frag_wait<AK, BKM>(a0, b0);
      if (full) read_half(S_, I1{}, a1, b1);
      mma_half(a0, b0);
      if (k + 1 < nk) wait_vm<0>();
      frag_wait<AK, BKM>(a1, b1);
      if (k + 1 < nk) {
        __builtin_amdgcn_s_barrier();
        if (k + 2 < nk)
          dma_slab<AK, BKM>(da, db, smem + S * STAGE_BYTES, wid, k + 2, half_tail && k + 2 == nk - 1, K, lane);
        read_half(std::integral_constant<int, 1 - S>{}, I0{}, a0, b0);
      }
      if (full) mma_half(a1, b1);
    };
    // Branch-free form for slabs whose successor exists and whose k+2
    // prefetch is a full slab, with the memory instructions interleaved.
    auto steady = [&](auto S_, int k) {
      constexpr int S = decltype(S_)::value;
      frag_wait<AK, BKM>(a0, b0);
      static_for<0, 64>([&](auto i_) {
        constexpr int i = decltype(i_)::value, r = i / 2;
        mfma(acc[i / FR][i % FR], as_operand(b0[i / FR]), as_operand(a0[i % FR]));
        if constexpr ((i & 1) && r < FR) read_one<AK, S, 1, r>(a1[r], aa);
        if constexpr ((i & 1) && r >= FR && r < 2 * FR) read_one<BKM, S, 1, r - FR>(b1[r - FR], ba);
      });
      wait_vm<0>();
      frag_wait<AK, BKM>(a1, b1);
      __builtin_amdgcn_s_barrier();
      const uint32_t soa = (uint32_t)(k + 2) * da.kstep, sob = (uint32_t)(k + 2) * db.kstep;
      lds_u8* dsta = smem + S * STAGE_BYTES + wid * NDMA * 1024;
      lds_u8* dstb = dsta + TILE_BYTES;
      static_for<0, 64>([&](auto i_) {
        constexpr int i = decltype(i_)::value, j = i / 4, r = (i - 1) / 2;
        mfma(acc[i / FR][i % FR], as_operand(b1[i / FR]), as_operand(a1[i % FR]));
        if constexpr (i % 4 == 0 && j < NDMA) dma_one(da, dsta + j * 1024, j, soa);
        if constexpr (i % 4 == 0 && j >= NDMA) dma_one(db, dstb + (j - NDMA) * 1024, j - NDMA, sob);
        if constexpr ((i & 1) && r < FR) read_one<AK, 1 - S, 0, r>(a0[r], aa);
        if constexpr ((i & 1) && r >= FR && r < 2 * FR) read_one<BKM, 1 - S, 0, r - FR>(b0[r - FR], ba);
      });
    };
    const int lim = half_tail ? nk - 1 : nk;  // slabs below lim are full
    int k = 0;
    for (; k + 3 < lim; k += 2) {
      steady(I0{}, k);
      steady(I1{}, k + 1);
    }
    for (; k < nk; k += 2) {
      slab(I0{}, k);
      if (k + 1 < nk) slab(I1{}, k + 1);
    }
  }
  mfma_drain();
  __syncthreads();
  float* stage = reinterpret_cast<float*>(smem_raw);
  if constexpr (EPI == EPI_ACT && ACT_DISPATCH) {  // activation chosen once per tile
    if (P.act == ACT_TANH)
      epilogue_via_lds<EPI, WT, WT, ACT_TANH>(stage, acc, P, m0, n0, wid, wm, wn, lane, vec_c);
    else if (P.act == ACT_SILU)
      epilogue_via_lds<EPI, WT, WT, ACT_SILU>(stage, acc, P, m0, n0, wid, wm, wn, lane, vec_c);
    else
      epilogue_via_lds<EPI, WT, WT, ACT_GELU>(stage, acc, P, m0, n0, wid, wm, wn, lane, vec_c);
  } else {
    epilogue_via_lds<EPI, WT, WT>(stage, acc, P, m0, n0, wid, wm, wn, lane, vec_c);
  }
}

// Block -> (problem, tile).  Every problem's tiles start at a multiple of X =
// nxcd blocks (padding blocks exit), so a block's XCD (blockIdx % X, the
// hardware's round-robin) is its position within the problem modulo X; each
// XCD gets one contiguous run of the problem's tiles, walked in grouped
// raster order (RASTER_M tile rows per group).
// ALT_ACT: the instance for batches of activation epilogues other than GELU
// (EPI_ACT problems only); the main instance keeps GELU as its one activation.
template <bool ALT_ACT>
__global__ __launch_bounds__(NTH, 1) void gemm_bf16_dma_kernel(const GemmBatch batch) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[2 * STAGE_BYTES];
  const int bid = blockIdx.x;
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < batch.count && bid >= batch.p[i].tile_start) g = i;
  const GemmProb P = batch.p[g];  // a copy: keeps the by-value batch out of scratch
  const int ntiles = P.tiles_m * P.tiles_n;
  const int l = bid - P.tile_start;
  const int X = batch.nxcd;
  const int per_xcd = (ntiles + X - 1) / X;
  int local = (l % X) * per_xcd + l / X;
  if (local >= ntiles) return;
  const int per_group = RASTER_M * P.tiles_n;
  const int first_m = (local / per_group) * RASTER_M;
  const int gsize = min(P.tiles_m - first_m, RASTER_M);
  local %= per_group;
  const int tm = first_m + local % gsize, tn = local / gsize;
  const int vec_c = P.kind >> 8;
  if constexpr (ALT_ACT) {
    switch (P.kind & 0xff) {
      case gemm_kind(true, false, EPI_ACT): gemm_tile<true, false, EPI_ACT, true>(P, tm, tn, smem_raw, vec_c); break;
      case gemm_kind(true, true, EPI_ACT): gemm_tile<true, true, EPI_ACT, true>(P, tm, tn, smem_raw, vec_c); break;
      default: break;  // the launcher sends only activation problems here
    }
    return;
  }
  switch (P.kind & 0xff) {
    case gemm_kind(true, false, EPI_F32): gemm_tile<true, false, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_F32): gemm_tile<true, true, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(false, false, EPI_F32): gemm_tile<false, false, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(false, true, EPI_F32): gemm_tile<false, true, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, false, EPI_ACT): gemm_tile<true, false, EPI_ACT>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_ACT): gemm_tile<true, true, EPI_ACT>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, false, EPI_MUL): gemm_tile<true, false, EPI_MUL>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_MUL): gemm_tile<true, true, EPI_MUL>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, false, EPI_BF16): gemm_tile<true, false, EPI_BF16>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_BF16): gemm_tile<true, true, EPI_BF16>(P, tm, tn, smem_raw, vec_c); break;
    default: break;  // layouts the library never issues with these epilogues
  }
}

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

}  // namespace

// Eligibility of a problem for the direct-to-LDS kernel: K a multiple of 32
// (whole MFMA steps; a last half slab is handled), 16-byte aligned rows along
// each operand's contiguous dimension, an extent along it that is a multiple
// of 8 elements, operand byte ranges that the 32-bit buffer offsets can
// address, and a (layout, epilogue) pair the kernel instantiates (the activation
// and bf16-output epilogues need a k-major A).
bool gemm_bf16_dma_eligible(const GemmProb& p, bool a_kmajor, bool b_kmajor, int epi) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.K % 32 != 0) return false;
  if (epi != EPI_F32 && !a_kmajor) return false;
  const int64_t a_ld = a_kmajor ? p.sa_m : p.sa_k, b_ld = b_kmajor ? p.sb_n : p.sb_k;
  if ((a_kmajor ? p.sa_k : p.sa_m) != 1 || (b_kmajor ? p.sb_k : p.sb_n) != 1) return false;
  const int a_ext = a_kmajor ? p.K : p.M, b_ext = b_kmajor ? p.K : p.N;
  if (!aligned(p.A, 16) || !aligned(p.B, 16) || a_ld % 8 || b_ld % 8 || a_ext % 8 || b_ext % 8) return false;
  const int64_t limit = (int64_t)1 << 30;
  const int64_t a_bytes = (a_kmajor ? (int64_t)p.M * a_ld : (int64_t)p.K * a_ld) * 2;
  const int64_t b_bytes = (b_kmajor ? (int64_t)p.N * b_ld : (int64_t)p.K * b_ld) * 2;
  return a_bytes < limit && b_bytes < limit;
}

// Output vector widths a problem's epilogue may use: bit 0 for 16-byte fp32
// or 8-byte bf16 vectors, bit 1 for 16-byte bf16 vectors (8 values).
static int output_vectors(const GemmProb& p, int epi) {
  const int cbytes = epi == EPI_F32 ? 16 : 8;
  const bool v = aligned(p.C, cbytes) && p.ldc % 4 == 0 && (epi != EPI_ACT || aligned(p.aux_out, 8)) &&
                 (epi != EPI_MUL || aligned(p.aux_in, 8));
  const bool v16 = epi != EPI_F32 && aligned(p.C, 16) && p.ldc % 8 == 0 && (epi != EPI_ACT || aligned(p.aux_out, 16)) &&
                   (epi != EPI_MUL || aligned(p.aux_in, 16));
  return (v ? 1 : 0) | (v && v16 ? 2 : 0);
}

// Problems arrive with `kind` set; the launcher lays out the flattened grid
// (each problem padded to a multiple of the device's XCD count) and records
// whether each problem's outputs allow vector stores (kind bit 8).
hipError_t launch_gemm_bf16_dma(GemmBatch& b, hipStream_t s) {
  const int X = device_topology().xcds;
  b.nxcd = X;
  int total = 0;
  for (int i = 0; i < b.count; ++i) {
    GemmProb& p = b.p[i];
    const int epi = (p.kind >> 2) & 3;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.tile_start = total;
    total += ((p.tiles_m * p.tiles_n + X - 1) / X) * X;
    p.kind = (p.kind & 0xff) | (output_vectors(p, epi) << 8);
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  bool alt = false, other = false;
  for (int i = 0; i < b.count; ++i) {
    const int epi = (b.p[i].kind >> 2) & 3;
    alt |= epi == EPI_ACT && b.p[i].act != ACT_GELU;
    other |= epi != EPI_ACT;
  }
  if (alt && other) return hipErrorInvalidValue;  // such batches must hold activation problems only
  if (alt)
    hipLaunchKernelGGL(gemm_bf16_dma_kernel<true>, dim3(total), dim3(NTH), 0, s, b);
  else
    hipLaunchKernelGGL(gemm_bf16_dma_kernel<false>, dim3(total), dim3(NTH), 0, s, b);
  return hipGetLastError();
}

}  // namespace tpr
