// bf16 GEMM for gfx950 with direct-to-LDS operand loads (the fast path of
// every aligned bf16 product of the sharded GEMM page's 解题路线 and the TP
// lesson's MLP; the register-staged kernel in gemm_bf16.hip covers the rest).
//
// Operand slabs go global -> LDS with buffer_load ... lds (16 bytes per lane,
// no registers, out-of-range lanes read zeros through the buffer's range
// check) into a 4-stage LDS ring of 32-deep k slabs (4 x 32 KB).  The 256 x
// 256 block tile is computed by 8 waves (2 per SIMD) in a 2 x 4 grid, each
// owning 128 x 64 outputs (8 x 4 MFMA 16x16 blocks).  Fragments
// come out of LDS with ds_read_b128 for a k-major operand and with the gfx950
// transpose read ds_read_b64_tr_b16 for an m/n-major one, so no layout needs a
// transpose in registers.  Fragments are double-buffered in registers: the
// reads for slab k+1 are issued between the two halves of slab k's 64 MFMAs,
// after the one barrier per slab.
//
// LDS layouts (16-byte chunks, XOR-swizzled so that every fragment read is
// free of bank conflicts for 32- and 64-bank LDS phases):
//   k-major tile:  16 blocks of 1 KB, block b = rows 16b..16b+15 x 4 chunks;
//                  chunk c of row r sits at position 4 (r%16) + (c ^ kswz(r%16)).
//   m/n-major tile: 32 k-rows of 512 B (256 elements); chunk c of k-row k sits
//                  at 32 k + (c ^ mswz(k)).
// The DMA of one wave instruction fills one 1 KB block lane-linearly, so each
// lane fetches the global chunk that belongs at its LDS position.
#include "gemm_common.h"

namespace tpr {
namespace {

using namespace gemm;

constexpr int BK = 32;                    // k per LDS stage
constexpr int NS = 4;                     // LDS stages in flight
constexpr int TILE_BYTES = 256 * BK * 2;  // one operand tile per stage: 16 KB
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr int NT8 = 512;                  // 8 waves
constexpr int TM8 = 128, TN8 = 64;        // wave tile
constexpr int FM8 = TM8 / 16, FN8 = TN8 / 16;
constexpr int LOADS_PER_STAGE = 4;        // DMA instructions per wave per stage (2 per operand)
constexpr uint32_t OOB = 0x80000000u;     // voffset beyond every num_records: the load returns zeros

static_assert(NS * STAGE_BYTES >= 8 * 32 * (TN8 + 4) * 4, "epilogue staging must fit in the stage ring");

typedef __attribute__((address_space(3))) uint8_t lds_u8;
typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// A fragment is held as two 64-bit halves until it is consumed: the transpose
// reads (inline assembly) write each half directly, and the halves are only
// combined into the MFMA's 128-bit operand after the lgkmcnt wait that covers
// them, so no register copy can ever read a half before its data has landed.
struct Frag {
  u32x2 lo, hi;
};
__device__ __forceinline__ bf16x8 as_operand(const Frag& f) {
  return __builtin_bit_cast(bf16x8, u32x4{f.lo[0], f.lo[1], f.hi[0], f.hi[1]});
}

__device__ __forceinline__ int kswz(int rr) { return ((rr >> 1) & 3) ^ (((rr >> 3) & 1) * 3); }
__device__ __forceinline__ int mswz(int k) { return (2 * (k & 3)) ^ (8 * ((k >> 3) & 1)); }

// s_waitcnt with only a vmcnt limit (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm() {
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most n of this wave's loads are outstanding (n is uniform;
// rounding it down to a supported count only waits longer).
__device__ __forceinline__ void wait_vm_dyn(int n) {
  if (n >= 8) wait_vm<8>();
  else if (n >= 4) wait_vm<4>();
  else wait_vm<0>();
}

struct DmaOperand {
  __amdgpu_buffer_rsrc_t rsrc;
  uint32_t voff[2];  // this lane's byte offsets for the wave's 2 loads of a stage (at k = 0)
  uint32_t kstep;    // bytes between consecutive k slabs
};

// Operand element (r, k): k-major at X[r * ld + k], m/n-major at X[k * ld + r].
template <bool KMAJ>
__device__ __forceinline__ void dma_setup(DmaOperand& d, const void* X, int64_t ld, int R, int K, int r0, int wid,
                                          int lane) {
  const int64_t bytes = KMAJ ? ((int64_t)(R - 1) * ld + K) * 2 : ((int64_t)(K - 1) * ld + R) * 2;
  d.rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(X), (short)0, (int)bytes, 0x00020000);
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int b = wid * 2 + j;
    if constexpr (KMAJ) {
      const int rr = lane >> 2, c = (lane & 3) ^ kswz(rr);
      const int gr = r0 + 16 * b + rr;
      d.voff[j] = gr < R ? (uint32_t)(((int64_t)gr * ld + 8 * c) * 2) : OOB;
    } else {
      const int kl = 2 * b + (lane >> 5), c = (lane & 31) ^ mswz(kl);
      const int gr = r0 + 8 * c;
      d.voff[j] = gr < R ? (uint32_t)(((int64_t)kl * ld + gr) * 2) : OOB;
    }
  }
  d.kstep = KMAJ ? BK * 2 : (uint32_t)(BK * ld * 2);
}

__device__ __forceinline__ void dma_issue(const DmaOperand& d, lds_u8* tile, int wid, int kt) {
  lds_u8* base = tile + wid * 2 * 1024;
  const uint32_t soff = (uint32_t)kt * d.kstep;
#pragma unroll
  for (int j = 0; j < 2; ++j)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsrc, (__attribute__((address_space(3))) void*)(base + j * 1024), 16,
                                             d.voff[j], soff, 0, 0);
}

__device__ __forceinline__ void dma_one(const DmaOperand& d, lds_u8* dst, int j, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rsrc, (__attribute__((address_space(3))) void*)dst, 16, d.voff[j], soff,
                                           0, 0);
}

// Per-lane LDS byte offsets of the NF fragments (rows row0 + 16 f .. +15) a
// wave reads from one tile.
template <bool KMAJ, int NF>
__device__ __forceinline__ void frag_offsets(uint32_t (&off)[NF], int row0, int lane) {
#pragma unroll
  for (int f = 0; f < NF; ++f) {
    if constexpr (KMAJ) {
      const int rr = lane & 15, c = lane >> 4;
      off[f] = (row0 / 16 + f) * 1024 + (rr * 4 + (c ^ kswz(rr))) * 16;
    } else {
      const int G = lane >> 4, q = lane & 15;
      const int kl = 8 * G + (q >> 2);
      const int c = row0 / 8 + 2 * f + ((q & 3) >> 1);
      off[f] = kl * 512 + ((c ^ mswz(kl)) * 16) + (q & 1) * 8;
    }
  }
}

// Transpose read of one m/n-major fragment: two ds_read_b64_tr_b16 (k = 8G..8G+3
// and 8G+4..8G+7 of the lane's row).  Issued as inline assembly because the
// compiler places a wait for every outstanding LDS DMA in front of the builtin
// form, which would drain the stage ring each slab; the caller therefore waits
// on lgkmcnt itself (frag_wait) before the fragments are used.
__device__ __forceinline__ Frag ds_read_tr_frag(uint32_t addr) {
  Frag f;
  asm volatile("ds_read_b64_tr_b16 %0, %2\n\tds_read_b64_tr_b16 %1, %2 offset:2048"
               : "=&v"(f.lo), "=&v"(f.hi)
               : "v"(addr));
  return f;
}

template <bool KMAJ>
__device__ __forceinline__ Frag read_frag(const lds_u8* tile, uint32_t off) {
  if constexpr (KMAJ) {
    const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(tile + off);
    return Frag{u32x2{v[0], v[1]}, u32x2{v[2], v[3]}};
  } else {
    return ds_read_tr_frag((uint32_t)(uintptr_t)(tile + off));
  }
}

template <bool KMAJ, int NF>
__device__ __forceinline__ void read_frags(Frag (&fr)[NF], const lds_u8* tile, const uint32_t (&off)[NF]) {
#pragma unroll
  for (int f = 0; f < NF; ++f) fr[f] = read_frag<KMAJ>(tile, off[f]);
}

// Wait for this wave's outstanding LDS reads and make both halves of every
// fragment depend on the wait, so nothing that reads them (MFMA operand
// assembly included) can be scheduled above it.
template <int NF>
__device__ __forceinline__ void frag_wait(Frag (&fr)[NF]) {
  static_assert(NF == 4 || NF == 8, "fragment count");
  if constexpr (NF == 4) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(fr[0].lo), "+v"(fr[0].hi), "+v"(fr[1].lo), "+v"(fr[1].hi), "+v"(fr[2].lo), "+v"(fr[2].hi),
                   "+v"(fr[3].lo), "+v"(fr[3].hi));
  } else {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(fr[0].lo), "+v"(fr[0].hi), "+v"(fr[1].lo), "+v"(fr[1].hi), "+v"(fr[2].lo), "+v"(fr[2].hi),
                   "+v"(fr[3].lo), "+v"(fr[3].hi), "+v"(fr[4].lo), "+v"(fr[4].hi), "+v"(fr[5].lo), "+v"(fr[5].hi),
                   "+v"(fr[6].lo), "+v"(fr[6].hi), "+v"(fr[7].lo), "+v"(fr[7].hi));
  }
}

template <int NI0>
__device__ __forceinline__ void mma_half(floatx4 (&acc)[FN8][FM8], const Frag (&a)[FM8], const Frag (&b)[FN8]) {
#pragma unroll
  for (int ni = NI0; ni < NI0 + FN8 / 2; ++ni)
#pragma unroll
    for (int mi = 0; mi < FM8; ++mi)
      acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_operand(b[ni]), as_operand(a[mi]), acc[ni][mi], 0, 0, 0);
}

// One 256 x 256 output tile of problem P.
template <bool AK, bool BKM, int EPI>
__device__ __forceinline__ void gemm_tile(const GemmProb& P, int tm, int tn, uint8_t* smem_raw, int vec_c) {
  lds_u8* smem = (lds_u8*)smem_raw;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wid >> 2, wn = wid & 3;
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tm * BM, n0 = tn * BN;

  DmaOperand da, db;
  dma_setup<AK>(da, P.A, AK ? P.sa_m : P.sa_k, M, K, m0, wid, lane);
  dma_setup<BKM>(db, P.B, BKM ? P.sb_n : P.sb_k, N, K, n0, wid, lane);
  uint32_t aoff[FM8], boff[FN8];
  frag_offsets<AK, FM8>(aoff, wm * TM8, lane);
  frag_offsets<BKM, FN8>(boff, wn * TN8, lane);

  floatx4 acc[FN8][FM8];
#pragma unroll
  for (int ni = 0; ni < FN8; ++ni)
#pragma unroll
    for (int mi = 0; mi < FM8; ++mi) acc[ni][mi] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / BK;
  if (nk > 0) {
    // Prologue: stages 0 .. NS-2 in flight, wait for stage 0, read its fragments.
#pragma unroll
    for (int s = 0; s < NS - 1; ++s)
      if (s < nk) {
        dma_issue(da, smem + s * STAGE_BYTES, wid, s);
        dma_issue(db, smem + s * STAGE_BYTES + TILE_BYTES, wid, s);
      }
    wait_vm_dyn(min(NS - 2, nk - 1) * LOADS_PER_STAGE);
    __builtin_amdgcn_s_barrier();

    Frag fa[2][FM8], fb[2][FN8];
    read_frags<AK, FM8>(fa[0], smem, aoff);
    read_frags<BKM, FN8>(fb[0], smem + TILE_BYTES, boff);

    // One slab per step; the fragment register sets alternate, so loops cover
    // a pair of slabs.  `step` is the general form (any position, guarded);
    // `steady` is the branch-free form used while every slab still has a
    // successor to read and a slab to prefetch.  In `steady` the second half
    // of the MFMAs is interleaved with the slab's 4 DMA issues and the next
    // fragment reads, and scheduling fences keep the first half ahead of the
    // barrier (the MFMAs carry no memory dependency the compiler could see).
    auto step = [&](int kt, Frag(&ca)[FM8], Frag(&cb)[FN8], Frag(&na)[FM8], Frag(&nb)[FN8]) {
      frag_wait<FM8>(ca);
      frag_wait<FN8>(cb);
      mma_half<0>(acc, ca, cb);
      if (kt + 1 < nk) {
        wait_vm_dyn((min(kt + NS - 2, nk - 1) - (kt + 1)) * LOADS_PER_STAGE);
        __builtin_amdgcn_s_barrier();
        const int s_new = kt + NS - 1;
        if (s_new < nk) {
          lds_u8* st = smem + (s_new % NS) * STAGE_BYTES;
          dma_issue(da, st, wid, s_new);
          dma_issue(db, st + TILE_BYTES, wid, s_new);
        }
        const lds_u8* nx = smem + ((kt + 1) % NS) * STAGE_BYTES;
        read_frags<AK, FM8>(na, nx, aoff);
        read_frags<BKM, FN8>(nb, nx + TILE_BYTES, boff);
      }
      mma_half<FN8 / 2>(acc, ca, cb);
    };
    auto steady = [&](int kt, Frag(&ca)[FM8], Frag(&cb)[FN8], Frag(&na)[FM8], Frag(&nb)[FN8]) {
      frag_wait<FM8>(ca);
      frag_wait<FN8>(cb);
      mma_half<0>(acc, ca, cb);
      __builtin_amdgcn_sched_barrier(0);
      wait_vm<(NS - 3) * LOADS_PER_STAGE>();
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      const int s_new = kt + NS - 1;
      lds_u8* st = smem + (s_new % NS) * STAGE_BYTES;
      const lds_u8* nx = smem + ((kt + 1) % NS) * STAGE_BYTES;
      const uint32_t soa = (uint32_t)s_new * da.kstep, sob = (uint32_t)s_new * db.kstep;
      lds_u8* dsta = st + wid * 2 * 1024;
      lds_u8* dstb = st + TILE_BYTES + wid * 2 * 1024;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int ni = FN8 / 2 + i / FM8, mi = i % FM8;
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_operand(cb[ni]), as_operand(ca[mi]), acc[ni][mi], 0, 0, 0);
        if (i == 0) dma_one(da, dsta, 0, soa);
        if (i == 2) dma_one(da, dsta + 1024, 1, soa);
        if (i == 4) dma_one(db, dstb, 0, sob);
        if (i == 6) dma_one(db, dstb + 1024, 1, sob);
        if (i >= 1 && i < 1 + FM8) na[i - 1] = read_frag<AK>(nx, aoff[i - 1]);
        if (i >= 1 + FM8 && i < 1 + FM8 + FN8) nb[i - 1 - FM8] = read_frag<BKM>(nx + TILE_BYTES, boff[i - 1 - FM8]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);  // one VMEM (the DMA)
      }
#pragma unroll
      for (int i = 0; i < 12; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
      }
      __builtin_amdgcn_sched_barrier(0);
    };
    int kt = 0;
    for (; kt + NS < nk; kt += 2) {
      steady(kt, fa[0], fb[0], fa[1], fb[1]);
      steady(kt + 1, fa[1], fb[1], fa[0], fb[0]);
    }
    for (; kt < nk; kt += 2) {
      step(kt, fa[0], fb[0], fa[1], fb[1]);
      if (kt + 1 < nk) step(kt + 1, fa[1], fb[1], fa[0], fb[0]);
    }
  }
  __syncthreads();
  epilogue_via_lds<EPI, TM8, TN8>(reinterpret_cast<float*>(smem_raw), acc, P, m0, n0, wid, wm, wn, lane, vec_c);
}

// Block -> (problem, tile).  Every problem's tiles start at a multiple of 8
// blocks (padding blocks exit), so a block's XCD (blockIdx % 8, the hardware's
// round-robin) is its position within the problem modulo 8; each XCD gets one
// contiguous run of the problem's tiles, walked in grouped raster order.
__global__ __launch_bounds__(NT8, 1) void gemm_bf16_dma_kernel(const GemmBatch batch) {
  __shared__ __attribute__((aligned(1024))) uint8_t smem_raw[NS * STAGE_BYTES];
  const int bid = blockIdx.x;
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < batch.count && bid >= batch.p[i].tile_start) g = i;
  const GemmProb& P = batch.p[g];
  const int ntiles = P.tiles_m * P.tiles_n;
  const int l = bid - P.tile_start;
  const int per_xcd = (ntiles + 7) >> 3;
  int local = (l & 7) * per_xcd + (l >> 3);
  if (local >= ntiles) return;
  const int per_group = GROUP_M * P.tiles_n;
  const int first_m = (local / per_group) * GROUP_M;
  const int gsize = min(P.tiles_m - first_m, GROUP_M);
  local %= per_group;
  const int tm = first_m + local % gsize, tn = local / gsize;
  const int vec_c = P.kind >> 8;
  switch (P.kind & 0xff) {
    case gemm_kind(true, false, EPI_F32): gemm_tile<true, false, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_F32): gemm_tile<true, true, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(false, false, EPI_F32): gemm_tile<false, false, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(false, true, EPI_F32): gemm_tile<false, true, EPI_F32>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, false, EPI_GELU): gemm_tile<true, false, EPI_GELU>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_GELU): gemm_tile<true, true, EPI_GELU>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, false, EPI_DGELU): gemm_tile<true, false, EPI_DGELU>(P, tm, tn, smem_raw, vec_c); break;
    case gemm_kind(true, true, EPI_DGELU): gemm_tile<true, true, EPI_DGELU>(P, tm, tn, smem_raw, vec_c); break;
    default: break;  // layouts the library never issues with these epilogues
  }
}

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

}  // namespace

// Eligibility of a problem for the direct-to-LDS kernel: K a multiple of the
// 32-deep slab, 16-byte aligned rows along each operand's contiguous
// dimension, an extent along it that is a multiple of 8 elements, operand byte
// ranges that the 32-bit buffer offsets can address, and a (layout, epilogue)
// pair the kernel instantiates (the GELU epilogues need a k-major A).
bool gemm_bf16_dma_eligible(const GemmProb& p, bool a_kmajor, bool b_kmajor, int epi) {
  if (p.M <= 0 || p.N <= 0 || p.K <= 0 || p.K % BK != 0) return false;
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

// Problems arrive with `kind` set; the launcher lays out the flattened grid
// (each problem padded to a multiple of 8 blocks) and records whether each
// problem's outputs allow vector stores (kind bit 8).
hipError_t launch_gemm_bf16_dma(GemmBatch& b, hipStream_t s) {
  int total = 0;
  for (int i = 0; i < b.count; ++i) {
    GemmProb& p = b.p[i];
    const int epi = (p.kind >> 2) & 3;
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.tile_start = total;
    total += ((p.tiles_m * p.tiles_n + 7) / 8) * 8;
    const int cbytes = epi == EPI_F32 ? 16 : 8;
    const bool vec_c = aligned(p.C, cbytes) && p.ldc % 4 == 0 && (epi != EPI_GELU || aligned(p.aux_out, 8)) &&
                       (epi != EPI_DGELU || aligned(p.aux_in, 8));
    p.kind = (p.kind & 0xff) | (vec_c ? 0x100 : 0);
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  hipLaunchKernelGGL(gemm_bf16_dma_kernel, dim3(total), dim3(NT8), 0, s, b);
  return hipGetLastError();
}

}  // namespace tpr
