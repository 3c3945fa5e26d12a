// bf16 GEMM on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fp32
// accumulation, with the activation / activation-derivative epilogues of the
// tensor-parallel MLP.
//
// Every per-rank product of the sharded GEMM page ("Sharded GEMM与Backprop：
// 行、列、内维三种切分", 解题路线 steps 1-4) and of the TP lesson's MLP
// ("第 6 课：张量并行 TP", 2.A; backward from "多卡张量：拆开计算，再合回同一
// 结果", 02 / BACKWARD) is one of three operand layouts:
//   NN  Y = A B       A k-major, B n-major   (forward products)
//   NT  dA = G B^T    A k-major, B k-major   (input gradients)
//   TN  dB = A^T G    A m-major, B n-major   (weight gradients)
// The kernel takes the layout of each operand as a template flag.
//
// Block tile 256 x 256 x 64, 256 threads = 4 waves in a 2 x 2 grid, each wave
// owning a 128 x 128 sub-tile = 8 x 8 MFMA 16x16 blocks (256 fp32
// accumulators per lane).  Operand tiles are staged global -> registers ->
// LDS in a k-contiguous, XOR-swizzled layout (two LDS stages, 128 KB); an
// m/n-major operand is transposed in registers (8 x 8 bf16 blocks) on its way
// into LDS, so every MFMA fragment is a single 16-byte LDS read.  The MFMA
// roles are swapped (B fragment as the 16-row operand) so that each lane ends
// with four consecutive output columns of one row: 16-byte fp32 stores.
//
// Grouped launch: up to kMaxGroup problems (one per simulated rank) share a
// flattened grid; each block finds its problem by tile_start.
#include "gemm_common.h"

namespace tpr {
namespace {

using namespace gemm;

constexpr int BK = 64;
constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per LDS stage

// 16-byte chunk swizzle of a k-contiguous LDS row (8 chunks per row); keeps
// both the fragment reads and the row writes free of bank conflicts for 8- and
// 16-lane LDS phases.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

// Load one 64-deep k-slab of an operand with R rows (the M or N side) into
// eight 16-byte registers.  Operand element (r, k) = X[r * s_r + k * s_k].
//  k-major: thread owns chunk c = tid%8 (k = 8c..8c+7) of rows tid/8 + 32 j.
//  r-major: thread owns the 8 x 8 block k = 8 (tid%8) + j, r = 8 (tid/8) + e.
template <bool KMAJ, bool VEC>
__device__ __forceinline__ void load_slab(u32x4 (&reg)[8], const uint16_t* __restrict__ X, int64_t s_r,
                                          int64_t s_k, int R, int K, int r0, int k0, int tid) {
  if constexpr (KMAJ) {
    const int c = tid & 7, rr = tid >> 3;
    const int k = k0 + 8 * c;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = r0 + rr + 32 * j;
      if constexpr (VEC) {
        reg[j] = (r < R && k < K) ? *reinterpret_cast<const u32x4*>(X + (int64_t)r * s_r + k) : u32x4{0, 0, 0, 0};
      } else {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ka = k + 2 * q, kb = ka + 1;
          const uint32_t lo = (r < R && ka < K) ? X[(int64_t)r * s_r + (int64_t)ka * s_k] : 0u;
          const uint32_t hi = (r < R && kb < K) ? X[(int64_t)r * s_r + (int64_t)kb * s_k] : 0u;
          w[q] = lo | (hi << 16);
        }
        reg[j] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  } else {
    const int kc = tid & 7, rc = tid >> 3;
    const int r = r0 + 8 * rc;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int k = k0 + 8 * kc + j;
      if constexpr (VEC) {
        reg[j] = (k < K && r < R) ? *reinterpret_cast<const u32x4*>(X + (int64_t)k * s_k + r) : u32x4{0, 0, 0, 0};
      } else {
        uint32_t w[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int ra = r + 2 * q, rb = ra + 1;
          const uint32_t lo = (k < K && ra < R) ? X[(int64_t)k * s_k + (int64_t)ra * s_r] : 0u;
          const uint32_t hi = (k < K && rb < R) ? X[(int64_t)k * s_k + (int64_t)rb * s_r] : 0u;
          w[q] = lo | (hi << 16);
        }
        reg[j] = u32x4{w[0], w[1], w[2], w[3]};
      }
    }
  }
}

// Write a slab loaded by load_slab into one LDS operand tile [rows][BK].
template <bool KMAJ>
__device__ __forceinline__ void store_slab(uint16_t* __restrict__ S, const u32x4 (&reg)[8], int tid) {
  if constexpr (KMAJ) {
    const int c = tid & 7, rr = tid >> 3;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int r = rr + 32 * j;
      *reinterpret_cast<u32x4*>(S + r * BK + ((c ^ swz(r)) << 3)) = reg[j];
    }
  } else {
    // reg[j] holds k = 8 kc + j for rows 8 rc .. 8 rc + 7 (dword q: rows 2q, 2q+1).
    const int kc = tid & 7, rc = tid >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int r = 8 * rc + i, q = i >> 1;
      uint32_t w[4];
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const uint32_t a = reg[2 * p][q], b = reg[2 * p + 1][q];
        w[p] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
      }
      *reinterpret_cast<u32x4*>(S + r * BK + ((kc ^ swz(r)) << 3)) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

__device__ __forceinline__ void mma_stage(const uint16_t* __restrict__ As, const uint16_t* __restrict__ Bs,
                                          floatx4 (&acc)[FN][FM], int lane, int wm, int wn) {
  const int r16 = lane & 15, grp = lane >> 4;
  const int s = swz(r16);  // fragment rows start at multiples of 16
#pragma unroll
  for (int kk = 0; kk < BK / 32; ++kk) {
    const int ch = ((kk * 4 + grp) ^ s) << 3;
    bf16x8 af[FM], bfr[FN];
#pragma unroll
    for (int mi = 0; mi < FM; ++mi)
      af[mi] = *reinterpret_cast<const bf16x8*>(As + (wm * WTM + mi * 16 + r16) * BK + ch);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
      bfr[ni] = *reinterpret_cast<const bf16x8*>(Bs + (wn * WTN + ni * 16 + r16) * BK + ch);
#pragma unroll
    for (int ni = 0; ni < FN; ++ni)
#pragma unroll
      for (int mi = 0; mi < FM; ++mi)
        acc[ni][mi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(bfr[ni], af[mi], acc[ni][mi], 0, 0, 0);
  }
}

// ACT: the activation of EPI_ACT (one kernel instance per activation).
template <bool AK, bool BKM, bool VEC, int EPI, int ACT = ACT_GELU>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const GemmBatch batch, int vec_c) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  const TileCoord tc = locate_tile(batch);
  const GemmProb& P = batch.p[tc.g];
  const int M = P.M, N = P.N, K = P.K;
  const int m0 = tc.tm * BM, n0 = tc.tn * BN;

  const uint16_t* __restrict__ A = static_cast<const uint16_t*>(P.A);
  const uint16_t* __restrict__ B = static_cast<const uint16_t*>(P.B);

  floatx4 acc[FN][FM];
#pragma unroll
  for (int ni = 0; ni < FN; ++ni)
#pragma unroll
    for (int mi = 0; mi < FM; ++mi) acc[ni][mi] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  u32x4 ra[8], rb[8];
  if (nk > 0) {
    load_slab<AK, VEC>(ra, A, P.sa_m, P.sa_k, M, K, m0, 0, tid);
    load_slab<BKM, VEC>(rb, B, P.sb_n, P.sb_k, N, K, n0, 0, tid);
    store_slab<AK>(smem, ra, tid);
    store_slab<BKM>(smem + BM * BK, rb, tid);
  }
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    uint16_t* cur = smem + (kt & 1) * STAGE;
    uint16_t* nxt = smem + ((kt + 1) & 1) * STAGE;
    const bool more = kt + 1 < nk;
    if (more) {
      load_slab<AK, VEC>(ra, A, P.sa_m, P.sa_k, M, K, m0, (kt + 1) * BK, tid);
      load_slab<BKM, VEC>(rb, B, P.sb_n, P.sb_k, N, K, n0, (kt + 1) * BK, tid);
    }
    mma_stage(cur, cur + BM * BK, acc, lane, wm, wn);
    if (more) {
      store_slab<AK>(nxt, ra, tid);
      store_slab<BKM>(nxt + BM * BK, rb, tid);
    }
    __syncthreads();
  }

  epilogue_via_lds<EPI, WTM, WTN, ACT>(reinterpret_cast<float*>(smem), acc, P, m0, n0, wid, wm, wn, lane, vec_c);
}

template <bool AK, bool BKM, bool VEC>
hipError_t launch_epi(const GemmBatch& b, int epi, int vec_c, hipStream_t s) {
  const dim3 grid(b.total_tiles), block(NT);
  const int act = b.count > 0 ? b.p[0].act : ACT_GELU;
  if (epi == EPI_ACT)
    for (int i = 1; i < b.count; ++i)
      if (b.p[i].act != act) return hipErrorInvalidValue;  // one activation per launch
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_F32>), grid, block, 0, s, b, vec_c); break;
    case EPI_ACT:
      if (act == ACT_TANH)
        hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_ACT, ACT_TANH>), grid, block, 0, s, b, vec_c);
      else if (act == ACT_SILU)
        hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_ACT, ACT_SILU>), grid, block, 0, s, b, vec_c);
      else
        hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_ACT, ACT_GELU>), grid, block, 0, s, b, vec_c);
      break;
    case EPI_BF16: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_BF16>), grid, block, 0, s, b, vec_c); break;
    default: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_MUL>), grid, block, 0, s, b, vec_c); break;
  }
  return hipGetLastError();
}

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

}  // namespace

hipError_t launch_gemm_bf16(GemmBatch& b, bool a_kmajor, bool b_kmajor, int epi, hipStream_t s) {
  b.nxcd = device_topology().xcds;
  int total = 0;
  bool vec = true, vec_c = true, vec16 = true;
  for (int i = 0; i < b.count; ++i) {
    GemmProb& p = b.p[i];
    p.tiles_m = (p.M + BM - 1) / BM;
    p.tiles_n = (p.N + BN - 1) / BN;
    p.tile_start = total;
    total += p.tiles_m * p.tiles_n;
    // Vector loads need 16-byte aligned rows along the contiguous dimension
    // and a contiguous extent that is a multiple of 8 elements.
    const int64_t a_ld = a_kmajor ? p.sa_m : p.sa_k, b_ld = b_kmajor ? p.sb_n : p.sb_k;
    const int a_ext = a_kmajor ? p.K : p.M, b_ext = b_kmajor ? p.K : p.N;
    vec = vec && aligned(p.A, 16) && aligned(p.B, 16) && a_ld % 8 == 0 && b_ld % 8 == 0 && a_ext % 8 == 0 &&
          b_ext % 8 == 0;
    const int cbytes = epi == EPI_F32 ? 16 : 8;
    vec_c = vec_c && aligned(p.C, cbytes) && p.ldc % 4 == 0 && (epi != EPI_ACT || aligned(p.aux_out, 8)) &&
            (epi != EPI_MUL || aligned(p.aux_in, 8));
    vec16 = vec16 && epi != EPI_F32 && aligned(p.C, 16) && p.ldc % 8 == 0 &&
            (epi != EPI_ACT || aligned(p.aux_out, 16)) && (epi != EPI_MUL || aligned(p.aux_in, 16));
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  const int vc = (vec_c ? 1 : 0) | (vec_c && vec16 ? 2 : 0);
  if (a_kmajor && !b_kmajor) return vec ? launch_epi<true, false, true>(b, epi, vc, s) : launch_epi<true, false, false>(b, epi, vc, s);
  if (a_kmajor && b_kmajor) return vec ? launch_epi<true, true, true>(b, epi, vc, s) : launch_epi<true, true, false>(b, epi, vc, s);
  if (!a_kmajor && !b_kmajor) return vec ? launch_epi<false, false, true>(b, epi, vc, s) : launch_epi<false, false, false>(b, epi, vc, s);
  return vec ? launch_epi<false, true, true>(b, epi, vc, s) : launch_epi<false, true, false>(b, epi, vc, s);
}

}  // namespace tpr
