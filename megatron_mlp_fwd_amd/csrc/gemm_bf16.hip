// bf16 GEMM on the gfx950 matrix cores (v_mfma_f32_16x16x32_bf16), fp32
// accumulation, with the GELU / GELU' epilogues of the tensor-parallel MLP.
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
#include "common.h"

namespace tpr {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NT = 256;
constexpr int WTM = 128, WTN = 128;
constexpr int FM = WTM / 16, FN = WTN / 16;
constexpr int STAGE = (BM + BN) * BK;  // bf16 elements per LDS stage
constexpr int GROUP_M = 8;             // tile rows per raster group (L2 reuse of B)

// 16-byte chunk swizzle of a k-contiguous LDS row (8 chunks per row); keeps
// both the fragment reads and the row writes free of bank conflicts for 8- and
// 16-lane LDS phases.
__device__ __forceinline__ int swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

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
// walks a contiguous range of tiles (neighbouring tiles share L2 there).
__device__ __forceinline__ int xcd_remap(int bid, int total) {
  const int per = total >> 3, rem = total & 7;
  const int x = bid & 7, slot = bid >> 3;
  return x * per + (x < rem ? x : rem) + slot;
}

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

constexpr int EP_LD = WTN + 4;  // padded fp32 row of the epilogue staging area

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

template <bool AK, bool BKM, bool VEC, int EPI>
__global__ __launch_bounds__(NT, 1) void gemm_bf16_kernel(const GemmBatch batch, int vec_c) {
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid >> 1, wn = wid & 1;

  const int bid = xcd_remap((int)blockIdx.x, batch.total_tiles);
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < batch.count && bid >= batch.p[i].tile_start) g = i;
  const GemmProb& P = batch.p[g];
  const int M = P.M, N = P.N, K = P.K;

  int local = bid - P.tile_start;
  const int per_group = GROUP_M * P.tiles_n;
  const int first_m = (local / per_group) * GROUP_M;
  const int gsize = min(P.tiles_m - first_m, GROUP_M);
  local %= per_group;
  const int tm = first_m + local % gsize;
  const int tn = local / gsize;
  const int m0 = tm * BM, n0 = tn * BN;

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

  // Epilogue, in four passes through LDS (the operand stages are free now):
  // pass q moves MFMA blocks mi = 2q, 2q+1 of every wave (a 32 x 128 region
  // per wave) into LDS, then each wave reads its region back row-contiguously
  // (32 lanes x 16 B per row) and applies the epilogue with coalesced stores.
  float* ep = reinterpret_cast<float*>(smem) + wid * (32 * EP_LD);
  const int64_t ldc = P.ldc;
#pragma unroll
  for (int q = 0; q < FM / 2; ++q) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int ni = 0; ni < FN; ++ni)
        *reinterpret_cast<floatx4*>(ep + (h * 16 + (lane & 15)) * EP_LD + ni * 16 + 4 * (lane >> 4)) =
            acc[ni][2 * q + h];
    __syncthreads();
    const int col = 4 * (lane & 31);
    const int n = n0 + wn * WTN + col;
    for (int it = 0; it < 16; ++it) {
      const int row = 2 * it + (lane >> 5);
      const int m = m0 + wm * WTM + 32 * q + row;
      if (m < M && n < N) {
        floatx4 v = *reinterpret_cast<const floatx4*>(ep + row * EP_LD + col);
        epilogue_store<EPI>(P, v, (int64_t)m * ldc + n, n, N, vec_c);
      }
    }
    __syncthreads();
  }
}

template <bool AK, bool BKM, bool VEC>
hipError_t launch_epi(const GemmBatch& b, int epi, int vec_c, hipStream_t s) {
  const dim3 grid(b.total_tiles), block(NT);
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_F32>), grid, block, 0, s, b, vec_c); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_GELU>), grid, block, 0, s, b, vec_c); break;
    default: hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKM, VEC, EPI_DGELU>), grid, block, 0, s, b, vec_c); break;
  }
  return hipGetLastError();
}

bool aligned(const void* p, int bytes) { return (reinterpret_cast<uintptr_t>(p) % bytes) == 0; }

}  // namespace

hipError_t launch_gemm_bf16(GemmBatch& b, bool a_kmajor, bool b_kmajor, int epi, hipStream_t s) {
  int total = 0;
  bool vec = true, vec_c = true;
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
    vec_c = vec_c && aligned(p.C, cbytes) && p.ldc % 4 == 0 && (epi != EPI_GELU || aligned(p.aux_out, 8)) &&
            (epi != EPI_DGELU || aligned(p.aux_in, 8));
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  const int vc = vec_c ? 1 : 0;
  if (a_kmajor && !b_kmajor) return vec ? launch_epi<true, false, true>(b, epi, vc, s) : launch_epi<true, false, false>(b, epi, vc, s);
  if (a_kmajor && b_kmajor) return vec ? launch_epi<true, true, true>(b, epi, vc, s) : launch_epi<true, true, false>(b, epi, vc, s);
  if (!a_kmajor && !b_kmajor) return vec ? launch_epi<false, false, true>(b, epi, vc, s) : launch_epi<false, false, false>(b, epi, vc, s);
  return vec ? launch_epi<false, true, true>(b, epi, vc, s) : launch_epi<false, true, false>(b, epi, vc, s);
}

}  // namespace tpr
