// fp32 GEMM for the fp32 workloads (the sharded GEMM page's walk-through
// sizes and the TP lesson's fp32 self-test MLP), with the same problem
// descriptors and epilogues as the bf16 MFMA kernel.
//
// These problems are tiny (the largest is 16 x 256 x 64), so the kernel is a
// plain LDS-tiled SIMT GEMM: 64 x 64 block tile, 16-deep k slabs, 256
// threads each owning a 4 x 4 patch, fp32 FMA accumulation in a fixed k
// order.  Any operand layout is read through its strides.
#include "activation.h"

namespace tpr {
namespace {

constexpr int TBM = 64, TBN = 64, TBK = 16;

template <int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const GemmBatch batch, int a_kmajor, int b_kmajor) {
  __shared__ float As[TBK][TBM + 1];
  __shared__ float Bs[TBK][TBN + 1];
  const int tid = threadIdx.x;
  const int bid = blockIdx.x;
  int g = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i)
    if (i < batch.count && bid >= batch.p[i].tile_start) g = i;
  const GemmProb& P = batch.p[g];
  const int local = bid - P.tile_start;
  const int m0 = (local / P.tiles_n) * TBM, n0 = (local % P.tiles_n) * TBN;
  const int M = P.M, N = P.N, K = P.K;
  const float* __restrict__ A = static_cast<const float*>(P.A);
  const float* __restrict__ B = static_cast<const float*>(P.B);
  const int tm = tid >> 4, tn = tid & 15;  // 16 x 16 threads, 4 x 4 outputs each

  float acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.f;

  for (int k0 = 0; k0 < K; k0 += TBK) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = tid + 256 * i;
      const int am = a_kmajor ? e / TBK : e % TBM, ak = a_kmajor ? e % TBK : e / TBM;
      const int bn = b_kmajor ? e / TBK : e % TBN, bk = b_kmajor ? e % TBK : e / TBN;
      const int gm = m0 + am, gk = k0 + ak, gn = n0 + bn, gkb = k0 + bk;
      As[ak][am] = (gm < M && gk < K) ? A[(int64_t)gm * P.sa_m + (int64_t)gk * P.sa_k] : 0.f;
      Bs[bk][bn] = (gn < N && gkb < K) ? B[(int64_t)gkb * P.sb_k + (int64_t)gn * P.sb_n] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < TBK; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][tm * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tn * 4 + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
    }
    __syncthreads();
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + tm * 4 + i;
    if (m >= M) continue;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int n = n0 + tn * 4 + j;
      if (n >= N) continue;
      const int64_t off = (int64_t)m * P.ldc + n;
      const float v = acc[i][j];
      if constexpr (EPI == EPI_F32) {
        static_cast<float*>(P.C)[off] = v;
      } else if constexpr (EPI == EPI_ACT) {  // v is the pre-activation
        float a, da;
        act_eval_f32(P.act, v, a, da);
        static_cast<float*>(P.C)[off] = da;
        static_cast<float*>(P.aux_out)[off] = a;
      } else {  // aux_in holds sigma'(pre-activation)
        static_cast<float*>(P.C)[off] = v * static_cast<const float*>(P.aux_in)[off];
      }
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(GemmBatch& b, bool a_kmajor, bool b_kmajor, int epi, hipStream_t s) {
  b.nxcd = device_topology().xcds;
  int total = 0;
  for (int i = 0; i < b.count; ++i) {
    GemmProb& p = b.p[i];
    p.tiles_m = (p.M + TBM - 1) / TBM;
    p.tiles_n = (p.N + TBN - 1) / TBN;
    p.tile_start = total;
    total += p.tiles_m * p.tiles_n;
  }
  b.total_tiles = total;
  if (total == 0) return hipSuccess;
  const dim3 grid(total), block(256);
  const int ak = a_kmajor ? 1 : 0, bk = b_kmajor ? 1 : 0;
  switch (epi) {
    case EPI_F32: hipLaunchKernelGGL(gemm_f32_kernel<EPI_F32>, grid, block, 0, s, b, ak, bk); break;
    case EPI_ACT: hipLaunchKernelGGL(gemm_f32_kernel<EPI_ACT>, grid, block, 0, s, b, ak, bk); break;
    default: hipLaunchKernelGGL(gemm_f32_kernel<EPI_MUL>, grid, block, 0, s, b, ak, bk); break;
  }
  return hipGetLastError();
}

}  // namespace tpr
