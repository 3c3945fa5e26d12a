// Element-wise steps of the gated (gate / up) MLP.
//
// TP lesson page ("第 6 课：张量并行 TP"), question 1: the gate and up
// projections and the activation sit on the column-parallel side, so each
// rank owns matching column blocks of A = X W1 (gate) and U = X W3 (up) and
// combines them locally:
//   forward   H  = sigma(A) * U
//   backward  dA = dH * U * sigma'(A),   dU = dH * sigma(A)
// (the multi-card tensor page's 02 / BACKWARD rule G_Z = G_H * sigma',
// applied to both factors of the product).  The rank blocks are contiguous in
// one T x f buffer, so one launch covers every rank.  Memory bound: 16-byte
// vectors of 8 bf16 (or 4 fp32) per thread and iteration, a scalar tail.
#include "activation.h"

namespace tpr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ uint16_t to_bf(float x) { return __builtin_bit_cast(uint16_t, (__bf16)x); }
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// One v_cvt_pk_bf16_f32 (round to nearest even) per pair.
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// bf16: fast fp32 activations (results rounded to bf16 anyway).
__global__ __launch_bounds__(256) void glu_fwd_bf16(const uint16_t* __restrict__ A, const uint16_t* __restrict__ U,
                                                    uint16_t* __restrict__ H, int64_t n, int act) {
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nv; i += stride) {
    const u32x4 a = reinterpret_cast<const u32x4*>(A)[i];
    const u32x4 u = reinterpret_cast<const u32x4*>(U)[i];
    u32x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s0, d0, s1, d1;
      act_eval(act, bf_lo(a[q]), s0, d0);
      act_eval(act, bf_hi(a[q]), s1, d1);
      h[q] = pack2(s0 * bf_lo(u[q]), s1 * bf_hi(u[q]));
    }
    reinterpret_cast<u32x4*>(H)[i] = h;
  }
  const int64_t t = 8 * nv + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) {
    float s, ds;
    act_eval(act, bf(A[t]), s, ds);
    H[t] = to_bf(s * bf(U[t]));
  }
}

// dA is read as dH and overwritten in place.
__global__ __launch_bounds__(256) void glu_bwd_bf16(uint16_t* __restrict__ dA, const uint16_t* __restrict__ A,
                                                    const uint16_t* __restrict__ U, uint16_t* __restrict__ dU,
                                                    int64_t n, int act) {
  const int64_t nv = n / 8;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nv; i += stride) {
    const u32x4 g = reinterpret_cast<const u32x4*>(dA)[i];
    const u32x4 a = reinterpret_cast<const u32x4*>(A)[i];
    const u32x4 u = reinterpret_cast<const u32x4*>(U)[i];
    u32x4 ga, gu;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s0, d0, s1, d1;
      act_eval(act, bf_lo(a[q]), s0, d0);
      act_eval(act, bf_hi(a[q]), s1, d1);
      const float g0 = bf_lo(g[q]), g1 = bf_hi(g[q]);
      ga[q] = pack2(g0 * bf_lo(u[q]) * d0, g1 * bf_hi(u[q]) * d1);
      gu[q] = pack2(g0 * s0, g1 * s1);
    }
    reinterpret_cast<u32x4*>(dA)[i] = ga;
    reinterpret_cast<u32x4*>(dU)[i] = gu;
  }
  const int64_t t = 8 * nv + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) {
    float s, ds;
    act_eval(act, bf(A[t]), s, ds);
    const float g = bf(dA[t]);
    dA[t] = to_bf(g * bf(U[t]) * ds);
    dU[t] = to_bf(g * s);
  }
}

// fp32: full-precision activations.
__global__ __launch_bounds__(256) void glu_fwd_f32(const float* __restrict__ A, const float* __restrict__ U,
                                                   float* __restrict__ H, int64_t n, int act) {
  const int64_t nv = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nv; i += stride) {
    const f32x4 a = reinterpret_cast<const f32x4*>(A)[i];
    const f32x4 u = reinterpret_cast<const f32x4*>(U)[i];
    f32x4 h;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s, ds;
      act_eval_f32(act, a[q], s, ds);
      h[q] = s * u[q];
    }
    reinterpret_cast<f32x4*>(H)[i] = h;
  }
  const int64_t t = 4 * nv + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) {
    float s, ds;
    act_eval_f32(act, A[t], s, ds);
    H[t] = s * U[t];
  }
}

__global__ __launch_bounds__(256) void glu_bwd_f32(float* __restrict__ dA, const float* __restrict__ A,
                                                   const float* __restrict__ U, float* __restrict__ dU, int64_t n,
                                                   int act) {
  const int64_t nv = n / 4;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nv; i += stride) {
    const f32x4 g = reinterpret_cast<const f32x4*>(dA)[i];
    const f32x4 a = reinterpret_cast<const f32x4*>(A)[i];
    const f32x4 u = reinterpret_cast<const f32x4*>(U)[i];
    f32x4 ga, gu;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float s, ds;
      act_eval_f32(act, a[q], s, ds);
      ga[q] = g[q] * u[q] * ds;
      gu[q] = g[q] * s;
    }
    reinterpret_cast<f32x4*>(dA)[i] = ga;
    reinterpret_cast<f32x4*>(dU)[i] = gu;
  }
  const int64_t t = 4 * nv + blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (t < n) {
    float s, ds;
    act_eval_f32(act, A[t], s, ds);
    const float g = dA[t];
    dA[t] = g * U[t] * ds;
    dU[t] = g * s;
  }
}

// The plain MLP's activation when dH = gy W2^T ran beside fc1 (TP lesson,
// 2.A steps 2-3, and the multi-card page's 02 / BACKWARD rule G_Z = G_H *
// sigma'): H = sigma(P) and dZ = dH * sigma'(P), from the fp32 P and dH tiles
// of that launch, each rounded once to bf16.  VEC: 8 elements per thread
// (16-byte aligned bases), then a scalar tail of n % 8.
template <int ACT, bool VEC>
__global__ __launch_bounds__(256) void act_mul_kernel(const float* __restrict__ P, const float* __restrict__ dH,
                                                      uint16_t* __restrict__ H, uint16_t* __restrict__ dZ,
                                                      int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int64_t tid = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  const int64_t nv = VEC ? n / 8 : 0;
  for (int64_t i = tid; i < nv; i += stride) {
    const f32x4 p0 = reinterpret_cast<const f32x4*>(P)[2 * i], p1 = reinterpret_cast<const f32x4*>(P)[2 * i + 1];
    const f32x4 g0 = reinterpret_cast<const f32x4*>(dH)[2 * i], g1 = reinterpret_cast<const f32x4*>(dH)[2 * i + 1];
    const float p[8] = {p0[0], p0[1], p0[2], p0[3], p1[0], p1[1], p1[2], p1[3]};
    const float g[8] = {g0[0], g0[1], g0[2], g0[3], g1[0], g1[1], g1[2], g1[3]};
    float h[8], z[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      float sv, ds;
      act_fast<ACT>(p[k], sv, ds);
      h[k] = sv;
      z[k] = g[k] * ds;
    }
    reinterpret_cast<u32x4*>(H)[i] = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]), pack2(h[6], h[7])};
    reinterpret_cast<u32x4*>(dZ)[i] = u32x4{pack2(z[0], z[1]), pack2(z[2], z[3]), pack2(z[4], z[5]), pack2(z[6], z[7])};
  }
  for (int64_t t = 8 * nv + tid; t < n; t += stride) {
    float sv, ds;
    act_fast<ACT>(P[t], sv, ds);
    H[t] = to_bf(sv);
    dZ[t] = to_bf(dH[t] * ds);
  }
}

// dA / dU of a rows x cols block: dH and the outputs rows `ld` apart, A and
// U contiguous.  VEC: 8 bf16 per thread (cols % 8 == 0, 16-byte aligned).
template <typename T, bool VEC>
__global__ __launch_bounds__(256) void glu_bwd_2d_kernel(T* __restrict__ dA, const T* __restrict__ A,
                                                         const T* __restrict__ U, T* __restrict__ dU, int64_t rows,
                                                         int64_t cols, int64_t ld, int act) {
  const int64_t per_row = VEC ? cols / 8 : cols;
  const int64_t n = rows * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / per_row, c = (i - r * per_row) * (VEC ? 8 : 1);
    T* ga = dA + r * ld + c;
    T* gu = dU + r * ld + c;
    const T* a = A + r * cols + c;
    const T* u = U + r * cols + c;
    if constexpr (VEC) {
      const u32x4 g = *reinterpret_cast<const u32x4*>(ga);
      const u32x4 av = *reinterpret_cast<const u32x4*>(a);
      const u32x4 uv = *reinterpret_cast<const u32x4*>(u);
      u32x4 oa, ou;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        float s0, d0, s1, d1;
        act_eval(act, bf_lo(av[q]), s0, d0);
        act_eval(act, bf_hi(av[q]), s1, d1);
        const float g0 = bf_lo(g[q]), g1 = bf_hi(g[q]);
        oa[q] = pack2(g0 * bf_lo(uv[q]) * d0, g1 * bf_hi(uv[q]) * d1);
        ou[q] = pack2(g0 * s0, g1 * s1);
      }
      *reinterpret_cast<u32x4*>(ga) = oa;
      *reinterpret_cast<u32x4*>(gu) = ou;
    } else if constexpr (sizeof(T) == 2) {
      float sv, dv;
      act_eval(act, bf(*a), sv, dv);
      const float g = bf(*ga);
      *ga = to_bf(g * bf(*u) * dv);
      *gu = to_bf(g * sv);
    } else {
      float sv, dv;
      act_eval_f32(act, *a, sv, dv);
      const float g = *ga;
      *ga = g * *u * dv;
      *gu = g * sv;
    }
  }
}

// rows x row_bytes, 16 bytes (VEC) or 2 bytes per thread and iteration.
template <bool VEC>
__global__ __launch_bounds__(256) void copy_2d_kernel(char* __restrict__ dst, int64_t ld_dst,
                                                      const char* __restrict__ src, int64_t ld_src, int64_t rows,
                                                      int64_t row_bytes) {
  constexpr int W = VEC ? 16 : 2;
  const int64_t per_row = row_bytes / W;
  const int64_t n = rows * per_row;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    const int64_t r = i / per_row, c = (i - r * per_row) * W;
    if constexpr (VEC)
      *reinterpret_cast<u32x4*>(dst + r * ld_dst + c) = *reinterpret_cast<const u32x4*>(src + r * ld_src + c);
    else
      *reinterpret_cast<uint16_t*>(dst + r * ld_dst + c) = *reinterpret_cast<const uint16_t*>(src + r * ld_src + c);
  }
}

unsigned grid_for(int64_t nvec) {
  const int64_t b = (nvec + 255) / 256;
  return (unsigned)(b < 1 ? 1 : (b > 4096 ? 4096 : b));
}

}  // namespace

// Buffers are 16-byte aligned and hold n contiguous elements of `dtype`.
hipError_t launch_glu_fwd(int dtype, const void* A, const void* U, void* H, int64_t n, int act, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(glu_fwd_bf16, dim3(grid_for(n / 8)), dim3(256), 0, s, static_cast<const uint16_t*>(A),
                       static_cast<const uint16_t*>(U), static_cast<uint16_t*>(H), n, act);
  else
    hipLaunchKernelGGL(glu_fwd_f32, dim3(grid_for(n / 4)), dim3(256), 0, s, static_cast<const float*>(A),
                       static_cast<const float*>(U), static_cast<float*>(H), n, act);
  return hipGetLastError();
}

hipError_t launch_glu_bwd(int dtype, void* dA, const void* A, const void* U, void* dU, int64_t n, int act,
                          hipStream_t s) {
  if (n <= 0) return hipSuccess;
  if (dtype == 1)
    hipLaunchKernelGGL(glu_bwd_bf16, dim3(grid_for(n / 8)), dim3(256), 0, s, static_cast<uint16_t*>(dA),
                       static_cast<const uint16_t*>(A), static_cast<const uint16_t*>(U), static_cast<uint16_t*>(dU),
                       n, act);
  else
    hipLaunchKernelGGL(glu_bwd_f32, dim3(grid_for(n / 4)), dim3(256), 0, s, static_cast<float*>(dA),
                       static_cast<const float*>(A), static_cast<const float*>(U), static_cast<float*>(dU), n, act);
  return hipGetLastError();
}

hipError_t launch_glu_bwd_2d(int dtype, void* dA, const void* A, const void* U, void* dU, int64_t rows, int64_t cols,
                             int64_t ld, int act, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (dtype == 1) {
    const bool vec = cols % 8 == 0 && ld % 8 == 0 && reinterpret_cast<uintptr_t>(dA) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(A) % 16 == 0 && reinterpret_cast<uintptr_t>(U) % 16 == 0 &&
                     reinterpret_cast<uintptr_t>(dU) % 16 == 0;
    uint16_t *ga = static_cast<uint16_t*>(dA), *gu = static_cast<uint16_t*>(dU);
    const uint16_t *a = static_cast<const uint16_t*>(A), *u = static_cast<const uint16_t*>(U);
    if (vec)
      hipLaunchKernelGGL((glu_bwd_2d_kernel<uint16_t, true>), dim3(grid_for(rows * cols / 8)), dim3(256), 0, s, ga, a,
                         u, gu, rows, cols, ld, act);
    else
      hipLaunchKernelGGL((glu_bwd_2d_kernel<uint16_t, false>), dim3(grid_for(rows * cols)), dim3(256), 0, s, ga, a, u,
                         gu, rows, cols, ld, act);
  } else {
    hipLaunchKernelGGL((glu_bwd_2d_kernel<float, false>), dim3(grid_for(rows * cols)), dim3(256), 0, s,
                       static_cast<float*>(dA), static_cast<const float*>(A), static_cast<const float*>(U),
                       static_cast<float*>(dU), rows, cols, ld, act);
  }
  return hipGetLastError();
}

hipError_t launch_copy_2d(void* dst, int64_t ld_dst, const void* src, int64_t ld_src, int64_t rows, int64_t row_bytes,
                          hipStream_t s) {
  if (rows <= 0 || row_bytes <= 0) return hipSuccess;
  const bool vec = row_bytes % 16 == 0 && ld_dst % 16 == 0 && ld_src % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(dst) % 16 == 0 && reinterpret_cast<uintptr_t>(src) % 16 == 0;
  if (vec)
    hipLaunchKernelGGL(copy_2d_kernel<true>, dim3(grid_for(rows * row_bytes / 16)), dim3(256), 0, s,
                       static_cast<char*>(dst), ld_dst, static_cast<const char*>(src), ld_src, rows, row_bytes);
  else
    hipLaunchKernelGGL(copy_2d_kernel<false>, dim3(grid_for(rows * row_bytes / 2)), dim3(256), 0, s,
                       static_cast<char*>(dst), ld_dst, static_cast<const char*>(src), ld_src, rows, row_bytes);
  return hipGetLastError();
}

hipError_t launch_act_mul(const float* P, const float* dH, void* H, void* dZ, int64_t n, int act, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const bool vec = reinterpret_cast<uintptr_t>(P) % 16 == 0 && reinterpret_cast<uintptr_t>(dH) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(H) % 16 == 0 && reinterpret_cast<uintptr_t>(dZ) % 16 == 0;
  uint16_t* h = static_cast<uint16_t*>(H);
  uint16_t* z = static_cast<uint16_t*>(dZ);
  const dim3 grid(grid_for(vec ? n / 8 : n)), block(256);
  if (act == ACT_TANH) {
    if (vec) hipLaunchKernelGGL((act_mul_kernel<ACT_TANH, true>), grid, block, 0, s, P, dH, h, z, n);
    else hipLaunchKernelGGL((act_mul_kernel<ACT_TANH, false>), grid, block, 0, s, P, dH, h, z, n);
  } else if (act == ACT_SILU) {
    if (vec) hipLaunchKernelGGL((act_mul_kernel<ACT_SILU, true>), grid, block, 0, s, P, dH, h, z, n);
    else hipLaunchKernelGGL((act_mul_kernel<ACT_SILU, false>), grid, block, 0, s, P, dH, h, z, n);
  } else {
    if (vec) hipLaunchKernelGGL((act_mul_kernel<ACT_GELU, true>), grid, block, 0, s, P, dH, h, z, n);
    else hipLaunchKernelGGL((act_mul_kernel<ACT_GELU, false>), grid, block, 0, s, P, dH, h, z, n);
  }
  return hipGetLastError();
}

}  // namespace tpr
