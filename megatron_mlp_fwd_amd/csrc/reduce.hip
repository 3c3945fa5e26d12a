// Cross-rank partial-sum reduction: the simulated all-reduce(sum) of every
// output that a split leaves as per-rank partials.  Sharded GEMM page
// ("Sharded GEMM与Backprop：行、列、内维三种切分", 解题路线 steps 2-4): dB for a
// row split, dA for a column split, Y for an inner split; TP lesson
// ("第 6 课：张量并行 TP", 2.A step 5) and the multi-card page's
// 02 / BACKWARD: the MLP output and the input gradient.
//
// out[i] = part[0][i] + part[1][i] + ... in slot order (deterministic), one
// HBM pass: each element is read once per partial and written once, with
// 16-byte loads and stores when the layout allows.  HBM-bound: per output
// element (nslots + 1) * 4 bytes move.
#include "common.h"

namespace tpr {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

// Partials are read once and the sum written once: non-temporal accesses keep
// them from displacing cached data.  Each thread sums kUnroll vectors that
// lie a block apart, and issues every load of a group of up to kGroup slots
// for all of them before the first add, so it keeps up to kUnroll * kGroup
// 16-byte loads in flight (measured on the 8 x 8192 x 8192 partials: 5.0 TB/s
// with one vector and one load per slot in flight per thread, 5.6 TB/s with
// two vectors, 5.9-6.0 TB/s with four, one pass over a grid of 16384 blocks).
// The adds still run in slot order, so the result does not depend on the
// grouping.
constexpr int kGroup = 8;
constexpr int kUnroll = 4;

template <int NS>
__global__ __launch_bounds__(256) void reduce_vec4_kernel(const floatx4* __restrict__ part, int nslots,
                                                          int64_t stride4, floatx4* __restrict__ out, int64_t n4) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x * kUnroll;
  for (int64_t i0 = (int64_t)blockIdx.x * blockDim.x * kUnroll + threadIdx.x; i0 < n4; i0 += step) {
    floatx4 s[kUnroll];
    constexpr int G = NS > 0 ? NS : kGroup;  // slots per group of loads
    const int ns = NS > 0 ? NS : nslots;
    for (int r0 = 0; r0 < ns; r0 += G) {
      floatx4 v[kUnroll][G];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t i = i0 + (int64_t)u * blockDim.x;
#pragma unroll
        for (int r = 0; r < G; ++r)
          if (i < n4 && (NS > 0 || r0 + r < ns)) v[u][r] = __builtin_nontemporal_load(part + (r0 + r) * stride4 + i);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u)
#pragma unroll
        for (int r = 0; r < G; ++r)
          if (NS > 0 || r0 + r < ns) s[u] = (r0 + r == 0) ? v[u][r] : s[u] + v[u][r];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t i = i0 + (int64_t)u * blockDim.x;
      if (i < n4) __builtin_nontemporal_store(s[u], out + i);
    }
  }
}

__global__ __launch_bounds__(256) void reduce_scalar_kernel(const float* __restrict__ part, int nslots,
                                                            int64_t stride, float* __restrict__ out, int64_t n) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step) {
    float s = part[i];
    for (int r = 1; r < nslots; ++r) s += part[r * stride + i];
    out[i] = s;
  }
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ out, int64_t rows, int64_t cols,
                                                        int64_t ld) {
  const int64_t n = rows * cols, step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += step)
    out[(i / cols) * ld + (i % cols)] = 0.f;
}

int grid_for(int64_t work) {
  const int64_t blocks = (work + 255) / 256;
  return (int)(blocks < 4096 ? (blocks > 0 ? blocks : 1) : 4096);
}

}  // namespace

hipError_t launch_reduce_partials(const float* part, int nslots, int64_t stride, float* out, int64_t n,
                                  hipStream_t s) {
  if (n <= 0 || nslots <= 0) return hipSuccess;
  const bool vec = n % 4 == 0 && stride % 4 == 0 && reinterpret_cast<uintptr_t>(part) % 16 == 0 &&
                   reinterpret_cast<uintptr_t>(out) % 16 == 0;
  if (vec) {
    const floatx4* p4 = reinterpret_cast<const floatx4*>(part);
    floatx4* o4 = reinterpret_cast<floatx4*>(out);
    const int64_t n4 = n / 4, s4 = stride / 4;
    const int64_t blocks = (n4 + 256 * kUnroll - 1) / (256 * kUnroll);
    const dim3 grid((unsigned)(blocks < 16384 ? blocks : 16384)), block(256);
    switch (nslots) {
      case 1: hipLaunchKernelGGL(reduce_vec4_kernel<1>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 2: hipLaunchKernelGGL(reduce_vec4_kernel<2>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 3: hipLaunchKernelGGL(reduce_vec4_kernel<3>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 4: hipLaunchKernelGGL(reduce_vec4_kernel<4>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 5: hipLaunchKernelGGL(reduce_vec4_kernel<5>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 6: hipLaunchKernelGGL(reduce_vec4_kernel<6>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 7: hipLaunchKernelGGL(reduce_vec4_kernel<7>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      case 8: hipLaunchKernelGGL(reduce_vec4_kernel<8>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
      default: hipLaunchKernelGGL(reduce_vec4_kernel<0>, grid, block, 0, s, p4, nslots, s4, o4, n4); break;
    }
  } else {
    hipLaunchKernelGGL(reduce_scalar_kernel, dim3(grid_for(n)), dim3(256), 0, s, part, nslots, stride, out, n);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(float* out, int64_t rows, int64_t cols, int64_t ld, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(rows * cols)), dim3(256), 0, s, out, rows, cols, ld);
  return hipGetLastError();
}

}  // namespace tpr
