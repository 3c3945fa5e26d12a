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
// them from displacing cached data.  Every load of a group of up to kGroup
// slots is issued before the first add, so a thread keeps kGroup 16-byte
// loads in flight instead of one; the adds still run in slot order, so the
// result does not depend on the grouping.
constexpr int kGroup = 8;

template <int NS>
__global__ __launch_bounds__(256) void reduce_vec4_kernel(const floatx4* __restrict__ part, int nslots,
                                                          int64_t stride4, floatx4* __restrict__ out, int64_t n4) {
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += step) {
    floatx4 s;
    if constexpr (NS > 0) {  // exactly NS slots
      floatx4 v[NS];
#pragma unroll
      for (int r = 0; r < NS; ++r) v[r] = __builtin_nontemporal_load(part + r * stride4 + i);
      s = v[0];
#pragma unroll
      for (int r = 1; r < NS; ++r) s += v[r];
    } else {  // any count, kGroup slots at a time
      s = __builtin_nontemporal_load(part + i);
      for (int r0 = 1; r0 < nslots; r0 += kGroup) {
        floatx4 v[kGroup];
#pragma unroll
        for (int r = 0; r < kGroup; ++r)
          if (r0 + r < nslots) v[r] = __builtin_nontemporal_load(part + (r0 + r) * stride4 + i);
#pragma unroll
        for (int r = 0; r < kGroup; ++r)
          if (r0 + r < nslots) s += v[r];
      }
    }
    __builtin_nontemporal_store(s, out + i);
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
    const dim3 grid(grid_for(n4)), block(256);
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
