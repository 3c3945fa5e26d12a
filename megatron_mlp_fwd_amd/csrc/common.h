// Internal declarations shared by the libtprank sources (not part of the ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

namespace tpr {

// ---------------------------------------------------------------- GEMM
// One GEMM problem C(m, n) = sum_k A(m, k) B(k, n) with
//   A(m, k) = A[m * sa_m + k * sa_k],  B(k, n) = B[k * sb_k + n * sb_n],
//   C(m, n) = C[m * ldc + n]   (aux_in / aux_out use the same ldc).
// Either sa_k == 1 (A "k-major") or sa_m == 1 (A "m-major"); likewise B is
// k-major (sb_k == 1) or n-major (sb_n == 1).  The launcher picks the kernel
// instance from the layout flags, never from the strides alone.
struct GemmProb {
  const void* A;
  const void* B;
  void* C;
  const void* aux_in;   // epilogue input (sigma'(pre-activation) for EPI_MUL)
  void* aux_out;        // epilogue second output (the activation for EPI_ACT)
  int64_t sa_m, sa_k, sb_k, sb_n, ldc;
  int M, N, K;
  int kind;              // gemm_kind(a_kmajor, b_kmajor, epilogue) for heterogeneous launches
  int act;               // activation of EPI_ACT (ACT_GELU / ACT_TANH / ACT_SILU)
  int tiles_m, tiles_n;  // filled by the launcher
  int tile_start;        // first flattened block index of this problem
};

constexpr int kMaxGroup = 16;  // problems per grouped launch

struct GemmBatch {
  GemmProb p[kMaxGroup];
  int count;
  int total_tiles;
  int nxcd;  // XCDs of the device: workgroup i runs on XCD i mod nxcd (set by the launcher)
};

// Compute units and XCDs of the calling thread's current device, read from
// the runtime once per device.  When no device answers (a workspace query on
// a host without a GPU) the counts of a whole MI355X, (256, 8), stand in.
struct Topology {
  int cus, xcds;
};
Topology device_topology();

enum Epilogue {
  EPI_F32 = 0,    // C (fp32) = acc
  EPI_ACT = 1,   // C (compute dtype) = sigma'(acc), aux_out = sigma(acc)  [acc = pre-activation]
  EPI_MUL = 2,   // C (compute dtype) = acc * aux_in                       [in place allowed]
  EPI_BF16 = 3,   // C (bf16) = acc, rounded to nearest even
};

// Element-wise activations (same values as TPR_ACT_* in tprank.h).
enum Activation { ACT_GELU = 0, ACT_TANH = 1, ACT_SILU = 2 };

constexpr int gemm_kind(bool a_kmajor, bool b_kmajor, int epi) {
  return (a_kmajor ? 1 : 0) | (b_kmajor ? 2 : 0) | (epi << 2);
}

// Register-staged bf16 kernel (gemm_bf16.hip): a group of problems sharing
// layout and epilogue, any shape or alignment.  Launchers return hipSuccess
// or the launch error.
hipError_t launch_gemm_bf16(GemmBatch& b, bool a_kmajor, bool b_kmajor, int epi, hipStream_t s);
// Direct-to-LDS bf16 kernel (gemm_bf16_dma.hip): a group of independent
// problems that may differ in layout and epilogue (GemmProb::kind), each of
// them eligible.  Problems should be ordered by decreasing K so the longest
// tiles are dispatched first.
bool gemm_bf16_dma_eligible(const GemmProb& p, bool a_kmajor, bool b_kmajor, int epi);
hipError_t launch_gemm_bf16_dma(GemmBatch& b, hipStream_t s);
hipError_t launch_gemm_f32(GemmBatch& b, bool a_kmajor, bool b_kmajor, int epi, hipStream_t s);

// ---------------------------------------------------------------- reductions
// out[i] = sum_{s < nslots} part[s * stride + i], summed in slot order.
hipError_t launch_reduce_partials(const float* part, int nslots, int64_t stride, float* out, int64_t n,
                                  hipStream_t s);
hipError_t launch_fill_zero(float* out, int64_t rows, int64_t cols, int64_t ld, hipStream_t s);

// Gated MLP element-wise steps over n contiguous elements of `dtype`
// (TPR_F32 / TPR_BF16), 16-byte aligned: H = sigma(A) U, and
// dA = dH U sigma'(A), dU = dH sigma(A) with dA holding dH on entry.
hipError_t launch_glu_fwd(int dtype, const void* A, const void* U, void* H, int64_t n, int act, hipStream_t s);
hipError_t launch_glu_bwd(int dtype, void* dA, const void* A, const void* U, void* dU, int64_t n, int act,
                          hipStream_t s);
// The same backward over a rows x cols block whose dH / dA and dU rows are
// `ld` elements apart (A and U are contiguous rows of cols).
hipError_t launch_glu_bwd_2d(int dtype, void* dA, const void* A, const void* U, void* dU, int64_t rows, int64_t cols,
                             int64_t ld, int act, hipStream_t s);
// Copy rows x row_bytes from src (rows ld_src bytes apart) to dst (ld_dst).
hipError_t launch_copy_2d(void* dst, int64_t ld_dst, const void* src, int64_t ld_src, int64_t rows, int64_t row_bytes,
                          hipStream_t s);
// H = sigma(P) and dZ = dH * sigma'(P) over n contiguous elements (act is
// an Activation): P and dH fp32, H and dZ bf16, each rounded once.
hipError_t launch_act_mul(const float* P, const float* dH, void* H, void* dZ, int64_t n, int act, hipStream_t s);

// ---------------------------------------------------------------- vocab CE
struct CeArgs {
  const void* logits;
  const int64_t* labels;
  void* dlogits;
  float* shard_stats;  // nullable, T x parts x 3
  float* row_loss;     // workspace, T floats
  float* loss;         // device scalar
  int64_t T, V;
  int parts;
  int dtype;  // TPR_F32 / TPR_BF16
  // Options (used when `opt` is set): columns >= v_valid are vocabulary
  // padding; rows whose label equals ignore_index add no loss and get a zero
  // gradient, and the mean is over the counted rows; label smoothing eps.
  bool opt;
  int64_t v_valid;
  int64_t ignore_index;
  float smoothing;
  int* count;        // workspace: counted rows (opt)
  float* inv_count;  // workspace: 1 / counted rows, 0 if none (opt)
};
hipError_t launch_vocab_ce(const CeArgs& a, hipStream_t s);

// Rows of the CE's static per-row-loss array (1 MiB of fp32 per device), and
// its device address on the current device (looked up on the first call per
// device, then cached).
constexpr int64_t kCeStaticRows = int64_t(1) << 18;
hipError_t ce_static_scratch(float** rows);

}  // namespace tpr
