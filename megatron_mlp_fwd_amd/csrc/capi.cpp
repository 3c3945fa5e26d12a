// C ABI of libtprank (declared in include/tprank.h): argument validation,
// shard planning, workspace carving and the launch sequence of each entry
// point.  All validation happens before the first launch, so an error leaves
// every output untouched.  Nothing here allocates device memory.
#include <algorithm>
#include <climits>
#include <cstdlib>
#include <cstring>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>
#include <vector>

#include "common.h"
#include "tprank.h"

namespace tpr {

Topology device_topology() {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static Topology known[kMaxDev];
  static bool have[kMaxDev];
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) {
    (void)hipGetLastError();
    return Topology{256, 8};
  }
  std::lock_guard<std::mutex> lock(mu);
  if (!have[dev]) {
    int cus = 0, xcds = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
    if (hipDeviceGetAttribute(&xcds, hipDeviceAttributeNumberOfXccs, dev) != hipSuccess || xcds <= 0) xcds = 1;
    (void)hipGetLastError();
    known[dev] = Topology{cus, xcds};
    have[dev] = true;
  }
  return known[dev];
}

}  // namespace tpr

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(TPR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
int64_t esize(int dtype) { return dtype == TPR_BF16 ? 2 : 4; }
bool dtype_ok(int dtype) { return dtype == TPR_F32 || dtype == TPR_BF16; }
bool dim_ok(int64_t n) { return n >= 0 && n <= INT_MAX; }

// Shard rule of the sharded GEMM page (题意与假设 / 手动走一遍): floor(n/P)
// indices each, one more for the first n mod P shards.
void shard_of(int64_t n, int parts, int r, int64_t* lo, int64_t* hi) {
  const int64_t base = n / parts, extra = n % parts;
  *lo = r * base + (r < extra ? r : extra);
  *hi = *lo + base + (r < extra ? 1 : 0);
}

const char* cb(const void* p) { return static_cast<const char*>(p); }

tpr::GemmProb prob(const void* A, int64_t sa_m, int64_t sa_k, const void* B, int64_t sb_k, int64_t sb_n, void* C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, const void* aux_in = nullptr,
                   void* aux_out = nullptr) {
  tpr::GemmProb p{};
  p.A = A;
  p.B = B;
  p.C = C;
  p.aux_in = aux_in;
  p.aux_out = aux_out;
  p.sa_m = sa_m;
  p.sa_k = sa_k;
  p.sb_k = sb_k;
  p.sb_n = sb_n;
  p.ldc = ldc;
  p.M = (int)M;
  p.N = (int)N;
  p.K = (int)K;
  return p;
}

// A GEMM to run: the problem plus its operand layouts and epilogue.
struct Job {
  tpr::GemmProb p;
  bool ak, bk;
  int epi;
};

Job job(const tpr::GemmProb& p, bool ak, bool bk, int epi) { return Job{p, ak, bk, epi}; }

// Run a set of mutually independent GEMMs.  bf16 problems the direct-to-LDS
// kernel accepts share heterogeneous launches (longest K first, so the
// longest tiles are dispatched first and short ones fill in behind them);
// everything else runs through the register-staged (bf16) or fp32 kernel,
// grouped by layout and epilogue.  TPRANK_GEMM_PATH=staged sends every bf16
// problem to the register-staged kernel (tests use it to cover that kernel).
hipError_t run_jobs(std::vector<Job> jobs, int dtype, hipStream_t s) {
  std::vector<Job> fast, rest;
  const char* path = getenv("TPRANK_GEMM_PATH");
  const bool staged_only = path != nullptr && strcmp(path, "staged") == 0;
  for (const Job& j : jobs) {
    if (j.p.M <= 0 || j.p.N <= 0) continue;
    const bool dma = dtype == TPR_BF16 && !staged_only && tpr::gemm_bf16_dma_eligible(j.p, j.ak, j.bk, j.epi);
    (dma ? fast : rest).push_back(j);
  }
  std::stable_sort(fast.begin(), fast.end(), [](const Job& x, const Job& y) { return x.p.K > y.p.K; });
  for (size_t i = 0; i < fast.size(); i += tpr::kMaxGroup) {
    tpr::GemmBatch b{};
    b.count = (int)std::min<size_t>(tpr::kMaxGroup, fast.size() - i);
    for (int k = 0; k < b.count; ++k) {
      const Job& j = fast[i + k];
      b.p[k] = j.p;
      b.p[k].kind = tpr::gemm_kind(j.ak, j.bk, j.epi);
    }
    const hipError_t e = tpr::launch_gemm_bf16_dma(b, s);
    if (e != hipSuccess) return e;
  }
  while (!rest.empty()) {
    const Job head = rest.front();
    std::vector<Job> same, other;
    for (const Job& j : rest)
      (j.ak == head.ak && j.bk == head.bk && j.epi == head.epi ? same : other).push_back(j);
    for (size_t i = 0; i < same.size(); i += tpr::kMaxGroup) {
      tpr::GemmBatch b{};
      b.count = (int)std::min<size_t>(tpr::kMaxGroup, same.size() - i);
      for (int k = 0; k < b.count; ++k) b.p[k] = same[i + k].p;
      const hipError_t e = dtype == TPR_BF16 ? tpr::launch_gemm_bf16(b, head.ak, head.bk, head.epi, s)
                                             : tpr::launch_gemm_f32(b, head.ak, head.bk, head.epi, s);
      if (e != hipSuccess) return e;
    }
    rest.swap(other);
  }
  return hipSuccess;
}

// Finish an output that the split sums: reduce the partials in slot order,
// or zero it when no rank contributed (empty contraction).
hipError_t finish_sum(float* out, int64_t rows, int64_t cols, const float* slots, int nslots, int64_t stride,
                      bool direct, hipStream_t s) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (nslots == 0) return tpr::launch_fill_zero(out, rows, cols, cols, s);
  if (direct) return hipSuccess;
  return tpr::launch_reduce_partials(slots, nslots, stride, out, rows * cols, s);
}

}  // namespace

extern "C" {

const char* tprank_last_error(void) { return g_err.c_str(); }

int tprank_shard_range(int64_t n, int parts, int rank, int64_t* begin, int64_t* end) {
  if (begin == nullptr || end == nullptr) return fail(TPR_ERR_NULLPTR, "begin/end must not be NULL");
  if (n < 0) return fail(TPR_ERR_SHAPE, "n must be >= 0 (got %lld)", (long long)n);
  if (parts < 1) return fail(TPR_ERR_PARTITION, "parts must be >= 1 (got %d)", parts);
  if (rank < 0 || rank >= parts) return fail(TPR_ERR_PARTITION, "rank %d outside [0, %d)", rank, parts);
  shard_of(n, parts, rank, begin, end);
  return TPR_OK;
}

// ---------------------------------------------------------------- sharded GEMM
size_t sharded_matmul_workspace_bytes(int axis, int parts, int dtype, int64_t M, int64_t K, int64_t N) {
  if (parts < 1 || axis < TPR_ROWS || axis > TPR_INNER || !dtype_ok(dtype) || M < 0 || K < 0 || N < 0) return 0;
  if (parts == 1) return 0;
  const int64_t sz = axis == TPR_ROWS ? K * N : axis == TPR_COLUMNS ? M * K : M * N;
  return (size_t)parts * align256((size_t)sz * 4);
}

int sharded_matmul_fwd_bwd(int axis, int parts, int dtype, int64_t M, int64_t K, int64_t N, const void* A,
                           const void* B, const void* G, float* Y, float* dA, float* dB, void* ws, size_t ws_bytes,
                           void* stream) {
  if (!dim_ok(M) || !dim_ok(K) || !dim_ok(N))
    return fail(TPR_ERR_SHAPE, "M, K, N must be in [0, 2^31) (got %lld, %lld, %lld)", (long long)M, (long long)K,
                (long long)N);
  if (parts < 1) return fail(TPR_ERR_PARTITION, "parts must be >= 1 (got %d)", parts);
  if (axis < TPR_ROWS || axis > TPR_INNER) return fail(TPR_ERR_PARTITION, "unknown axis %d", axis);
  if (!dtype_ok(dtype)) return fail(TPR_ERR_DTYPE, "unknown dtype %d", dtype);
  if ((M * K > 0 && (A == nullptr || dA == nullptr)) || (K * N > 0 && (B == nullptr || dB == nullptr)) ||
      (M * N > 0 && (G == nullptr || Y == nullptr)))
    return fail(TPR_ERR_NULLPTR, "a non-empty input or output pointer is NULL");
  const size_t need = sharded_matmul_workspace_bytes(axis, parts, dtype, M, K, N);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(TPR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t e = esize(dtype);
  const int64_t sum_n = axis == TPR_ROWS ? K * N : axis == TPR_COLUMNS ? M * K : M * N;
  const int64_t stride = (int64_t)(align256((size_t)sum_n * 4) / 4);
  float* slots = static_cast<float*>(ws);
  const bool direct = parts == 1;
  int nslots = 0;
  std::vector<Job> jobs;  // Y (NN), dA (NT) and dB (TN) of every rank are independent

  for (int r = 0; r < parts; ++r) {
    int64_t lo, hi;
    if (axis == TPR_ROWS) {
      shard_of(M, parts, r, &lo, &hi);
      const int64_t m = hi - lo;
      if (m == 0) continue;
      // Y_r = A_r B and dA_r = G_r B^T land in their row slices; dB_r = A_r^T G_r is a partial.
      jobs.push_back(job(prob(cb(A) + lo * K * e, K, 1, B, N, 1, Y + lo * N, N, m, N, K), true, false, tpr::EPI_F32));
      jobs.push_back(job(prob(cb(G) + lo * N * e, N, 1, B, 1, N, dA + lo * K, K, m, K, N), true, true, tpr::EPI_F32));
      float* dst = direct ? dB : slots + nslots * stride;
      jobs.push_back(job(prob(cb(A) + lo * K * e, 1, K, cb(G) + lo * N * e, N, 1, dst, N, K, N, m), false, false, tpr::EPI_F32));
      ++nslots;
    } else if (axis == TPR_COLUMNS) {
      shard_of(N, parts, r, &lo, &hi);
      const int64_t n = hi - lo;
      if (n == 0) continue;
      // Y_r = A B_r and dB_r = A^T G_r land in their column slices; dA_r = G_r B_r^T is a partial.
      jobs.push_back(job(prob(A, K, 1, cb(B) + lo * e, N, 1, Y + lo, N, M, n, K), true, false, tpr::EPI_F32));
      jobs.push_back(job(prob(A, 1, K, cb(G) + lo * e, N, 1, dB + lo, N, K, n, M), false, false, tpr::EPI_F32));
      float* dst = direct ? dA : slots + nslots * stride;
      jobs.push_back(job(prob(cb(G) + lo * e, N, 1, cb(B) + lo * e, 1, N, dst, K, M, K, n), true, true, tpr::EPI_F32));
      ++nslots;
    } else {
      shard_of(K, parts, r, &lo, &hi);
      const int64_t k = hi - lo;
      if (k == 0) continue;
      // Y_r = A_r B_r is a partial; dA_r = G B_r^T and dB_r = A_r^T G land in their K slices.
      float* dst = direct ? Y : slots + nslots * stride;
      jobs.push_back(job(prob(cb(A) + lo * e, K, 1, cb(B) + lo * N * e, N, 1, dst, N, M, N, k), true, false, tpr::EPI_F32));
      jobs.push_back(job(prob(G, N, 1, cb(B) + lo * N * e, 1, N, dA + lo, K, M, k, N), true, true, tpr::EPI_F32));
      jobs.push_back(job(prob(cb(A) + lo * e, 1, K, G, N, 1, dB + lo * N, N, k, N, M), false, false, tpr::EPI_F32));
      ++nslots;
    }
  }

  hipError_t he;
  if ((he = run_jobs(jobs, dtype, s)) != hipSuccess) return hip_fail(he, "sharded GEMM launch");
  if (axis == TPR_ROWS)
    he = finish_sum(dB, K, N, slots, nslots, stride, direct, s);
  else if (axis == TPR_COLUMNS)
    he = finish_sum(dA, M, K, slots, nslots, stride, direct, s);
  else
    he = finish_sum(Y, M, N, slots, nslots, stride, direct, s);
  if (he != hipSuccess) return hip_fail(he, "partial-sum reduction");
  return TPR_OK;
}

// ---------------------------------------------------------------- partial sum
int tprank_partial_sum(int nslots, int64_t n, const float* partials, int64_t slot_stride, float* out,
                       void* stream) {
  if (n < 0 || nslots < 0 || slot_stride < n)
    return fail(TPR_ERR_SHAPE, "need n >= 0, nslots >= 0 and slot_stride >= n (got %lld, %d, %lld)", (long long)n,
                nslots, (long long)slot_stride);
  if (n == 0) return TPR_OK;
  if (out == nullptr || (nslots > 0 && partials == nullptr))
    return fail(TPR_ERR_NULLPTR, "out or partials is NULL");
  if (nslots > 0) {
    const uintptr_t o0 = reinterpret_cast<uintptr_t>(out), o1 = o0 + (uintptr_t)n * 4;
    const uintptr_t p0 = reinterpret_cast<uintptr_t>(partials),
                    p1 = p0 + ((uintptr_t)(nslots - 1) * (uintptr_t)slot_stride + (uintptr_t)n) * 4;
    if (o0 < p1 && p0 < o1) return fail(TPR_ERR_VALUE, "out overlaps the partials");
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const hipError_t he = nslots == 0 ? tpr::launch_fill_zero(out, 1, n, n, s)
                                    : tpr::launch_reduce_partials(partials, nslots, slot_stride, out, n, s);
  if (he != hipSuccess) return hip_fail(he, "partial-sum reduction");
  return TPR_OK;
}

// ---------------------------------------------------------------- TP MLP
namespace {

constexpr int kTile = 256;   // block tile of the bf16 GEMM

// Whether dH = gy W2^T joins the fc1 launch of the plain bf16 MLP.  fc1
// fills sum_r ceil(T/256) ceil(f_r/256) tiles of K = d; when its last round
// leaves enough compute units idle for every dH tile (same K), dH runs there
// instead of in the next launch.  fc1 then writes P in fp32 and one
// element-wise pass forms H = sigma(P) and dZ = dH * sigma'(P) from the two
// fp32 tiles, so no activation epilogue sits on the launch's critical path.
// Moving only some leading row blocks of dH measured no gain (the fc1 launch
// grew by what the next one lost, plus the separate multiply), so it is all
// of dH or none.
bool cosched_dh(int dtype, int tp, int64_t T, int64_t f) {
  if (dtype != TPR_BF16 || T <= 0) return false;
  const int64_t tiles_m = (T + kTile - 1) / kTile;
  int64_t n1 = 0, nb = 0;
  for (int r = 0; r < tp; ++r) {
    int64_t lo, hi;
    shard_of(f, tp, r, &lo, &hi);
    const int64_t tn = (hi - lo + kTile - 1) / kTile;
    n1 += tiles_m * tn;
    nb += tn;
  }
  if (nb == 0) return false;
  const int64_t cus = tpr::device_topology().cus;
  const int64_t free = (cus - n1 % cus) % cus;
  return (free / nb) * kTile >= T;
}

size_t mlp_workspace(int tp, int dtype, bool gated, int64_t T, int64_t d, int64_t f) {
  if (tp < 1 || !dtype_ok(dtype) || T < 0 || d < 0 || f < 0) return 0;
  const size_t tf = align256((size_t)(T * f * esize(dtype))), td = align256((size_t)(T * d * 4));
  if (!gated)  // sigma'(P) / dZ, H, partials; with dH beside fc1, fp32 dH and fp32 P
    return 2 * tf + (tp > 1 ? 2 * (size_t)tp * td : 0) +
           (cosched_dh(dtype, tp, T, f) ? 2 * align256((size_t)(T * f * 4)) : 0);
  // gate, up, H; [dA | dU] per rank (dH first); [W1_r | W3_r] per rank; y and dx partials when tp > 1
  return 5 * tf + align256((size_t)(d * 2 * f * esize(dtype))) + (tp > 1 ? 2 * (size_t)tp * td : 0);
}

int check_act(int act) {
  if (act != TPR_ACT_GELU && act != TPR_ACT_TANH && act != TPR_ACT_SILU)
    return fail(TPR_ERR_VALUE, "unknown activation %d", act);
  return TPR_OK;
}

// Plain MLP: fc1's epilogue writes H = sigma(P) and sigma'(P) from the fp32
// accumulator; then fc2 (row-parallel) with the two backward products that
// need only H and gy: dW2 and dZ = (gy W2^T) * sigma'(P) (in place over
// sigma'(P)); then dW1 and dx.  When dH joins the fc1 launch (cosched_dh),
// fc1 and dH write fp32 P and dH, one element-wise pass forms H and dZ, and
// fc2, dW2, dW1 and dx share the next launch: with dZ complete none of them
// reads what another writes, and the short fc2 / dx tiles fill in behind the
// long dW2 / dW1 tiles instead of leaving two partly empty rounds.
int mlp_plain(int tp, int dtype, bool math, int act, int64_t T, int64_t d, int64_t f, const void* x, const void* w1,
              const void* w2, const void* gy, float* y, float* dx, float* dw1, float* dw2, void* ws, hipStream_t s) {
  const int64_t e = esize(dtype);
  char* wsb = static_cast<char*>(ws);
  char* pre = wsb;                                  // T x f sigma'(pre-activation), then dZ in place
  char* actv = wsb + align256((size_t)(T * f * e));  // T x f activation
  const int64_t pstride = (int64_t)(align256((size_t)(T * d * 4)) / 4);
  float* zpart = reinterpret_cast<float*>(wsb + 2 * align256((size_t)(T * f * e)));
  float* xpart = zpart + (int64_t)tp * pstride;
  const bool co = cosched_dh(dtype, tp, T, f);
  // With dH beside fc1: T x f fp32 dH, then T x f fp32 P (rank blocks T x f_r).
  float* dh32 = reinterpret_cast<float*>(wsb + 2 * align256((size_t)(T * f * e)) +
                                         (tp > 1 ? 2 * (size_t)tp * align256((size_t)(T * d * 4)) : 0));
  float* p32 = dh32 + align256((size_t)(T * f * 4)) / 4;
  const bool direct = tp == 1;
  int nslots = 0;
  std::vector<Job> fwd1, mid, last;  // launch groups: fc1 (+ dH) | fc2, dW2 (+ dH) | dW1, dx
  for (int r = 0; r < tp; ++r) {
    int64_t lo, hi;
    shard_of(f, tp, r, &lo, &hi);
    const int64_t fr = hi - lo;
    if (fr == 0) continue;
    char* Pr = pre + T * lo * e;  // rank-local T x fr blocks
    char* Hr = actv + T * lo * e;
    float* ydst = direct ? y : zpart + nslots * pstride;
    float* xdst = direct ? dx : xpart + nslots * pstride;
    tpr::GemmProb p1;
    if (math) {  // w1 d x f, w2 f x d
      p1 = co ? prob(x, d, 1, cb(w1) + lo * e, f, 1, p32 + T * lo, fr, T, fr, d)
              : prob(x, d, 1, cb(w1) + lo * e, f, 1, Pr, fr, T, fr, d, nullptr, Hr);
      p1.act = act;
      fwd1.push_back(job(p1, true, false, co ? tpr::EPI_F32 : tpr::EPI_ACT));
      mid.push_back(job(prob(Hr, fr, 1, cb(w2) + lo * d * e, d, 1, ydst, d, T, d, fr), true, false, tpr::EPI_F32));
      mid.push_back(job(prob(Hr, 1, fr, gy, d, 1, dw2 + lo * d, d, fr, d, T), false, false, tpr::EPI_F32));
      if (co)
        fwd1.push_back(job(prob(gy, d, 1, cb(w2) + lo * d * e, 1, d, dh32 + T * lo, fr, T, fr, d), true, true,
                           tpr::EPI_F32));
      else
        mid.push_back(job(prob(gy, d, 1, cb(w2) + lo * d * e, 1, d, Pr, fr, T, fr, d, Pr), true, true, tpr::EPI_MUL));
      last.push_back(job(prob(x, 1, d, Pr, fr, 1, dw1 + lo, f, d, fr, T), false, false, tpr::EPI_F32));
      last.push_back(job(prob(Pr, fr, 1, cb(w1) + lo * e, 1, f, xdst, d, T, d, fr), true, true, tpr::EPI_F32));
    } else {  // w1 (f, d), w2 (d, f)
      p1 = co ? prob(x, d, 1, cb(w1) + lo * d * e, 1, d, p32 + T * lo, fr, T, fr, d)
              : prob(x, d, 1, cb(w1) + lo * d * e, 1, d, Pr, fr, T, fr, d, nullptr, Hr);
      p1.act = act;
      fwd1.push_back(job(p1, true, true, co ? tpr::EPI_F32 : tpr::EPI_ACT));
      mid.push_back(job(prob(Hr, fr, 1, cb(w2) + lo * e, 1, f, ydst, d, T, d, fr), true, true, tpr::EPI_F32));
      mid.push_back(job(prob(gy, 1, d, Hr, fr, 1, dw2 + lo, f, d, fr, T), false, false, tpr::EPI_F32));
      if (co)
        fwd1.push_back(job(prob(gy, d, 1, cb(w2) + lo * e, f, 1, dh32 + T * lo, fr, T, fr, d), true, false,
                           tpr::EPI_F32));
      else
        mid.push_back(job(prob(gy, d, 1, cb(w2) + lo * e, f, 1, Pr, fr, T, fr, d, Pr), true, false, tpr::EPI_MUL));
      last.push_back(job(prob(Pr, 1, fr, x, d, 1, dw1 + lo * d, d, fr, d, T), false, false, tpr::EPI_F32));
      last.push_back(job(prob(Pr, fr, 1, cb(w1) + lo * d * e, d, 1, xdst, d, T, d, fr), true, false, tpr::EPI_F32));
    }
    ++nslots;
  }
  hipError_t he;
  if ((he = run_jobs(fwd1, dtype, s)) != hipSuccess) return hip_fail(he, "fc1 GEMM");
  if (co) {
    // H = sigma(P) and dZ = dH * sigma'(P); the rank blocks of P, dH, H and
    // dZ sit at the same element offsets (T * lo), so one pass covers all.
    if ((he = tpr::launch_act_mul(p32, dh32, actv, pre, T * f, act, s)) != hipSuccess)
      return hip_fail(he, "activation and dZ");
    mid.insert(mid.end(), last.begin(), last.end());
    last.clear();
  }
  if ((he = run_jobs(mid, dtype, s)) != hipSuccess) return hip_fail(he, "fc2 / dW2 / dH GEMMs");
  if ((he = run_jobs(last, dtype, s)) != hipSuccess) return hip_fail(he, "dW1 / dx GEMMs");
  // The block's one reduction each way: y = sum_r Z_r, dx = sum_r dx_r.
  if ((he = finish_sum(y, T, d, zpart, nslots, pstride, direct, s)) != hipSuccess) return hip_fail(he, "y reduction");
  if ((he = finish_sum(dx, T, d, xpart, nslots, pstride, direct, s)) != hipSuccess)
    return hip_fail(he, "dx reduction");
  return TPR_OK;
}

// Gated MLP: {A_r = X W1_r, U_r = X W3_r} | H = sigma(A) U | {Z_r = H_r W2_r,
// dW2_r = H_r^T gy, dH_r = gy W2_r^T} | dA = dH U sigma'(A), dU = dH sigma(A)
// | {dW1_r = X^T dA_r, dW3_r = X^T dU_r, dx_r = [dA_r | dU_r] [W1_r | W3_r]^T}.
// dA_r and dU_r sit side by side (T x 2 f_r, dH written into the dA half),
// and a copy of the rank's weight columns [W1_r | W3_r] makes dx_r one
// product of inner size 2 f_r, written straight to dx for tp == 1.
int mlp_gated(int tp, int dtype, bool math, int act, int64_t T, int64_t d, int64_t f, const void* x, const void* w1,
              const void* w3, const void* w2, const void* gy, float* y, float* dx, float* dw1, float* dw3, float* dw2,
              void* ws, hipStream_t s) {
  const int64_t e = esize(dtype);
  const size_t tf = align256((size_t)(T * f * e));
  char* wsb = static_cast<char*>(ws);
  char* Ab = wsb;             // gate pre-activation, rank blocks T x f_r
  char* Ub = wsb + tf;        // up projection
  char* Hb = wsb + 2 * tf;    // sigma(A) U
  char* dAUb = wsb + 3 * tf;  // rank blocks T x 2 f_r: [dH, then dA | dU]
  char* Wc = wsb + 5 * tf;    // rank blocks of [W1_r | W3_r]: d x 2 f_r (math) or 2 f_r x d (torch)
  const int64_t pstride = (int64_t)(align256((size_t)(T * d * 4)) / 4);
  float* zpart = reinterpret_cast<float*>(wsb + 5 * tf + align256((size_t)(d * 2 * f * e)));
  float* xpart = zpart + (int64_t)tp * pstride;
  const bool direct = tp == 1;
  const int raw = dtype == TPR_BF16 ? tpr::EPI_BF16 : tpr::EPI_F32;  // output in the compute dtype
  int nslots = 0;
  struct Rank {
    int64_t lo, fr;
  };
  std::vector<Rank> ranks;
  std::vector<Job> fwd1, mid, last;
  for (int r = 0; r < tp; ++r) {
    int64_t lo, hi;
    shard_of(f, tp, r, &lo, &hi);
    const int64_t fr = hi - lo;
    if (fr == 0) continue;
    ranks.push_back(Rank{lo, fr});
    char* Ar = Ab + T * lo * e;
    char* Ur = Ub + T * lo * e;
    char* Hr = Hb + T * lo * e;
    char* dAr = dAUb + 2 * T * lo * e;  // T x 2 fr, dA in columns [0, fr), dU in [fr, 2 fr)
    char* dUr = dAr + fr * e;
    char* Wr = Wc + 2 * d * lo * e;
    float* ydst = direct ? y : zpart + nslots * pstride;
    float* xdst = direct ? dx : xpart + nslots * pstride;
    if (math) {  // w1, w3 d x f, w2 f x d; Wr is d x 2 fr
      fwd1.push_back(job(prob(x, d, 1, cb(w1) + lo * e, f, 1, Ar, fr, T, fr, d), true, false, raw));
      fwd1.push_back(job(prob(x, d, 1, cb(w3) + lo * e, f, 1, Ur, fr, T, fr, d), true, false, raw));
      mid.push_back(job(prob(Hr, fr, 1, cb(w2) + lo * d * e, d, 1, ydst, d, T, d, fr), true, false, tpr::EPI_F32));
      mid.push_back(job(prob(Hr, 1, fr, gy, d, 1, dw2 + lo * d, d, fr, d, T), false, false, tpr::EPI_F32));
      mid.push_back(job(prob(gy, d, 1, cb(w2) + lo * d * e, 1, d, dAr, 2 * fr, T, fr, d), true, true, raw));
      last.push_back(job(prob(x, 1, d, dAr, 2 * fr, 1, dw1 + lo, f, d, fr, T), false, false, tpr::EPI_F32));
      last.push_back(job(prob(x, 1, d, dUr, 2 * fr, 1, dw3 + lo, f, d, fr, T), false, false, tpr::EPI_F32));
      last.push_back(job(prob(dAr, 2 * fr, 1, Wr, 1, 2 * fr, xdst, d, T, d, 2 * fr), true, true, tpr::EPI_F32));
    } else {  // w1, w3 (f, d), w2 (d, f); Wr is 2 fr x d
      fwd1.push_back(job(prob(x, d, 1, cb(w1) + lo * d * e, 1, d, Ar, fr, T, fr, d), true, true, raw));
      fwd1.push_back(job(prob(x, d, 1, cb(w3) + lo * d * e, 1, d, Ur, fr, T, fr, d), true, true, raw));
      mid.push_back(job(prob(Hr, fr, 1, cb(w2) + lo * e, 1, f, ydst, d, T, d, fr), true, true, tpr::EPI_F32));
      mid.push_back(job(prob(gy, 1, d, Hr, fr, 1, dw2 + lo, f, d, fr, T), false, false, tpr::EPI_F32));
      mid.push_back(job(prob(gy, d, 1, cb(w2) + lo * e, f, 1, dAr, 2 * fr, T, fr, d), true, false, raw));
      last.push_back(job(prob(dAr, 1, 2 * fr, x, d, 1, dw1 + lo * d, d, fr, d, T), false, false, tpr::EPI_F32));
      last.push_back(job(prob(dUr, 1, 2 * fr, x, d, 1, dw3 + lo * d, d, fr, d, T), false, false, tpr::EPI_F32));
      last.push_back(job(prob(dAr, 2 * fr, 1, Wr, d, 1, xdst, d, T, d, 2 * fr), true, false, tpr::EPI_F32));
    }
    ++nslots;
  }
  hipError_t he;
  // The rank's weight columns side by side (independent of everything else).
  for (const Rank& rk : ranks) {
    char* Wr = Wc + 2 * d * rk.lo * e;
    if (math) {  // rows of W1[:, lo:hi] then W3[:, lo:hi]
      if ((he = tpr::launch_copy_2d(Wr, 2 * rk.fr * e, cb(w1) + rk.lo * e, f * e, d, rk.fr * e, s)) != hipSuccess ||
          (he = tpr::launch_copy_2d(Wr + rk.fr * e, 2 * rk.fr * e, cb(w3) + rk.lo * e, f * e, d, rk.fr * e, s)) !=
              hipSuccess)
        return hip_fail(he, "gate / up weight copy");
    } else {  // rows lo..hi of w1, then of w3
      if ((he = tpr::launch_copy_2d(Wr, d * e, cb(w1) + rk.lo * d * e, d * e, rk.fr, d * e, s)) != hipSuccess ||
          (he = tpr::launch_copy_2d(Wr + rk.fr * d * e, d * e, cb(w3) + rk.lo * d * e, d * e, rk.fr, d * e, s)) !=
              hipSuccess)
        return hip_fail(he, "gate / up weight copy");
    }
  }
  if ((he = run_jobs(fwd1, dtype, s)) != hipSuccess) return hip_fail(he, "gate / up GEMMs");
  if ((he = tpr::launch_glu_fwd(dtype, Ab, Ub, Hb, T * f, act, s)) != hipSuccess) return hip_fail(he, "gate * up");
  if ((he = run_jobs(mid, dtype, s)) != hipSuccess) return hip_fail(he, "down / dW2 / dH GEMMs");
  for (const Rank& rk : ranks) {
    char* dAr = dAUb + 2 * T * rk.lo * e;
    if ((he = tpr::launch_glu_bwd_2d(dtype, dAr, Ab + T * rk.lo * e, Ub + T * rk.lo * e, dAr + rk.fr * e, T, rk.fr,
                                     2 * rk.fr, act, s)) != hipSuccess)
      return hip_fail(he, "gate / up gradients");
  }
  if ((he = run_jobs(last, dtype, s)) != hipSuccess) return hip_fail(he, "dW1 / dW3 / dx GEMMs");
  if ((he = finish_sum(y, T, d, zpart, nslots, pstride, direct, s)) != hipSuccess) return hip_fail(he, "y reduction");
  if ((he = finish_sum(dx, T, d, xpart, nslots, pstride, direct, s)) != hipSuccess) return hip_fail(he, "dx reduction");
  return TPR_OK;
}

int mlp_checked(int tp, int dtype, int w_layout, int act, int64_t T, int64_t d, int64_t f, const void* x,
                const void* w1, const void* w3, const void* w2, const void* gy, float* y, float* dx, float* dw1,
                float* dw3, float* dw2, void* ws, size_t ws_bytes, void* stream) {
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(f))
    return fail(TPR_ERR_SHAPE, "T, d, f must be in [0, 2^31) (got %lld, %lld, %lld)", (long long)T, (long long)d,
                (long long)f);
  if (tp < 1) return fail(TPR_ERR_PARTITION, "tp must be >= 1 (got %d)", tp);
  if (!dtype_ok(dtype)) return fail(TPR_ERR_DTYPE, "unknown dtype %d", dtype);
  if (w_layout != TPR_W_MATH && w_layout != TPR_W_TORCH) return fail(TPR_ERR_DTYPE, "unknown w_layout %d", w_layout);
  if (check_act(act) != TPR_OK) return TPR_ERR_VALUE;
  const bool gated = w3 != nullptr;
  if ((T * d > 0 && (x == nullptr || gy == nullptr || y == nullptr || dx == nullptr)) ||
      (d * f > 0 && (w1 == nullptr || w2 == nullptr || dw1 == nullptr || dw2 == nullptr)) ||
      (gated && d * f > 0 && dw3 == nullptr))
    return fail(TPR_ERR_NULLPTR, "a non-empty input or output pointer is NULL");
  const size_t need = mlp_workspace(tp, dtype, gated, T, d, f);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(TPR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const bool math = w_layout == TPR_W_MATH;
  if (gated) return mlp_gated(tp, dtype, math, act, T, d, f, x, w1, w3, w2, gy, y, dx, dw1, dw3, dw2, ws, s);
  return mlp_plain(tp, dtype, math, act, T, d, f, x, w1, w2, gy, y, dx, dw1, dw2, ws, s);
}

}  // namespace

size_t tp_mlp_workspace_bytes(int tp, int dtype, int64_t T, int64_t d, int64_t f) {
  return mlp_workspace(tp, dtype, false, T, d, f);
}

int tp_mlp_fwd_bwd(int tp, int dtype, int w_layout, int64_t T, int64_t d, int64_t f, const void* x, const void* w1,
                   const void* w2, const void* gy, float* y, float* dx, float* dw1, float* dw2, void* ws,
                   size_t ws_bytes, void* stream) {
  return mlp_checked(tp, dtype, w_layout, TPR_ACT_GELU, T, d, f, x, w1, nullptr, w2, gy, y, dx, dw1, nullptr, dw2, ws,
                     ws_bytes, stream);
}

size_t tp_mlp_act_workspace_bytes(int tp, int dtype, int gated, int64_t T, int64_t d, int64_t f) {
  return mlp_workspace(tp, dtype, gated != 0, T, d, f);
}

int tp_mlp_act_fwd_bwd(int tp, int dtype, int w_layout, int act, int64_t T, int64_t d, int64_t f, const void* x,
                       const void* w1, const void* w3, const void* w2, const void* gy, float* y, float* dx,
                       float* dw1, float* dw3, float* dw2, void* ws, size_t ws_bytes, void* stream) {
  return mlp_checked(tp, dtype, w_layout, act, T, d, f, x, w1, w3, w2, gy, y, dx, dw1, dw3, dw2, ws, ws_bytes,
                     stream);
}

// ---------------------------------------------------------------- attention projections
size_t tp_attn_proj_workspace_bytes(int tp, int dtype, int64_t T, int64_t d, int n_q_heads, int n_kv_heads,
                                    int head_dim) {
  if (tp < 1 || !dtype_ok(dtype) || T < 0 || d < 0 || n_q_heads < 1 || n_kv_heads < 1 || head_dim < 1) return 0;
  return tp > 1 ? 2 * (size_t)tp * align256((size_t)(T * d * 4)) : 0;  // y and dx partials
}

int tp_attn_proj_fwd_bwd(int tp, int dtype, int w_layout, int64_t T, int64_t d, int n_q_heads, int n_kv_heads,
                         int head_dim, const void* x, const void* w_qkv, const void* w_o, const void* ctx,
                         const void* gy, const void* dqkv, void* qkv, float* y, void* dctx, float* dx, float* dw_qkv,
                         float* dw_o, void* ws, size_t ws_bytes, void* stream) {
  if (!dim_ok(T) || !dim_ok(d) || head_dim < 1)
    return fail(TPR_ERR_SHAPE, "T, d must be in [0, 2^31) and head_dim >= 1 (got %lld, %lld, %d)", (long long)T,
                (long long)d, head_dim);
  if (n_q_heads < 1 || n_kv_heads < 1 || n_q_heads % n_kv_heads != 0)
    return fail(TPR_ERR_SHAPE, "query heads (%d) must be a positive multiple of KV heads (%d)", n_q_heads,
                n_kv_heads);
  if (tp < 1) return fail(TPR_ERR_PARTITION, "tp must be >= 1 (got %d)", tp);
  if (n_q_heads % tp != 0 || n_kv_heads % tp != 0)
    return fail(TPR_ERR_PARTITION, "tp = %d must divide the query heads (%d) and the KV heads (%d)", tp, n_q_heads,
                n_kv_heads);
  if (!dtype_ok(dtype)) return fail(TPR_ERR_DTYPE, "unknown dtype %d", dtype);
  if (w_layout != TPR_W_MATH && w_layout != TPR_W_TORCH) return fail(TPR_ERR_DTYPE, "unknown w_layout %d", w_layout);
  const int64_t nq = (int64_t)n_q_heads * head_dim, nkv = (int64_t)n_kv_heads * head_dim;
  const int64_t nqkv = nq + 2 * nkv;
  if (!dim_ok(nqkv)) return fail(TPR_ERR_SHAPE, "projection width %lld out of range", (long long)nqkv);
  if ((T * d > 0 && (x == nullptr || gy == nullptr || y == nullptr || dx == nullptr)) ||
      (T * nqkv > 0 && (dqkv == nullptr || qkv == nullptr || ctx == nullptr || dctx == nullptr)) ||
      (d * nqkv > 0 && (w_qkv == nullptr || w_o == nullptr || dw_qkv == nullptr || dw_o == nullptr)))
    return fail(TPR_ERR_NULLPTR, "a non-empty input or output pointer is NULL");
  const size_t need = tp_attn_proj_workspace_bytes(tp, dtype, T, d, n_q_heads, n_kv_heads, head_dim);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(TPR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t e = esize(dtype);
  const bool math = w_layout == TPR_W_MATH;
  const bool direct = tp == 1;
  const int64_t pstride = (int64_t)(align256((size_t)(T * d * 4)) / 4);
  float* ypart = static_cast<float*>(ws);
  float* xpart = direct ? nullptr : ypart + (int64_t)tp * pstride;
  const int raw = dtype == TPR_BF16 ? tpr::EPI_BF16 : tpr::EPI_F32;  // outputs the core consumes
  const int64_t wr = nqkv / tp, kr = nq / tp;  // rank r: QKV columns [r wr, (r+1) wr), W_O rows [r kr, (r+1) kr)
  std::vector<Job> jobs;  // every product is independent of the others: one grouped launch
  for (int r = 0; r < tp; ++r) {
    const int64_t c0 = r * wr, k0 = r * kr;
    float* ydst = direct ? y : ypart + r * pstride;
    float* xdst = direct ? dx : xpart + r * pstride;
    // Column-parallel QKV: qkv_r = x W_r; dW_r = x^T dqkv_r; dx_r = dqkv_r W_r^T.
    // Row-parallel output: y_r = ctx_r W_O,r; dctx_r = gy W_O,r^T; dW_O,r = ctx_r^T gy.
    if (math) {  // w_qkv d x nqkv, w_o nq x d
      jobs.push_back(job(prob(x, d, 1, cb(w_qkv) + c0 * e, nqkv, 1, static_cast<char*>(qkv) + c0 * e, nqkv, T, wr, d), true, false, raw));
      jobs.push_back(job(prob(x, 1, d, cb(dqkv) + c0 * e, nqkv, 1, dw_qkv + c0, nqkv, d, wr, T), false, false, tpr::EPI_F32));
      jobs.push_back(job(prob(cb(dqkv) + c0 * e, nqkv, 1, cb(w_qkv) + c0 * e, 1, nqkv, xdst, d, T, d, wr), true, true, tpr::EPI_F32));
      jobs.push_back(job(prob(cb(ctx) + k0 * e, nq, 1, cb(w_o) + k0 * d * e, d, 1, ydst, d, T, d, kr), true, false, tpr::EPI_F32));
      jobs.push_back(job(prob(gy, d, 1, cb(w_o) + k0 * d * e, 1, d, static_cast<char*>(dctx) + k0 * e, nq, T, kr, d), true, true, raw));
      jobs.push_back(job(prob(cb(ctx) + k0 * e, 1, nq, gy, d, 1, dw_o + k0 * d, d, kr, d, T), false, false, tpr::EPI_F32));
    } else {  // w_qkv (nqkv, d), w_o (d, nq)
      jobs.push_back(job(prob(x, d, 1, cb(w_qkv) + c0 * d * e, 1, d, static_cast<char*>(qkv) + c0 * e, nqkv, T, wr, d), true, true, raw));
      jobs.push_back(job(prob(cb(dqkv) + c0 * e, 1, nqkv, x, d, 1, dw_qkv + c0 * d, d, wr, d, T), false, false, tpr::EPI_F32));
      jobs.push_back(job(prob(cb(dqkv) + c0 * e, nqkv, 1, cb(w_qkv) + c0 * d * e, d, 1, xdst, d, T, d, wr), true, false, tpr::EPI_F32));
      jobs.push_back(job(prob(cb(ctx) + k0 * e, nq, 1, cb(w_o) + k0 * e, 1, nq, ydst, d, T, d, kr), true, true, tpr::EPI_F32));
      jobs.push_back(job(prob(gy, d, 1, cb(w_o) + k0 * e, nq, 1, static_cast<char*>(dctx) + k0 * e, nq, T, kr, d), true, false, raw));
      jobs.push_back(job(prob(gy, 1, d, cb(ctx) + k0 * e, nq, 1, dw_o + k0, nq, d, kr, T), false, false, tpr::EPI_F32));
    }
  }
  hipError_t he;
  if ((he = run_jobs(jobs, dtype, s)) != hipSuccess) return hip_fail(he, "projection GEMMs");
  // The block's one reduction each way: y = sum_r y_r, dx = sum_r dx_r.
  if ((he = finish_sum(y, T, d, ypart, tp, pstride, direct, s)) != hipSuccess) return hip_fail(he, "y reduction");
  if ((he = finish_sum(dx, T, d, xpart, tp, pstride, direct, s)) != hipSuccess) return hip_fail(he, "dx reduction");
  return TPR_OK;
}

// ---------------------------------------------------------------- vocab CE
size_t vocab_parallel_ce_workspace_bytes(int parts, int64_t T, int64_t V) {
  if (parts < 1 || T < 0 || V < 0) return 0;
  return align256((size_t)T * 4);
}

}  // extern "C"

namespace {

// Checks shared by the two plain CE entry points (everything but the workspace).
int ce_args_checked(int parts, int dtype, int64_t T, int64_t V, const void* logits, const int64_t* labels,
                    const float* loss, const void* dlogits) {
  if (T < 0 || V < 0 || T > UINT_MAX || V / 8 > INT_MAX)
    return fail(TPR_ERR_SHAPE, "T and V out of range (got %lld, %lld)", (long long)T, (long long)V);
  if (T > 0 && V == 0) return fail(TPR_ERR_SHAPE, "V must be >= 1 when T > 0");
  if (parts < 1) return fail(TPR_ERR_PARTITION, "parts must be >= 1 (got %d)", parts);
  if (!dtype_ok(dtype)) return fail(TPR_ERR_DTYPE, "unknown dtype %d", dtype);
  if (loss == nullptr || (T > 0 && (logits == nullptr || labels == nullptr || dlogits == nullptr)))
    return fail(TPR_ERR_NULLPTR, "loss, logits, labels or dlogits is NULL");
  return TPR_OK;
}

int ce_launch(int parts, int dtype, int64_t T, int64_t V, const void* logits, const int64_t* labels, float* loss,
              void* dlogits, float* shard_stats, float* row_loss, void* stream) {
  tpr::CeArgs a{};
  a.logits = logits;
  a.labels = labels;
  a.dlogits = dlogits;
  a.shard_stats = shard_stats;
  a.row_loss = row_loss;
  a.loss = loss;
  a.T = T;
  a.V = V;
  a.parts = parts;
  a.dtype = dtype;
  const hipError_t he = tpr::launch_vocab_ce(a, static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "vocab CE launch");
  return TPR_OK;
}

}  // namespace

extern "C" {

int vocab_parallel_ce_fwd_bwd(int parts, int dtype, int64_t T, int64_t V, const void* logits, const int64_t* labels,
                              float* loss, void* dlogits, float* shard_stats, void* ws, size_t ws_bytes,
                              void* stream) {
  const int st = ce_args_checked(parts, dtype, T, V, logits, labels, loss, dlogits);
  if (st != TPR_OK) return st;
  const size_t need = vocab_parallel_ce_workspace_bytes(parts, T, V);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(TPR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  return ce_launch(parts, dtype, T, V, logits, labels, loss, dlogits, shard_stats, static_cast<float*>(ws), stream);
}

int vocab_parallel_ce_fwd_bwd_noalloc(int parts, int dtype, int64_t T, int64_t V, const void* logits,
                                      const int64_t* labels, float* loss, void* dlogits, float* shard_stats,
                                      void* stream) {
  const int st = ce_args_checked(parts, dtype, T, V, logits, labels, loss, dlogits);
  if (st != TPR_OK) return st;
  if (T > tpr::kCeStaticRows)
    return fail(TPR_ERR_WORKSPACE, "T = %lld rows exceed the %lld rows of the library's static scratch", (long long)T,
                (long long)tpr::kCeStaticRows);
  float* rows = nullptr;
  const hipError_t he = tpr::ce_static_scratch(&rows);
  if (he != hipSuccess) return hip_fail(he, "static scratch of the current device");
  return ce_launch(parts, dtype, T, V, logits, labels, loss, dlogits, shard_stats, rows, stream);
}

// ---------------------------------------------------------------- CE options
size_t vocab_parallel_ce_opts_workspace_bytes(int parts, int64_t T, int64_t V) {
  if (parts < 1 || T < 0 || V < 0) return 0;
  return align256((size_t)T * 4) + 256;  // per-row losses, then the counted-row total and its reciprocal
}

int vocab_parallel_ce_opts_fwd_bwd(int parts, int dtype, int64_t T, int64_t V, int64_t v_valid, int64_t ignore_index,
                                   float label_smoothing, const void* logits, const int64_t* labels, float* loss,
                                   void* dlogits, float* shard_stats, void* ws, size_t ws_bytes, void* stream) {
  if (T < 0 || V < 0 || T > UINT_MAX || V / 8 > INT_MAX)
    return fail(TPR_ERR_SHAPE, "T and V out of range (got %lld, %lld)", (long long)T, (long long)V);
  if (T > 0 && V == 0) return fail(TPR_ERR_SHAPE, "V must be >= 1 when T > 0");
  if (v_valid < (V > 0 ? 1 : 0) || v_valid > V)
    return fail(TPR_ERR_SHAPE, "v_valid must be in [1, V] (got %lld, V = %lld)", (long long)v_valid, (long long)V);
  if (parts < 1) return fail(TPR_ERR_PARTITION, "parts must be >= 1 (got %d)", parts);
  if (!dtype_ok(dtype)) return fail(TPR_ERR_DTYPE, "unknown dtype %d", dtype);
  if (!(label_smoothing >= 0.f && label_smoothing <= 1.f))
    return fail(TPR_ERR_VALUE, "label_smoothing must be in [0, 1] (got %g)", (double)label_smoothing);
  if (loss == nullptr || (T > 0 && (logits == nullptr || labels == nullptr || dlogits == nullptr)))
    return fail(TPR_ERR_NULLPTR, "loss, logits, labels or dlogits is NULL");
  const size_t need = vocab_parallel_ce_opts_workspace_bytes(parts, T, V);
  if (ws_bytes < need || ws == nullptr)
    return fail(TPR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);
  char* wsb = static_cast<char*>(ws);
  tpr::CeArgs a{};
  a.logits = logits;
  a.labels = labels;
  a.dlogits = dlogits;
  a.shard_stats = shard_stats;
  a.row_loss = reinterpret_cast<float*>(wsb);
  a.loss = loss;
  a.T = T;
  a.V = V;
  a.parts = parts;
  a.dtype = dtype;
  a.opt = true;
  a.v_valid = v_valid;
  a.ignore_index = ignore_index;
  a.smoothing = label_smoothing;
  a.count = reinterpret_cast<int*>(wsb + align256((size_t)T * 4));
  a.inv_count = reinterpret_cast<float*>(wsb + align256((size_t)T * 4) + 4);
  const hipError_t he = tpr::launch_vocab_ce(a, static_cast<hipStream_t>(stream));
  if (he != hipSuccess) return hip_fail(he, "vocab CE launch");
  return TPR_OK;
}

// ---------------------------------------------------------------- vocab head + CE
size_t vocab_parallel_head_ce_workspace_bytes(int parts, int dtype, int64_t T, int64_t d, int64_t V) {
  if (parts < 1 || !dtype_ok(dtype) || T < 0 || d < 0 || V < 0) return 0;
  size_t b = 2 * align256((size_t)(T * V * esize(dtype)));  // logits, dlogits
  b += vocab_parallel_ce_workspace_bytes(parts, T, V);       // per-row losses
  if (parts > 1) b += (size_t)parts * align256((size_t)(T * d * 4));  // dh partials
  return b;
}

int vocab_parallel_head_ce_fwd_bwd(int parts, int dtype, int w_layout, int64_t T, int64_t d, int64_t V,
                                   const void* h, const void* w, const int64_t* labels, float* loss, float* dh,
                                   float* dw, void* ws, size_t ws_bytes, void* stream) {
  if (!dim_ok(T) || !dim_ok(d) || !dim_ok(V) || V / 8 > INT_MAX)
    return fail(TPR_ERR_SHAPE, "T, d, V must be in [0, 2^31) (got %lld, %lld, %lld)", (long long)T, (long long)d,
                (long long)V);
  if (T > 0 && V == 0) return fail(TPR_ERR_SHAPE, "V must be >= 1 when T > 0");
  if (parts < 1) return fail(TPR_ERR_PARTITION, "parts must be >= 1 (got %d)", parts);
  if (!dtype_ok(dtype)) return fail(TPR_ERR_DTYPE, "unknown dtype %d", dtype);
  if (w_layout != TPR_W_MATH && w_layout != TPR_W_TORCH) return fail(TPR_ERR_DTYPE, "unknown w_layout %d", w_layout);
  if (loss == nullptr || (T > 0 && labels == nullptr) || (T * d > 0 && (h == nullptr || dh == nullptr)) ||
      (d * V > 0 && (w == nullptr || dw == nullptr)))
    return fail(TPR_ERR_NULLPTR, "a required input or output pointer is NULL");
  const size_t need = vocab_parallel_head_ce_workspace_bytes(parts, dtype, T, d, V);
  if (ws_bytes < need || (need > 0 && ws == nullptr))
    return fail(TPR_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need, ws_bytes);

  hipStream_t s = static_cast<hipStream_t>(stream);
  const int64_t e = esize(dtype);
  char* wsb = static_cast<char*>(ws);
  char* logits = wsb;
  char* dl = wsb + align256((size_t)(T * V * e));
  float* row_loss = reinterpret_cast<float*>(wsb + 2 * align256((size_t)(T * V * e)));
  float* slots = reinterpret_cast<float*>(reinterpret_cast<char*>(row_loss) + align256((size_t)T * 4));
  const int64_t stride = (int64_t)(align256((size_t)(T * d * 4)) / 4);
  const bool direct = parts == 1;
  const bool math = w_layout == TPR_W_MATH;
  int nslots = 0;
  std::vector<Job> fwd, bwd;

  for (int r = 0; r < parts; ++r) {
    int64_t lo, hi;
    shard_of(V, parts, r, &lo, &hi);
    const int64_t n = hi - lo;
    if (n == 0) continue;
    // Rank r's head columns W_r (d x n): math w is d x V, torch w is V x d.
    const char* wr = math ? cb(w) + lo * e : cb(w) + lo * d * e;
    const int64_t wk = math ? V : 1, wn = math ? 1 : d;  // W_r(k, j) = wr[k * wk + j * wn]
    // logits_r = h W_r (in the compute dtype), landing in its column slice.
    fwd.push_back(job(prob(h, d, 1, wr, wk, wn, logits + lo * e, V, T, n, d), true, !math,
                      dtype == TPR_BF16 ? tpr::EPI_BF16 : tpr::EPI_F32));
    // dW_r = h^T dlogits_r (math, d x n) or its transpose (torch, n x d), in place.
    if (math)
      bwd.push_back(job(prob(h, 1, d, dl + lo * e, V, 1, dw + lo, V, d, n, T), false, false, tpr::EPI_F32));
    else
      bwd.push_back(job(prob(dl + lo * e, 1, V, h, d, 1, dw + lo * d, d, n, d, T), false, false, tpr::EPI_F32));
    // dh_r = dlogits_r W_r^T, a full-shape partial: W_r^T(j, k) = W_r(k, j).
    float* dst = direct ? dh : slots + nslots * stride;
    bwd.push_back(job(prob(dl + lo * e, V, 1, wr, wn, wk, dst, d, T, d, n), true, math, tpr::EPI_F32));
    ++nslots;
  }

  hipError_t he;
  if ((he = run_jobs(fwd, dtype, s)) != hipSuccess) return hip_fail(he, "logits GEMMs");
  tpr::CeArgs a{};
  a.logits = logits;
  a.labels = labels;
  a.dlogits = dl;
  a.shard_stats = nullptr;
  a.row_loss = row_loss;
  a.loss = loss;
  a.T = T;
  a.V = V;
  a.parts = parts;
  a.dtype = dtype;
  if ((he = tpr::launch_vocab_ce(a, s)) != hipSuccess) return hip_fail(he, "vocab CE launch");
  if ((he = run_jobs(bwd, dtype, s)) != hipSuccess) return hip_fail(he, "dW / dh GEMMs");
  // The shared hidden state's gradient, summed across the vocabulary shards.
  if ((he = finish_sum(dh, T, d, slots, nslots, stride, direct, s)) != hipSuccess) return hip_fail(he, "dh reduction");
  return TPR_OK;
}

}  // extern "C"
