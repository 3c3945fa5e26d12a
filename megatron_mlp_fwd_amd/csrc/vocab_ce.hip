// Vocabulary-parallel cross-entropy, forward and backward, for T positions
// with the vocabulary split into `parts` contiguous shards.
//
// Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), section
// 04 / VOCABULARY SHARDS: each shard r finds its local maximum m_r; the
// global maximum m combines them; each shard sums exp(z - m) over its range
// (s_r) and, if it owns the target, contributes z_y - m (t_r); the loss is
// log(sum s_r) - sum t_r and the gradient is exp(z - m)/s minus the one-hot
// target.  The workload averages over positions, so every row's gradient
// carries 1/T.
//
// Fast path (bf16, shard edges on 8-element boundaries, up to 16 shards):
// one 1024-thread workgroup per row holds the whole row in registers (16
// slots of 16 bytes per thread; a slot is a 1024-vector run inside one
// shard), so the logits are read from HBM once and dlogits written once --
// the kernel is bound by HBM bandwidth (4 bytes per logit).  Each exponential
// is computed once: the sum pass keeps exp(z - m) in place of the logit as
// fp16 for the gradient pass (round-to-nearest; only terms below 2^-24 of the
// row maximum flush to zero, which is far below bf16 output resolution).  Per-shard
// statistics are reduced per wave (shuffles) and across waves in LDS in a
// fixed order; the cross-shard combine ("all-reduce" of max, then of the
// sums) is a loop over the shard slots in rank order.
//
// General path (fp32 logits, any shard layout or count): one 256-thread
// workgroup per row, three passes over the row (max per shard, sum and
// target per shard, gradient).  Same arithmetic, the logits are re-read.
//
// Options (a padded vocabulary, ignored rows, label smoothing; the same
// page's list of what a real cross-entropy must also handle) run in the
// paired kernel's CE_OPT / CE_OPT_SMOOTH instances or the general path, after
// a one-workgroup kernel that counts the rows that take part in the mean.
//
// A final single-workgroup kernel averages the per-row losses in a fixed
// order (fp64 accumulation).
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <type_traits>

#include "common.h"

namespace tpr {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int CE_NT = 1024;
constexpr int CE_NW = CE_NT / 64;
constexpr int CE_SLOTS = 16;
constexpr int CE_PMAX = 16;
constexpr float LOG2E = 1.4426950408889634f;

struct CeSlots {
  int nslot;
  int P;
  int shard[CE_SLOTS];  // shard of each slot, non-decreasing
  int vbeg[CE_SLOTS];   // first 8-logit vector of the slot within the row
  int nv[CE_SLOTS];     // vectors in the slot (<= CE_NT)
  int64_t sbeg[CE_PMAX + 1];
};

// Wave-wide reductions with DPP lane moves (no LDS traffic): swap neighbours,
// pairs, half-rows and rows of 16, then broadcast row 0 into row 1 and rows
// 0-1 into rows 2-3; lane 63 ends with the total, read back as a scalar.
// Lanes a move does not feed keep the identity `id`.
#define TPR_DPP(v, id, ctrl, rmask)                                                                           \
  __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, id), __builtin_bit_cast(int, v), \
                                                        ctrl, rmask, 0xf, false))
__device__ __forceinline__ float wave_max(float v) {
  const float id = -INFINITY;
  v = fmaxf(v, TPR_DPP(v, id, 0xB1, 0xf));   // quad_perm [1,0,3,2]
  v = fmaxf(v, TPR_DPP(v, id, 0x4E, 0xf));   // quad_perm [2,3,0,1]
  v = fmaxf(v, TPR_DPP(v, id, 0x141, 0xf));  // row_half_mirror
  v = fmaxf(v, TPR_DPP(v, id, 0x140, 0xf));  // row_mirror
  v = fmaxf(v, TPR_DPP(v, id, 0x142, 0xa));  // row_bcast:15
  v = fmaxf(v, TPR_DPP(v, id, 0x143, 0xc));  // row_bcast:31
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}
__device__ __forceinline__ float wave_sum(float v) {
  const float id = 0.f;
  v += TPR_DPP(v, id, 0xB1, 0xf);
  v += TPR_DPP(v, id, 0x4E, 0xf);
  v += TPR_DPP(v, id, 0x141, 0xf);
  v += TPR_DPP(v, id, 0x140, 0xf);
  v += TPR_DPP(v, id, 0x142, 0xa);
  v += TPR_DPP(v, id, 0x143, 0xc);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float lo16(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi16(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Pairs are converted as two-element vectors: one v_cvt_pk_bf16_f32 /
// v_cvt_pk_f16_f32 (round to nearest even) instead of two single conversions,
// a shift and an or.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, f16x2_t));
}
__device__ __forceinline__ float f16_elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (float)__builtin_bit_cast(_Float16, (uint16_t)((e & 1) ? (w >> 16) : (w & 0xffffu)));
}
// Maximum of the 8 bf16 logits of a vector.
__device__ __forceinline__ float vec_max(const u32x4& v) {
  const float a = fmaxf(fmaxf(lo16(v[0]), hi16(v[0])), lo16(v[1]));
  const float b = fmaxf(fmaxf(hi16(v[1]), lo16(v[2])), hi16(v[2]));
  return fmaxf(fmaxf(a, b), fmaxf(lo16(v[3]), hi16(v[3])));
}
__device__ __forceinline__ float elem(const u32x4& v, int e) {
  const uint32_t w = v[e >> 1];
  return (e & 1) ? hi16(w) : lo16(w);
}

template <bool STATS>
__global__ __launch_bounds__(CE_NT, 1) void ce_fast_kernel(const uint16_t* __restrict__ logits,
                                                          const int64_t* __restrict__ labels,
                                                          uint16_t* __restrict__ dlogits, float* __restrict__ row_loss,
                                                          float* __restrict__ stats, int64_t V, float invT,
                                                          const CeSlots S) {
  __shared__ float red_max[CE_NW][CE_PMAX];
  __shared__ float red_sum[CE_NW][CE_PMAX];
  __shared__ float sh_m[CE_PMAX], sh_s[CE_PMAX];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t row = blockIdx.x;
  const uint16_t* __restrict__ z = logits + row * V;
  uint16_t* __restrict__ dz = dlogits + row * V;
  const int64_t y = labels[row];

  if (tid < CE_NW * CE_PMAX) {
    (&red_max[0][0])[tid] = -INFINITY;
    (&red_sum[0][0])[tid] = 0.f;
  }

  // Load the row once: slot s, lane tid owns vector vbeg[s] + tid.  Idle
  // lanes hold bf16 -inf, which drops out of the max and contributes exp = 0.
  u32x4 v[CE_SLOTS];
#pragma unroll
  for (int s = 0; s < CE_SLOTS; ++s) {
    const bool on = s < S.nslot && tid < S.nv[s];
    v[s] = on ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(z + 8 * ((int64_t)S.vbeg[s] + tid)))
              : u32x4{0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u};
  }
  __syncthreads();

  // Maxima.  With per-shard statistics requested: m_r per shard, a running
  // max over the slots of one shard flushed (wave reduce, one LDS word per
  // wave) when the slot's shard changes, then m = max_r m_r.  Otherwise only
  // the row maximum m is formed (the same value; one wave reduce per wave).
  if constexpr (STATS) {
    float run = -INFINITY;
    int cur = S.shard[0];
#pragma unroll
    for (int s = 0; s < CE_SLOTS; ++s) {
      if (s >= S.nslot) continue;
      if (S.shard[s] != cur) {
        const float w = wave_max(run);
        if (lane == 0) red_max[wid][cur] = w;
        run = -INFINITY;
        cur = S.shard[s];
      }
      run = fmaxf(run, vec_max(v[s]));
    }
    if (S.nslot > 0) {
      const float w = wave_max(run);
      if (lane == 0) red_max[wid][cur] = w;
    }
  } else {
    float run = -INFINITY;
#pragma unroll
    for (int s = 0; s < CE_SLOTS; ++s)
      if (s < S.nslot) run = fmaxf(run, vec_max(v[s]));
    const float w = wave_max(run);
    if (lane == 0) red_max[wid][0] = w;
  }
  __syncthreads();
  if (STATS && tid < S.P) {
    float mr = -INFINITY;
    for (int w = 0; w < CE_NW; ++w) mr = fmaxf(mr, red_max[w][tid]);
    sh_m[tid] = mr;
  }
  if (!STATS && tid == 0) {
    float mr = -INFINITY;
    for (int w = 0; w < CE_NW; ++w) mr = fmaxf(mr, red_max[w][0]);
    sh_m[0] = mr;
  }
  __syncthreads();
  float m = -INFINITY;
  for (int r = 0; r < (STATS ? S.P : 1); ++r) m = fmaxf(m, sh_m[r]);  // all-reduce(max)
  const float mL = m * LOG2E;

  // Per-shard sums s_r with the global maximum.  The target logit is read once
  // from memory (a uniform address); no per-element target test is needed.
  const bool y_ok = y >= 0 && y < V;
  const float zy = y_ok ? __uint_as_float((uint32_t)z[y_ok ? y : 0] << 16) : 0.f;
  {
    float run = 0.f;
    int cur = S.shard[0];
#pragma unroll
    for (int s = 0; s < CE_SLOTS; ++s) {
      if (s >= S.nslot) continue;
      if (STATS && S.shard[s] != cur) {
        const float w = wave_sum(run);
        if (lane == 0) red_sum[wid][cur] = w;
        run = 0.f;
        cur = S.shard[s];
      }
      // exp(z - m) once per logit: summed in fp32, then kept in place of the
      // logit as fp16 (values in (0, 1]) for the gradient pass.
      float ex[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) ex[e] = __builtin_amdgcn_exp2f(elem(v[s], e) * LOG2E - mL);
      run += ((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7]));
#pragma unroll
      for (int q = 0; q < 4; ++q) v[s][q] = pack_f16(ex[2 * q], ex[2 * q + 1]);
    }
    if (S.nslot > 0 || !STATS) {
      const float w = wave_sum(run);
      if (lane == 0) red_sum[wid][STATS ? cur : 0] = w;
    }
  }
  __syncthreads();
  if (tid < (STATS ? S.P : 1)) {
    float sr = 0.f;
    for (int w = 0; w < CE_NW; ++w) sr += red_sum[w][tid];
    sh_s[tid] = sr;
  }
  __syncthreads();
  float ssum = 0.f;
  for (int r = 0; r < (STATS ? S.P : 1); ++r) ssum += sh_s[r];  // all-reduce(sum), rank order
  const float t = y_ok ? zy - m : 0.f;  // the owning shard's target term
  if (tid == 0) row_loss[row] = logf(ssum) - t;
  if (STATS && tid < S.P) {
    const bool owns = y >= S.sbeg[tid] && y < S.sbeg[tid + 1];
    float* st = stats + (row * S.P + tid) * 3;
    st[0] = sh_m[tid];
    st[1] = sh_s[tid];
    st[2] = owns ? t : 0.f;
  }

  // Gradient: exp(z - m) / s / T for every logit, rounded to bf16 and written
  // once; the lane that wrote the vector holding the target then rewrites that
  // element as (exp(z_y - m) / s - 1) / T (same thread, so program order makes
  // the second store the final value).
  const float scale = invT / ssum;
  const int vy = y_ok ? (int)(y >> 3) : -1;
  bool owner = false;
#pragma unroll
  for (int s = 0; s < CE_SLOTS; ++s) {
    if (s < S.nslot && tid < S.nv[s]) {
      const int vi = S.vbeg[s] + tid;
      owner |= vi == vy;
      float g[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) g[e] = f16_elem(v[s], e) * scale;
      __builtin_nontemporal_store(
          u32x4{pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3]), pack_bf16(g[4], g[5]), pack_bf16(g[6], g[7])},
          reinterpret_cast<u32x4*>(dz + 8 * (int64_t)vi));
    }
  }
  if (owner) {
    const float gy = __builtin_amdgcn_exp2f(zy * LOG2E - mL) * scale - invT;
    dz[y] = __builtin_bit_cast(uint16_t, (__bf16)gy);
  }
}


// ---------------------------------------------------------------- options
// Padded vocabulary, ignored rows, label smoothing (see CeArgs).  For a
// counted row with n counted rows in all, v_valid vocabulary columns and
// smoothing eps, the target distribution is q = (1 - eps) onehot(y) +
// eps / v_valid, the row loss is log s - (1 - eps)(z_y - m) - eps (mean z - m)
// over the vocabulary columns, and dL/dz_j = (p_j - q_j) / n; padding columns
// and ignored rows get zero gradient.
struct CeOpt {
  int64_t vv;            // vocabulary columns per row (<= V)
  int64_t ignore;        // label of ignored rows
  float eps;             // label smoothing
  const float* inv_cnt;  // 1 / counted rows, written by ce_count_kernel
  float* stats;          // CE_STATS: T x P x {m_r, s_r, t_r}
  int P;                 // CE_STATS: shards, each vps 8-logit vectors
  int vps;
  uint32_t vps_magic;    // floor((2^32 - 1) / vps) + 1: i / vps = umulhi(i, magic) for i, vps < 2^16
};
enum { CE_PLAIN = 0, CE_OPT = 1, CE_OPT_SMOOTH = 2, CE_STATS = 3 };

// ---------------------------------------------------------------- paired path
// Rows without per-shard statistics, bf16: two 512-thread workgroups per CU,
// each holding its whole row: CP_RS 16-byte slots per thread in registers
// (88 VGPRs) and the remainder in LDS (filled by buffer_load ... lds, so no
// register staging).  With two rows resident per CU, one row's arithmetic
// overlaps the other's loads and stores, which a single register-resident row
// per CU cannot do.  Same arithmetic as ce_fast_kernel<false>.
constexpr int CP_NT = 512;
constexpr int CP_NW = CP_NT / 64;
constexpr int CP_RS = 22;           // register slots per thread
constexpr int CP_RA = 11;           // of which part A (see ce_pair_kernel)
constexpr int CP_LDS_VEC = 4864;    // LDS capacity in 16-byte vectors (76 KB)
constexpr uint32_t CP_OOB = 0x80000000u;

template <int MODE>
__global__ __launch_bounds__(CP_NT) __attribute__((amdgpu_waves_per_eu(4, 4))) void ce_pair_kernel(
    const uint16_t* __restrict__ logits, const int64_t* __restrict__ labels, uint16_t* __restrict__ dlogits,
    float* __restrict__ row_loss, int64_t V, float invT, CeOpt o) {
  constexpr bool OPT = MODE == CE_OPT || MODE == CE_OPT_SMOOTH, SMOOTH = MODE == CE_OPT_SMOOTH;
  constexpr bool STATS = MODE == CE_STATS;
  __shared__ __attribute__((aligned(1024))) u32x4 part[CP_LDS_VEC];
  // CE_STATS: per wave and shard, the maximum and the part A / part B sums
  // (each wave writes only its own row; the rows are combined in order).
  constexpr int TABW = CP_NW * CE_PMAX;
  __shared__ float tab[STATS ? 4 * TABW : 1];
  __shared__ float red[CP_NW];
  __shared__ float red_a[CP_NW];
  __shared__ float red_b[CP_NW];
  __shared__ float red_z[CP_NW];
  __shared__ float tail_sh[8];  // the vocabulary's last rem logits, then their exp
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int64_t row = blockIdx.x;
  const int nvec = (int)(V / 8);
  // With options, whole vocabulary vectors go through the slots; the
  // vocabulary's last rem (< 8) columns are one element each on lanes 0..rem-1
  // of wave 0, and the padding vectors after them are only zero-filled.
  const int nfull = OPT ? (int)(o.vv >> 3) : nvec;
  const int rem = OPT ? (int)(o.vv & 7) : 0;
  const int nreg = nfull < CP_RS * CP_NT ? nfull : CP_RS * CP_NT;  // vectors held in registers
  const int nlds = nfull - nreg;                                    // vectors held in LDS
  const __amdgpu_buffer_rsrc_t rz =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(logits + row * V), (short)0, (int)(V * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t rd =
      __builtin_amdgcn_make_buffer_rsrc(dlogits + row * V, (short)0, (int)(V * 2), 0x00020000);
  const int64_t y = labels[row];
  const u32x4 zero{0u, 0u, 0u, 0u};
  if constexpr (OPT) {
    if (y == o.ignore) {  // ignored row (uniform over the workgroup): zero gradient, no loss
      for (int i = tid; i < nvec; i += CP_NT)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, zero),
                                               rd, (uint32_t)(16 * i), 0, 2);
      if (tid == 0) row_loss[row] = 0.f;
      return;
    }
  }
  const float inv = OPT ? *o.inv_cnt : invT;
  const bool tail = OPT && wid == 0 && lane < rem;
  if (tail) tail_sh[lane] = __uint_as_float((uint32_t)logits[row * V + 8 * nfull + lane] << 16);
  if constexpr (STATS)
    for (int i = tid; i < 4 * TABW; i += CP_NT) tab[i] = i < 2 * TABW ? -INFINITY : 0.f;

  // CE_STATS: fold a group of 64 consecutive vectors [fv, fv + 64) (lane l
  // holds vector fv + l when `on`) into the per-shard tables.  Shards hold
  // vps >= 64 vectors, so at most two shards meet in a group.  A wave keeps
  // one running value for its current shard cs; within a pass it visits
  // shards in increasing order, so each shard's value is complete when the
  // wave moves past it and is reduced (DPP) and written into the wave's
  // table row once per pass: a plain store, no read back.  A group that
  // straddles two shards completes the first with the lanes before the
  // boundary and starts the second with the rest.
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  auto shard_flush = [&](auto max_, float r, int c, float* t) {
    constexpr bool MX = decltype(max_)::value;
    if (c < 0) return;
    const float w = MX ? wave_max(r) : wave_sum(r);
    if (lane == 0) t[wid_u * CE_PMAX + c] = w;
  };
  auto shard_acc = [&](auto max_, float x, bool on, int fv, float& run, int& cs, float* t) {
    constexpr bool MX = decltype(max_)::value;
    const float id = MX ? -INFINITY : 0.f;
    const int lastv = fv + 63 < nvec - 1 ? fv + 63 : nvec - 1;
    const int sa = (int)__umulhi((uint32_t)fv, o.vps_magic), sb = (int)__umulhi((uint32_t)lastv, o.vps_magic);
    const float xv = on ? x : id;
    if (sa != cs) {  // the running shard is complete
      shard_flush(max_, run, cs, t);
      run = id;
      cs = sa;
    }
    if (sa == sb) {
      run = MX ? fmaxf(run, xv) : run + xv;
    } else {
      const bool in_b = fv + lane >= sb * o.vps;
      const float xa = in_b ? id : xv;
      run = MX ? fmaxf(run, xa) : run + xa;
      shard_flush(max_, run, sa, t);
      run = in_b ? xv : id;
      cs = sb;
    }
  };
  using MaxOp = std::integral_constant<bool, true>;
  using SumOp = std::integral_constant<bool, false>;
  float* const tabMA = tab;  // per wave and shard: maximum of part A, of part B, sums of part A, of part B
  float* const tabMB = tab + (STATS ? TABW : 0);
  float* const tabA = tab + (STATS ? 2 * TABW : 0);
  float* const tabB = tab + (STATS ? 3 * TABW : 0);
  // Which vectors each thread holds.  Plain and option instances: register
  // slot s of thread tid holds vector s * CP_NT + tid (a workgroup's loads of
  // one slot are one contiguous run), and the LDS part is walked the same way.
  // CE_STATS: wave w holds the contiguous run [w RW, (w + 1) RW) of the
  // register part (its slot s is vectors w RW + 64 s .. + 63) and walks the
  // run [w RL, (w + 1) RL) of the LDS part, so a wave meets a shard boundary
  // about once per pass instead of every few slots; each wave instruction
  // still loads 64 consecutive vectors.
  const int RW = STATS ? (nreg + 64 * CP_NW - 1) / (64 * CP_NW) * 64 : 0;
  const int RL = STATS ? (nlds + 64 * CP_NW - 1) / (64 * CP_NW) * 64 : 0;
  auto reg_vec = [&](int s, int t) { return STATS ? wid_u * RW + 64 * s + (t & 63) : s * CP_NT + t; };
  auto reg_on = [&](int s, int t) { return (!STATS || 64 * s < RW) && reg_vec(s, t) < nreg; };
  auto reg_fv = [&](int s) { return STATS ? wid_u * RW + 64 * s : s * CP_NT + 64 * wid_u; };
  auto reg_grp = [&](int s) { return STATS ? 64 * s < RW && reg_fv(s) < nreg : reg_fv(s) < nvec; };
  const int nli = STATS ? RL / 64 : (nlds + CP_NT - 1) / CP_NT;  // LDS-part groups per thread
  auto lds_vec = [&](int i) { return STATS ? wid_u * RL + 64 * i + lane : i * CP_NT + tid; };
  auto lds_fv = [&](int i) { return nreg + (STATS ? wid_u * RL + 64 * i : i * CP_NT + 64 * wid_u); };

  // Loads, in issue order: register slots [0, CP_RA), the LDS part, register
  // slots [CP_RA, CP_RS).  Lanes past the row end load zeros (out of range)
  // and are skipped below.
  // Part A (the first slots, the LDS part and the tail) is reduced and
  // exponentiated against its own maximum m_A while part B still arrives;
  // part B then uses the row maximum m, and part A's values are scaled by
  // exp(m_A - m) <= 1 wherever they are used (exact up to rounding).
  u32x4 v[CP_RS];
#pragma unroll
  for (int s = 0; s < CP_RA; ++s) {
    const int i = reg_vec(s, tid);
    v[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rz, reg_on(s, tid) ? (uint32_t)(16 * i) : CP_OOB, 0, 2));
  }
  asm volatile("" ::: "memory");  // keep the issue order
  // LDS part: wave instruction j moves vectors nreg + 64 j .. + 63 (lanes past
  // the row end read zeros and are never used).
  for (int j = wid; 64 * j < nlds; j += CP_NW)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rz, (__attribute__((address_space(3))) void*)&part[64 * j], 16,
                                             (uint32_t)(16 * (nreg + 64 * j + lane)), 0, 0, 2);
  asm volatile("" ::: "memory");
#pragma unroll
  for (int s = CP_RA; s < CP_RS; ++s) {
    const int i = reg_vec(s, tid);
    v[s] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                         rz, reg_on(s, tid) ? (uint32_t)(16 * i) : CP_OOB, 0, 2));
  }
  // Only part B's loads may still be outstanding: this wave's DMA into LDS
  // and its part-A slots have landed.
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(CP_RS - CP_RA) : "memory");
  __syncthreads();

  // ---- part A: maximum, then exp(z - m_A) once per logit (fp16, in place)
  float run = tail ? tail_sh[lane] : -INFINITY;
  if constexpr (STATS) {  // the same, with per-shard maxima of part A
    float r = -INFINITY;
    int cs = -1;
#pragma unroll
    for (int s = 0; s < CP_RA; ++s) {
      const bool on = reg_on(s, tid);
      const float x = on ? vec_max(v[s]) : -INFINITY;
      run = fmaxf(run, x);
      if (reg_grp(s)) shard_acc(MaxOp{}, x, on, reg_fv(s), r, cs, tabMA);
    }
    for (int i = 0; i < nli; ++i) {
      const int j = lds_vec(i), fv = lds_fv(i);
      const float x = j < nlds ? vec_max(part[j]) : -INFINITY;
      run = fmaxf(run, x);
      if (fv < nvec) shard_acc(MaxOp{}, x, j < nlds, fv, r, cs, tabMA);
    }
    shard_flush(MaxOp{}, r, cs, tabMA);
  } else {
#pragma unroll
    for (int s = 0; s < CP_RA; ++s)
      if (s * CP_NT + tid < nreg) run = fmaxf(run, vec_max(v[s]));
    for (int j = tid; j < nlds; j += CP_NT) run = fmaxf(run, vec_max(part[j]));
  }
  {
    const float w = wave_max(run);
    if (lane == 0) red_a[wid] = w;
  }
  __syncthreads();
  float mA = red_a[0];
  for (int w = 1; w < CP_NW; ++w) mA = fmaxf(mA, red_a[w]);
  // Opaque to the compiler: otherwise it keeps the max pass's widened logits
  // alive for the exp pass, which needs far more registers than the row.
#pragma unroll
  for (int s = 0; s < CP_RA; ++s) asm volatile("" : "+v"(v[s]));
  int t2 = tid;  // likewise for the per-slot offsets and masks derived from tid
  asm volatile("" : "+v"(t2));

  // (with smoothing, the exp passes also sum the vocabulary logits)
  float sumA = 0.f, sumB = 0.f, zs = 0.f;
  auto expv = [&](u32x4& x, float mL, float& sum) {
    float ex[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) ex[e] = __builtin_amdgcn_exp2f(elem(x, e) * LOG2E - mL);
    if constexpr (SMOOTH)
      zs += ((elem(x, 0) + elem(x, 1)) + (elem(x, 2) + elem(x, 3))) + ((elem(x, 4) + elem(x, 5)) + (elem(x, 6) + elem(x, 7)));
    sum += ((ex[0] + ex[1]) + (ex[2] + ex[3])) + ((ex[4] + ex[5]) + (ex[6] + ex[7]));
#pragma unroll
    for (int q = 0; q < 4; ++q) x[q] = pack_f16(ex[2 * q], ex[2 * q + 1]);
  };
  {
    const float mAL = mA * LOG2E;
    if (tail) {
      const float zt = tail_sh[lane];
      sumA = __builtin_amdgcn_exp2f(zt * LOG2E - mAL);
      zs = zt;
      tail_sh[lane] = sumA;  // the same lane reads it back for the gradient
    }
    // (the scheduling fences keep the compiler from overlapping slots, which
    // would need registers the 88 data registers leave no room for)
    if constexpr (STATS) {  // the same, with per-shard part A sums
      float r = 0.f;
      int cs = -1;
#pragma unroll
      for (int s = 0; s < CP_RA; ++s) {
        const bool on = reg_on(s, t2);
        float vs = 0.f;
        if (on) expv(v[s], mAL, vs);
        sumA += vs;
        if (reg_grp(s)) shard_acc(SumOp{}, vs, on, reg_fv(s), r, cs, tabA);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int i = 0; i < nli; ++i) {
        const int j = lds_vec(i), fv = lds_fv(i);
        float vs = 0.f;
        if (j < nlds) {
          u32x4 x = part[j];
          expv(x, mAL, vs);
          part[j] = x;  // read in the gradient pass, after the next barriers
        }
        sumA += vs;
        if (fv < nvec) shard_acc(SumOp{}, vs, j < nlds, fv, r, cs, tabA);
      }
      shard_flush(SumOp{}, r, cs, tabA);
    } else {
#pragma unroll
      for (int s = 0; s < CP_RA; ++s) {
        if (s * CP_NT + t2 < nreg) expv(v[s], mAL, sumA);
        __builtin_amdgcn_sched_barrier(0);
      }
      for (int j = tid; j < nlds; j += CP_NT) {
        u32x4 x = part[j];
        expv(x, mAL, sumA);
        part[j] = x;  // the same thread reads it back in the gradient pass
      }
    }
  }

  // ---- part B: the row maximum m, then exp(z - m)
  run = -INFINITY;
  if constexpr (STATS) {  // the same, with per-shard maxima of part B
    float r = -INFINITY;
    int cs = -1;
#pragma unroll
    for (int s = CP_RA; s < CP_RS; ++s) {
      const bool on = reg_on(s, t2);
      const float x = on ? vec_max(v[s]) : -INFINITY;
      run = fmaxf(run, x);
      if (reg_grp(s)) shard_acc(MaxOp{}, x, on, reg_fv(s), r, cs, tabMB);
    }
    shard_flush(MaxOp{}, r, cs, tabMB);
  } else {
#pragma unroll
    for (int s = CP_RA; s < CP_RS; ++s)
      if (s * CP_NT + t2 < nreg) run = fmaxf(run, vec_max(v[s]));
  }
  {
    const float w = wave_max(run);
    if (lane == 0) red_b[wid] = w;
  }
  __syncthreads();
  float m = mA;
  for (int w = 0; w < CP_NW; ++w) m = fmaxf(m, red_b[w]);
  const float mL = m * LOG2E;
  const float fA = __builtin_amdgcn_exp2f((mA - m) * LOG2E);  // part A's values times fA are exp(z - m)
#pragma unroll
  for (int s = CP_RA; s < CP_RS; ++s) asm volatile("" : "+v"(v[s]));
  if constexpr (STATS) {  // the same, with per-shard part B sums
    float r = 0.f;
    int cs = -1;
#pragma unroll
    for (int s = CP_RA; s < CP_RS; ++s) {
      const bool on = reg_on(s, t2);
      float vs = 0.f;
      if (on) expv(v[s], mL, vs);
      sumB += vs;
      if (reg_grp(s)) shard_acc(SumOp{}, vs, on, reg_fv(s), r, cs, tabB);
      __builtin_amdgcn_sched_barrier(0);
    }
    shard_flush(SumOp{}, r, cs, tabB);
  } else {
#pragma unroll
    for (int s = CP_RA; s < CP_RS; ++s) {
      if (s * CP_NT + t2 < nreg) expv(v[s], mL, sumB);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  // exp(z - m) is fp16 in place; the row's values sum to s.
  const int vlim = OPT ? (int)o.vv : nvec * 8;
  const bool y_ok = y >= 0 && y < vlim;
  const float zy = y_ok ? __uint_as_float((uint32_t)logits[row * V + (y_ok ? y : 0)] << 16) : 0.f;
  {
    const float w = wave_sum(sumA * fA + sumB);
    if (lane == 0) red[wid] = w;
    if constexpr (SMOOTH) {
      const float wz = wave_sum(zs);
      if (lane == 0) red_z[wid] = wz;
    }
  }
  __syncthreads();
  float ssum = red[0];
  for (int w = 1; w < CP_NW; ++w) ssum += red[w];
  float zsum = 0.f;
  if constexpr (SMOOTH)
    for (int w = 0; w < CP_NW; ++w) zsum += red_z[w];
  if constexpr (STATS) {  // (m_r, s_r, t_r) per shard; part A sums rescaled by fA
    if (tid < o.P) {
      float mr = -INFINITY, sa = 0.f, sb = 0.f;
      for (int w = 0; w < CP_NW; ++w) {
        mr = fmaxf(mr, fmaxf(tabMA[w * CE_PMAX + tid], tabMB[w * CE_PMAX + tid]));
        sa += tabA[w * CE_PMAX + tid];
        sb += tabB[w * CE_PMAX + tid];
      }
      float* st = o.stats + (row * o.P + tid) * 3;
      st[0] = mr;
      st[1] = sa * fA + sb;
      st[2] = (y_ok && y / (8 * (int64_t)o.vps) == tid) ? zy - m : 0.f;
    }
  }
  const float eps = SMOOTH ? o.eps : 0.f;
  if (tid == 0)
    row_loss[row] =
        logf(ssum) - (1.f - eps) * (y_ok ? zy - m : 0.f) - (SMOOTH ? eps * (zsum / (float)vlim - m) : 0.f);

  // Gradient, written once; the lane that wrote the vector holding the
  // target rewrites that element afterwards (program order).
  const float scale = inv / ssum;
  const float scaleA = scale * fA;
  const float c = SMOOTH ? eps * inv / (float)vlim : 0.f;  // smoothing share of each vocabulary column
  const float cy = (1.f - eps) * inv;                       // the target's share
  const int vy = y_ok ? (int)(y >> 3) : -1;
  auto grad = [&](const u32x4& x, int i, float sc) {
    float g[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) g[e] = SMOOTH ? f16_elem(x, e) * sc - c : f16_elem(x, e) * sc;
    const u32x4 w{pack_bf16(g[0], g[1]), pack_bf16(g[2], g[3]), pack_bf16(g[4], g[5]), pack_bf16(g[6], g[7])};
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, w), rd,
                                           (uint32_t)(16 * i), 0, 2);
  };
  bool owner = false;
#pragma unroll
  for (int s = 0; s < CP_RS; ++s) {
    const int i = reg_vec(s, t2);
    if (reg_on(s, t2)) {
      owner |= i == vy;
      grad(v[s], i, s < CP_RA ? scaleA : scale);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  for (int j = tid; j < nlds; j += CP_NT) {
    owner |= nreg + j == vy;
    grad(part[j], nreg + j, scaleA);
  }
  if (owner) {
    const float gy = __builtin_amdgcn_exp2f(zy * LOG2E - mL) * scale - c - cy;
    dlogits[row * V + y] = __builtin_bit_cast(uint16_t, (__bf16)gy);
  }
  if constexpr (OPT) {
    // The partial last vector (vocabulary lanes, then padding) and the
    // padding vectors after it.
    if (rem > 0 && wid == 0 && lane < 8) {
      const int col = 8 * nfull + lane;
      const float g = lane < rem ? tail_sh[lane] * scaleA - c - (col == y ? cy : 0.f) : 0.f;
      dlogits[row * V + col] = __builtin_bit_cast(uint16_t, (__bf16)g);
    }
    for (int i = nfull + (rem > 0 ? 1 : 0) + tid; i < nvec; i += CP_NT)
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(__attribute__((ext_vector_type(4))) int, zero), rd,
                                             (uint32_t)(16 * i), 0, 2);
  }
}

// ---------------------------------------------------------------- general path
template <typename T>
__device__ __forceinline__ float ld_logit(const T* p, int64_t j);
template <>
__device__ __forceinline__ float ld_logit<float>(const float* p, int64_t j) { return p[j]; }
template <>
__device__ __forceinline__ float ld_logit<uint16_t>(const uint16_t* p, int64_t j) {
  return __uint_as_float((uint32_t)p[j] << 16);
}
template <typename T>
__device__ __forceinline__ void st_grad(T* p, int64_t j, float g);
template <>
__device__ __forceinline__ void st_grad<float>(float* p, int64_t j, float g) { p[j] = g; }
template <>
__device__ __forceinline__ void st_grad<uint16_t>(uint16_t* p, int64_t j, float g) {
  p[j] = __builtin_bit_cast(uint16_t, (__bf16)g);
}

// Block-wide reduction of 256 threads; every thread gets the result.
template <bool MAX>
__device__ __forceinline__ float block_reduce(float v, float* scratch) {
  v = MAX ? wave_max(v) : wave_sum(v);
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  __syncthreads();  // scratch reuse across calls
  if (lane == 0) scratch[wid] = v;
  __syncthreads();
  float r = scratch[0];
  for (int w = 1; w < 4; ++w) r = MAX ? fmaxf(r, scratch[w]) : r + scratch[w];
  return r;
}

template <typename T>
__global__ __launch_bounds__(256) void ce_general_kernel(const T* __restrict__ logits,
                                                         const int64_t* __restrict__ labels, T* __restrict__ dlogits,
                                                         float* __restrict__ row_loss, float* __restrict__ stats,
                                                         int64_t V, int P, float invT, bool opt, CeOpt o) {
  __shared__ float scratch[4];
  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const T* __restrict__ z = logits + row * V;
  T* __restrict__ dz = dlogits + row * V;
  const int64_t y = labels[row];
  const int64_t base = V / P, extra = V % P;
  const int64_t vv = opt ? o.vv : V;         // columns past vv are padding
  const bool counted = !opt || y != o.ignore;
  const float eps = opt ? o.eps : 0.f;
  const float inv = opt ? *o.inv_cnt : invT;

  float m = -INFINITY;
  for (int r = 0; r < P; ++r) {
    const int64_t lo = r * base + (r < extra ? r : extra), hi0 = lo + base + (r < extra ? 1 : 0);
    const int64_t hi = hi0 < vv ? hi0 : vv;
    float loc = -INFINITY;
    for (int64_t j = lo + tid; j < hi; j += 256) loc = fmaxf(loc, ld_logit(z, j));
    const float mr = block_reduce<true>(loc, scratch);
    m = fmaxf(m, mr);
    if (stats != nullptr && tid == 0) stats[(row * P + r) * 3 + 0] = mr;
  }
  const float mL = m * LOG2E;
  float ssum = 0.f, tsum = 0.f, zloc = 0.f;
  for (int r = 0; r < P; ++r) {
    const int64_t lo = r * base + (r < extra ? r : extra), hi0 = lo + base + (r < extra ? 1 : 0);
    const int64_t hi = hi0 < vv ? hi0 : vv;
    float loc = 0.f;
    for (int64_t j = lo + tid; j < hi; j += 256) {
      const float zj = ld_logit(z, j);
      loc += __builtin_amdgcn_exp2f(zj * LOG2E - mL);
      zloc += zj;
    }
    const float sr = block_reduce<false>(loc, scratch);
    const float tr = (counted && y >= lo && y < hi) ? ld_logit(z, y) - m : 0.f;
    ssum += sr;
    tsum += tr;
    if (stats != nullptr && tid == 0) {
      stats[(row * P + r) * 3 + 1] = sr;
      stats[(row * P + r) * 3 + 2] = tr;
    }
  }
  const float zsum = eps != 0.f ? block_reduce<false>(zloc, scratch) : 0.f;
  if (tid == 0)
    row_loss[row] = counted ? logf(ssum) - (1.f - eps) * tsum - eps * (zsum / (float)vv - m) : 0.f;
  const float scale = counted ? inv / ssum : 0.f;
  const float c = counted ? eps * inv / (float)vv : 0.f;
  const float cy = counted ? (1.f - eps) * inv : 0.f;
  for (int64_t j = tid; j < V; j += 256) {
    float g = 0.f;
    if (j < vv && counted) {
      g = __builtin_amdgcn_exp2f(ld_logit(z, j) * LOG2E - mL) * scale - c;
      if (j == y) g -= cy;
    }
    st_grad(dz, j, g);
  }
}

// Counted rows (label != ignore_index) and their reciprocal, for the options.
__global__ __launch_bounds__(1024) void ce_count_kernel(const int64_t* __restrict__ labels, int64_t T,
                                                        int64_t ignore, int* __restrict__ count,
                                                        float* __restrict__ inv_count) {
  __shared__ int part[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int c = 0;
  for (int64_t i = tid; i < T; i += 1024) c += labels[i] != ignore ? 1 : 0;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) c += __shfl_xor(c, off, 64);
  if (lane == 0) part[wid] = c;
  __syncthreads();
  if (tid == 0) {
    int n = 0;
    for (int w = 0; w < 16; ++w) n += part[w];
    count[0] = n;
    inv_count[0] = n > 0 ? (float)(1.0 / (double)n) : 0.f;
  }
}

// Mean of the per-row losses over T rows, or over *count rows when count is
// given (NaN when that is 0: a mean over no rows).
__global__ __launch_bounds__(1024) void loss_mean_kernel(const float* __restrict__ row_loss, int64_t T,
                                                         const int* __restrict__ count, float* __restrict__ loss) {
  __shared__ double part[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  double acc = 0.0;
  for (int64_t i = tid; i < T; i += 1024) acc += (double)row_loss[i];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
  if (lane == 0) part[wid] = acc;
  __syncthreads();
  if (tid == 0) {
    double s = 0.0;
    for (int w = 0; w < 16; ++w) s += part[w];
    if (count != nullptr) {
      const int n = T > 0 ? count[0] : 0;
      loss[0] = n > 0 ? (float)(s / (double)n) : __builtin_nanf("");
    } else {
      loss[0] = T > 0 ? (float)(s / (double)T) : 0.f;
    }
  }
}

bool aligned16(const void* p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// The per-row losses of vocab_parallel_ce_fwd_bwd_noalloc(), for callers that
// cannot allocate a workspace: one copy per device, held until the process
// ends.  Every row kernel writes its row's entry before loss_mean_kernel
// reads it, so nothing needs clearing between calls.
static __device__ __align__(256) float scratch[kCeStaticRows];

}  // namespace

hipError_t ce_static_scratch(float** rows) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static float* addr[kMaxDev];
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    // The array's device address on the current device (the name itself is
    // only a host-side handle).
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = static_cast<float*>(p);
  }
  *rows = addr[dev];
  return hipSuccess;
}

hipError_t launch_vocab_ce(const CeArgs& a, hipStream_t s) {
  CeOpt o{};
  o.vv = a.opt ? a.v_valid : a.V;
  o.ignore = a.ignore_index;
  o.eps = a.opt ? a.smoothing : 0.f;
  o.inv_cnt = a.inv_count;
  if (a.T > 0) {
    const float invT = (float)(1.0 / (double)a.T);
    if (a.opt) {
      hipLaunchKernelGGL(ce_count_kernel, dim3(1), dim3(1024), 0, s, a.labels, a.T, a.ignore_index, a.count,
                         a.inv_count);
      const hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    const int64_t base = a.V / a.parts, extra = a.V % a.parts;
    // Fast path eligibility and slot table (rows with per-shard statistics
    // and no options).
    bool fast = !a.opt && a.dtype == 1 && a.V % 8 == 0 && a.parts <= CE_PMAX && aligned16(a.logits) &&
                aligned16(a.dlogits);
    CeSlots S{};
    S.P = a.parts;
    if (fast) {
      for (int r = 0; r <= a.parts && fast; ++r) {
        const int64_t lo = r * base + (r < extra ? r : extra);
        S.sbeg[r] = r < a.parts ? lo : a.V;
        if (S.sbeg[r] % 8 != 0) fast = false;
      }
      for (int r = 0; r < a.parts && fast; ++r) {
        int64_t vb = S.sbeg[r] / 8, nv = (S.sbeg[r + 1] - S.sbeg[r]) / 8;
        while (nv > 0) {
          if (S.nslot == CE_SLOTS) {
            fast = false;
            break;
          }
          const int64_t take = nv < CE_NT ? nv : CE_NT;
          S.shard[S.nslot] = r;
          S.vbeg[S.nslot] = (int)vb;
          S.nv[S.nslot] = (int)take;
          ++S.nslot;
          vb += take;
          nv -= take;
        }
      }
    }
    // Without per-shard statistics the shard layout does not matter: the
    // paired kernel takes any bf16 row that fits its registers + LDS.
    const int64_t nvec = a.V / 8, nlds = nvec - (nvec < CP_RS * CP_NT ? nvec : CP_RS * CP_NT);
    const bool pair = a.dtype == 1 && a.shard_stats == nullptr && a.V % 8 == 0 && aligned16(a.logits) &&
                      aligned16(a.dlogits) && (nlds + 63) / 64 * 64 <= CP_LDS_VEC;
    const uint16_t* zb = static_cast<const uint16_t*>(a.logits);
    uint16_t* db = static_cast<uint16_t*>(a.dlogits);
    // With per-shard statistics the paired kernel needs equal shards of whole
    // 8-logit vectors, at least 64 of them (a wave's group of 64 consecutive
    // vectors then meets at most two shards), and at most CE_PMAX shards.
    const int64_t vps = a.parts > 0 ? nvec / a.parts : 0;
    const bool pair_stats = a.dtype == 1 && a.shard_stats != nullptr && !a.opt && a.V % 8 == 0 &&
                            a.parts <= CE_PMAX && nvec % a.parts == 0 && vps >= 64 && nvec < 65536 &&
                            aligned16(a.logits) &&
                            aligned16(a.dlogits) && (nlds + 63) / 64 * 64 <= CP_LDS_VEC &&
                            !(getenv("TPRANK_CE_STATS_PATH") && strcmp(getenv("TPRANK_CE_STATS_PATH"), "onerow") == 0);
    if (pair_stats) {
      o.stats = a.shard_stats;
      o.P = a.parts;
      o.vps = (int)vps;
      o.vps_magic = 0xffffffffu / (uint32_t)vps + 1u;
      hipLaunchKernelGGL(ce_pair_kernel<CE_STATS>, dim3((unsigned)a.T), dim3(CP_NT), 0, s, zb, a.labels, db,
                         a.row_loss, a.V, invT, o);
    } else if (pair) {
      if (!a.opt)
        hipLaunchKernelGGL(ce_pair_kernel<CE_PLAIN>, dim3((unsigned)a.T), dim3(CP_NT), 0, s, zb, a.labels, db,
                           a.row_loss, a.V, invT, o);
      else if (a.smoothing == 0.f)
        hipLaunchKernelGGL(ce_pair_kernel<CE_OPT>, dim3((unsigned)a.T), dim3(CP_NT), 0, s, zb, a.labels, db,
                           a.row_loss, a.V, invT, o);
      else
        hipLaunchKernelGGL(ce_pair_kernel<CE_OPT_SMOOTH>, dim3((unsigned)a.T), dim3(CP_NT), 0, s, zb, a.labels, db,
                           a.row_loss, a.V, invT, o);
    } else if (fast) {
      if (a.shard_stats != nullptr)
        hipLaunchKernelGGL(ce_fast_kernel<true>, dim3((unsigned)a.T), dim3(CE_NT), 0, s, zb, a.labels, db,
                           a.row_loss, a.shard_stats, a.V, invT, S);
      else
        hipLaunchKernelGGL(ce_fast_kernel<false>, dim3((unsigned)a.T), dim3(CE_NT), 0, s, zb, a.labels, db,
                           a.row_loss, nullptr, a.V, invT, S);
    } else if (a.dtype == 1) {
      hipLaunchKernelGGL(ce_general_kernel<uint16_t>, dim3((unsigned)a.T), dim3(256), 0, s, zb, a.labels, db,
                         a.row_loss, a.shard_stats, a.V, a.parts, invT, a.opt, o);
    } else {
      hipLaunchKernelGGL(ce_general_kernel<float>, dim3((unsigned)a.T), dim3(256), 0, s,
                         static_cast<const float*>(a.logits), a.labels, static_cast<float*>(a.dlogits), a.row_loss,
                         a.shard_stats, a.V, a.parts, invT, a.opt, o);
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(loss_mean_kernel, dim3(1), dim3(1024), 0, s, a.row_loss, a.T,
                     a.opt ? static_cast<const int*>(a.count) : nullptr, a.loss);
  return hipGetLastError();
}

}  // namespace tpr
