/*
 * tprank.h -- C ABI of libtprank: one tensor-parallel rank's hot path on an
 * AMD Instinct MI355X (gfx950), with every simulated rank computed on the one
 * GPU.
 *
 * Sources of the operations (page titles as printed, then the section):
 *   [GEMM]  "Sharded GEMM与Backprop：行、列、内维三种切分"
 *           sections 题意与假设 (assumptions) and 解题路线 (solution route)
 *   [CARDS] "多卡张量：拆开计算，再合回同一结果"
 *           sections 01 / COLUMN THEN ROW, 02 / BACKWARD, 04 / VOCABULARY SHARDS
 *           (and the output-head paragraph after section 04's tables)
 *   [TP]    "第 6 课：张量并行 TP"
 *           section 1 (column- and row-parallel linears) and 2.A (the MLP)
 *
 * Conventions shared by every entry point
 *   - Tensors are dense and row-major (C order); sizes are element counts.
 *   - Every data pointer is a DEVICE pointer owned by the caller; the library
 *     never allocates, frees or keeps a pointer after a call returns.
 *   - `ws` is a caller-owned device workspace of at least the size that the
 *     matching *_workspace_bytes() returns (NULL is allowed when that size is
 *     0).  Its contents on entry do not matter and are clobbered.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work is
 *     enqueued on it; calls return without waiting for the GPU.
 *   - dtype: TPR_F32 (inputs are float) or TPR_BF16 (inputs are bfloat16
 *     bit patterns stored as uint16).  Products accumulate in fp32.
 *   - Return value: TPR_OK or one of the TPR_ERR_* codes.  Every argument is
 *     validated on the host before anything is enqueued, so a non-zero
 *     status leaves every output untouched.  tprank_last_error() then holds
 *     a message (per thread).  TPR_ERR_HIP reports a failed launch.
 *   - Device pointers to bf16 data must be 2-byte aligned and to fp32 data
 *     4-byte aligned; 16-byte alignment (with row lengths that are multiples
 *     of 8) selects the vectorised kernels, anything else the element-wise
 *     ones.  Results do not depend on which is chosen beyond fp32 rounding
 *     order.
 *   - Two environment variables select fallback kernels on the same inputs
 *     (the tests use them to cover those kernels): TPRANK_GEMM_PATH=staged
 *     sends every bf16 product to the register-staged GEMM, and
 *     TPRANK_CE_STATS_PATH=onerow computes a requested shard_stats output
 *     with the one-row-per-workgroup CE kernel.
 */
#ifndef TPRANK_H
#define TPRANK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define TPR_OK 0
#define TPR_ERR_SHAPE 1      /* shape mismatch / negative size ([GEMM] reference code: ValueError('shape')) */
#define TPR_ERR_PARTITION 2  /* parts < 1, bad axis or rank ([GEMM] reference code: ValueError('partition')) */
#define TPR_ERR_DTYPE 3      /* unknown dtype or weight layout */
#define TPR_ERR_WORKSPACE 4  /* ws_bytes smaller than the *_workspace_bytes() value */
#define TPR_ERR_NULLPTR 5    /* a pointer that must be non-NULL is NULL */
#define TPR_ERR_HIP 6        /* a HIP launch failed */
#define TPR_ERR_VALUE 7      /* a scalar option outside its range */

/* ---- enumerations ------------------------------------------------------ */
#define TPR_ROWS 0     /* split M: A and G by rows        ([GEMM] 解题路线 step 2) */
#define TPR_COLUMNS 1  /* split N: B and G by columns     ([GEMM] 解题路线 step 3) */
#define TPR_INNER 2    /* split K: A by columns, B by rows ([GEMM] 解题路线 step 4) */

#define TPR_F32 0
#define TPR_BF16 1

#define TPR_W_MATH 0   /* w1 is d x f and w2 is f x d: y = gelu(x w1) w2      ([TP] 2.A) */
#define TPR_W_TORCH 1  /* w1 is (f, d) and w2 is (d, f): y = gelu(x w1^T) w2^T ([TP] 1, solution code) */

/* Element-wise activations of the MLP ([TP] 2.A names GeLU and SiLU; the
 * [CARDS] demo uses tanh, whose derivative 1 - H^2 its 02 / BACKWARD shows). */
#define TPR_ACT_GELU 0  /* x Phi(x), exact erf */
#define TPR_ACT_TANH 1  /* tanh(x) */
#define TPR_ACT_SILU 2  /* x / (1 + exp(-x)) */

/* ---- shard planning ----------------------------------------------------- */
/*
 * Half-open index range [*begin, *end) of shard `rank` when `n` indices are
 * split into `parts` contiguous shards.  [GEMM] 题意与假设 allows uneven and
 * empty shards; 手动走一遍 fixes the order (K=5 over 2 parts is 3 then 2):
 * every shard gets floor(n/parts) indices and the first n mod parts shards
 * one more.  Host-only, touches no device.
 * Errors: TPR_ERR_SHAPE if n < 0; TPR_ERR_PARTITION if parts < 1 or rank is
 * outside [0, parts); TPR_ERR_NULLPTR if begin or end is NULL.
 */
int tprank_shard_range(int64_t n, int parts, int rank, int64_t* begin, int64_t* end);

/* ---- sharded matrix multiply, forward and backward ------------------- */
/*
 * Bytes of workspace sharded_matmul_fwd_bwd() needs: one fp32 partial per
 * rank for the output that the chosen axis sums (dB for rows, dA for
 * columns, Y for inner), or 0 when parts == 1.  Returns 0 for invalid
 * arguments (the call itself then reports the error).
 */
size_t sharded_matmul_workspace_bytes(int axis, int parts, int dtype, int64_t M, int64_t K, int64_t N);

/*
 * [GEMM] 题意与假设 / 解题路线: with A (M x K), B (K x N) and the upstream
 * gradient G (M x N) of the loss L = <G, A B>, simulate `parts` ranks split
 * along `axis` and produce the full logical results
 *     Y = A B (M x N),  dA = G B^T (M x K),  dB = A^T G (K x N),
 * all fp32.  Each rank computes its local products with the bf16 (MFMA) or
 * fp32 GEMM kernels; outputs the axis stacks are written in place by each
 * rank (no concatenation kernel), outputs the axis sums are reduced from
 * per-rank fp32 partials in a fixed rank order (the simulated all-reduce).
 * Empty shards are skipped; an inner rank with no K indices contributes the
 * zero product.  Zero-size M, K or N are valid (outputs of zero size are not
 * touched; dA/dB/Y of non-zero size whose contraction is empty are zeroed).
 *   A, B, G: inputs in `dtype`; Y, dA, dB: fp32 outputs (may be NULL only if
 *   they have zero elements).
 * Errors: SHAPE (negative size), PARTITION (parts < 1 or unknown axis),
 * DTYPE, NULLPTR, WORKSPACE, HIP.
 */
int sharded_matmul_fwd_bwd(int axis, int parts, int dtype, int64_t M, int64_t K, int64_t N,
                           const void* A, const void* B, const void* G,
                           float* Y, float* dA, float* dB,
                           void* ws, size_t ws_bytes, void* stream);

/* ---- cross-rank partial sum -------------------------------------------- */
/*
 * The sum a split leaves behind, as the simulated all-reduce(sum) on one GPU:
 * [GEMM] 复杂度 and 解题路线 steps 2-4 (dB for a row split, dA for a column
 * split, Y for an inner split), [TP] 2.A step 5 and [CARDS] 02 / BACKWARD
 * (the MLP's y and dx).  The entry points above run it on their own
 * partials; this call exposes it on caller-provided ones:
 *     out[i] = partials[i] + partials[slot_stride + i] + ...
 *              + partials[(nslots - 1) * slot_stride + i],
 * added in slot (rank) order in fp32, so every call gives the same bits.
 *   partials: nslots fp32 slots of n elements, slot s at element offset
 *   s * slot_stride (slot_stride >= n);  out: n fp32 elements, not
 *   overlapping the partials.  n == 0 enqueues nothing; nslots == 0 writes
 *   zeros (the empty sum).  One HBM pass: (nslots + 1) * 4 bytes move per
 *   output element.
 * Errors: SHAPE (n < 0, nslots < 0 or slot_stride < n), NULLPTR (out, or
 * partials when nslots > 0, NULL with n > 0), VALUE (out overlaps the
 * partials), HIP.
 */
int tprank_partial_sum(int nslots, int64_t n, const float* partials, int64_t slot_stride, float* out,
                       void* stream);

/* ---- column-then-row tensor-parallel GELU MLP ------------------------- */
/*
 * Bytes of workspace tp_mlp_fwd_bwd() needs: gelu' of the pre-activation
 * and the activation (T x f each, in `dtype`; the first buffer is reused for
 * the gradient at the pre-activation), plus, when tp > 1, the tp full-shape
 * fp32 partials of y and of dx, plus (TPR_BF16, when gy W2^T fits in the
 * idle compute units of the forward launch's last round) that product and
 * the pre-activation, both in fp32 (T x f each).  Returns 0 for invalid
 * arguments.
 */
size_t tp_mlp_workspace_bytes(int tp, int dtype, int64_t T, int64_t d, int64_t f);

/*
 * [TP] 2.A and [CARDS] 01 / 02: `tp` ranks each own hidden columns [lo, hi)
 * of W1 (column-parallel) and the same rows of W2 (row-parallel).  Per rank,
 *   forward:  P_r = x W1_r;  H_r = gelu(P_r) (exact erf, fused in the GEMM
 *             epilogue, which also keeps gelu'(P_r) for the backward);
 *             Z_r = H_r W2_r, a full-shape T x d partial;
 *   backward (L = sum(y * gy), the same gy used once by every rank):
 *             dW2_r = H_r^T gy;  dZ_r = (gy W2_r^T) * gelu'(P_r) (fused);
 *             dW1_r = x^T dZ_r;  dx_r = dZ_r W1_r^T;
 * then y = sum_r Z_r and dx = sum_r dx_r (the MLP's one reduction each way,
 * fixed rank order).  For TPR_BF16, when the forward launch leaves enough
 * compute units idle, gy W2_r^T is computed alongside P_r (it does not
 * depend on it); both are kept in fp32 and one element-wise pass forms H_r
 * and dZ_r from them, each rounded once (no rounded gelu' in between).
 * With tp == 1 the call
 * computes one rank's share: pass
 * the rank's weight shards (w1 d x f_r, w2 f_r x d in TPR_W_MATH) and y, dx
 * are that rank's partials Z_r, dx_r.  For TPR_BF16 the activation and the
 * pre-activation gradient are rounded to bf16 (they are GEMM operands), and
 * so is the kept gelu'(P_r) of the fused-epilogue schedule.
 *   x, gy: T x d in `dtype` (leading dims of an activation flatten into T);
 *   w1, w2: weights in `dtype` and `w_layout`;
 *   y, dx: fp32 T x d;  dw1, dw2: fp32, same shapes/layout as w1, w2.
 * Errors: SHAPE, PARTITION (tp < 1), DTYPE (dtype or w_layout), NULLPTR,
 * WORKSPACE, HIP.
 */
int tp_mlp_fwd_bwd(int tp, int dtype, int w_layout, int64_t T, int64_t d, int64_t f,
                   const void* x, const void* w1, const void* w2, const void* gy,
                   float* y, float* dx, float* dw1, float* dw2,
                   void* ws, size_t ws_bytes, void* stream);

/* ---- MLP with another activation, or gated (gate / up) --------------- */
/*
 * Bytes of workspace tp_mlp_act_fwd_bwd() needs.  Plain (gated == 0): as
 * tp_mlp_workspace_bytes().  Gated: five T x f buffers in `dtype` (gate and
 * up pre-activations, H, and their gradients), a d x 2f copy of the gate and
 * up weights in `dtype` (each rank's columns side by side, so that its dx is
 * one product), and, when tp > 1, tp fp32 T x d partials of y and of dx.
 * 0 for invalid arguments.
 */
size_t tp_mlp_act_workspace_bytes(int tp, int dtype, int gated, int64_t T, int64_t d, int64_t f);

/*
 * [TP] 2.A (the element-wise activation sigma, e.g. GeLU or SiLU, applied
 * locally on each rank's column block) and its question 1 (gate and up
 * projections with the activation on the column-parallel side, the down
 * projection row-parallel); backward as [CARDS] 02 / BACKWARD.
 *   w3 == NULL: the MLP of tp_mlp_fwd_bwd() with sigma = `act` (TPR_ACT_*;
 *     sigma' of tanh is 1 - H^2, of SiLU s (1 + x (1 - s)), s the sigmoid).
 *   w3 != NULL (gated): rank r also owns columns [lo, hi) of the up
 *     projection W3 (same shape and layout as w1) and
 *       forward:  A_r = x W1_r;  U_r = x W3_r;  H_r = sigma(A_r) * U_r;
 *                 Z_r = H_r W2_r;
 *       backward: dH_r = gy W2_r^T;  dW2_r = H_r^T gy;
 *                 dA_r = dH_r * U_r * sigma'(A_r);  dU_r = dH_r * sigma(A_r);
 *                 dW1_r = x^T dA_r;  dW3_r = x^T dU_r;
 *                 dx_r = dA_r W1_r^T + dU_r W3_r^T;
 *     then y = sum_r Z_r and dx = sum_r dx_r in rank order.  For TPR_BF16
 *     A, U, H, dH, dA and dU are rounded to bf16.
 *   Arguments as tp_mlp_fwd_bwd(), plus act, w3 (NULL or like w1) and dw3
 *   (fp32 like w1; required when w3 is given).
 * Errors: SHAPE, PARTITION, DTYPE (dtype or w_layout), VALUE (unknown act),
 * NULLPTR, WORKSPACE, HIP.
 */
int tp_mlp_act_fwd_bwd(int tp, int dtype, int w_layout, int act, int64_t T, int64_t d, int64_t f,
                       const void* x, const void* w1, const void* w3, const void* w2, const void* gy,
                       float* y, float* dx, float* dw1, float* dw3, float* dw2,
                       void* ws, size_t ws_bytes, void* stream);

/* ---- attention-block projections -------------------------------------- */
/*
 * Bytes of workspace tp_attn_proj_fwd_bwd() needs: when tp > 1, the tp
 * full-shape fp32 partials of y and of dx (T x d each); 0 for tp == 1 and
 * for invalid arguments.
 */
size_t tp_attn_proj_workspace_bytes(int tp, int dtype, int64_t T, int64_t d, int n_q_heads, int n_kv_heads,
                                    int head_dim);

/*
 * [TP] 2.B (figure 6-2) and section 3's head-count constraints: the QKV
 * projection is column-parallel by heads, the output projection
 * row-parallel; the attention core between them is not computed here (its
 * forward output ctx and its input gradient dqkv are inputs).  With
 * nq = n_q_heads * head_dim and nkv = n_kv_heads * head_dim (grouped-query
 * attention when n_kv_heads < n_q_heads), rank r of `tp` owns
 * n_q_heads / tp query heads and n_kv_heads / tp KV heads:
 *   forward:  qkv_r = x W_qkv,r  (its column block of the fused projection),
 *             y = sum_r ctx_r W_o,r  (ctx_r: its heads' context columns,
 *             W_o,r: the matching rows of W_o);
 *   backward: dW_qkv,r = x^T dqkv_r;  dx = sum_r dqkv_r W_qkv,r^T;
 *             dctx_r = gy W_o,r^T;  dW_o,r = ctx_r^T gy;
 * y and dx summed in rank order (the block's one reduction each way).
 * Fused QKV column order: one contiguous block of (nq + 2 nkv) / tp columns
 * per rank, holding that rank's query heads, then its K heads, then its V
 * heads (head_dim columns per head); qkv and dqkv use the same order, ctx
 * and dctx the plain head order (nq columns).
 *   x, gy: T x d;  ctx: T x nq;  dqkv: T x (nq + 2 nkv), all in `dtype`;
 *   w_qkv: d x (nq + 2 nkv) for TPR_W_MATH or its transpose for
 *   TPR_W_TORCH;  w_o: nq x d (math) or d x nq (torch), in `dtype`;
 *   qkv: T x (nq + 2 nkv) and dctx: T x nq in `dtype` (the core's operands);
 *   y, dx: fp32 T x d;  dw_qkv, dw_o: fp32 like w_qkv, w_o.
 * Errors: SHAPE (n_q_heads not a multiple of n_kv_heads, head_dim < 1),
 * PARTITION (tp < 1, or tp not dividing both head counts: KV heads are not
 * replicated), DTYPE, NULLPTR, WORKSPACE, HIP.
 */
int tp_attn_proj_fwd_bwd(int tp, int dtype, int w_layout, int64_t T, int64_t d, int n_q_heads, int n_kv_heads,
                         int head_dim, const void* x, const void* w_qkv, const void* w_o, const void* ctx,
                         const void* gy, const void* dqkv, void* qkv, float* y, void* dctx, float* dx,
                         float* dw_qkv, float* dw_o, void* ws, size_t ws_bytes, void* stream);

/* ---- vocabulary-parallel cross-entropy -------------------------------- */
/*
 * Bytes of workspace vocab_parallel_ce_fwd_bwd() needs (the T per-row
 * losses, fp32).  Returns 0 for invalid arguments.
 */
size_t vocab_parallel_ce_workspace_bytes(int parts, int64_t T, int64_t V);

/*
 * [CARDS] 04 / VOCABULARY SHARDS, for T positions with logits z (T x V) and
 * targets y, the vocabulary split into `parts` contiguous shards V_r:
 *   m_r = max_{V_r} z,  m = max_r m_r,
 *   s_r = sum_{V_r} exp(z - m),  s = sum_r s_r,
 *   t_r = [y in V_r] (z_y - m),  L_i = log s - sum_r t_r,
 *   loss = (1/T) sum_i L_i  (mean over positions, no smoothing),
 *   dlogits_ij = (exp(z_ij - m_i)/s_i - [j = y_i]) / T.
 * One fused kernel keeps each row on chip: it reads the logits once and
 * writes dlogits once; the per-shard statistics are combined in a fixed
 * order.
 *   logits: T x V in `dtype`;  labels: T int64 with 0 <= y < V (not checked
 *   on the device; a label outside that range gives an unspecified loss and
 *   no target term, but no out-of-bounds access);
 *   loss: one fp32 on the device;  dlogits: T x V in `dtype`;
 *   shard_stats: NULL, or T x parts x 3 fp32 receiving (m_r, s_r, t_r)
 *   (m_r = -inf and s_r = 0 for an empty shard).
 * T == 0 writes loss = 0.  V must be >= 1 when T > 0.
 * Errors: SHAPE, PARTITION, DTYPE, NULLPTR, WORKSPACE, HIP.
 */
int vocab_parallel_ce_fwd_bwd(int parts, int dtype, int64_t T, int64_t V,
                              const void* logits, const int64_t* labels,
                              float* loss, void* dlogits, float* shard_stats,
                              void* ws, size_t ws_bytes, void* stream);

/*
 * The same call for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It takes no workspace: the per-row losses live in a static array inside
 * the library, 2^18 fp32 (1 MiB) per device, held until the process ends;
 * the call itself allocates nothing (its first call on a device only looks
 * up that array's address there).  Arguments, results and errors are those of
 * vocab_parallel_ce_fwd_bwd(), plus WORKSPACE when T > 2^18 (the array's
 * capacity).  Every call on one device shares that device's array, so calls
 * that overlap in time on one device (different streams, no ordering between
 * them) race and give undefined results; calls ordered on one stream do not.
 */
int vocab_parallel_ce_fwd_bwd_noalloc(int parts, int dtype, int64_t T, int64_t V,
                                      const void* logits, const int64_t* labels,
                                      float* loss, void* dlogits, float* shard_stats, void* stream);

/* ---- cross-entropy options: padded vocabulary, ignore index, smoothing - */
/*
 * Bytes of workspace vocab_parallel_ce_opts_fwd_bwd() needs (the T per-row
 * losses, fp32, and the counted-row total).  Returns 0 for invalid arguments.
 */
size_t vocab_parallel_ce_opts_workspace_bytes(int parts, int64_t T, int64_t V);

/*
 * [CARDS] 04 / VOCABULARY SHARDS, last paragraph: besides the plain loss a
 * real implementation handles vocabulary padding, an ignore index and label
 * smoothing, with the normalisation of an unsharded full-vocabulary
 * reference.  Same shards and statistics as vocab_parallel_ce_fwd_bwd(),
 * with these readings:
 *   - columns j >= v_valid of each row (1 <= v_valid <= V) are padding: they
 *     are not part of the softmax and their dlogits are 0;
 *   - a row whose label equals ignore_index adds no loss and gets a zero
 *     dlogits row; the mean is over the n counted rows (loss = NaN and all
 *     dlogits 0 when n = 0, the mean over no rows); pass a value no label
 *     takes (e.g. INT64_MIN) to count every row;
 *   - label smoothing eps in [0, 1]: a counted row's target distribution is
 *     q = (1 - eps) onehot(y) + eps / v_valid over the vocabulary columns,
 *     L_i = -sum_j q_j log p_j = log s - (1 - eps)(z_y - m) - eps (mean_j z_j - m),
 *     dlogits_ij = (p_ij - q_ij) / n.
 *   logits: T x V in `dtype`;  labels: T int64, each ignore_index or in
 *   [0, v_valid) (not checked on the device; another label gives an
 *   unspecified loss but no out-of-bounds access);  loss: one fp32 on the
 *   device;  dlogits: T x V in `dtype`;  shard_stats: NULL, or T x parts x 3
 *   fp32 (m_r, s_r, t_r) over each shard's vocabulary columns (m_r = -inf,
 *   s_r = 0 for a shard of padding only; t_r = 0 on ignored rows).
 * T == 0 writes loss = NaN.
 * Errors: SHAPE (also v_valid out of range), PARTITION, DTYPE, NULLPTR,
 * WORKSPACE, VALUE (eps outside [0, 1]), HIP.
 */
int vocab_parallel_ce_opts_fwd_bwd(int parts, int dtype, int64_t T, int64_t V, int64_t v_valid,
                                   int64_t ignore_index, float label_smoothing,
                                   const void* logits, const int64_t* labels,
                                   float* loss, void* dlogits, float* shard_stats,
                                   void* ws, size_t ws_bytes, void* stream);

/* ---- vocabulary-parallel output head with cross-entropy --------------- */
/*
 * Bytes of workspace vocab_parallel_head_ce_fwd_bwd() needs: the logits and
 * their gradient (T x V each, in `dtype`), the T per-row losses (fp32) and,
 * when parts > 1, the parts full-shape fp32 partials of dh (T x d).  Returns
 * 0 for invalid arguments.
 */
size_t vocab_parallel_head_ce_workspace_bytes(int parts, int dtype, int64_t T, int64_t d, int64_t V);

/*
 * [CARDS] 04 / VOCABULARY SHARDS and the paragraph after its tables: the
 * output head split by vocabulary columns.  Rank r holds the columns V_r of
 * the head matrix W (d x V) and computes
 *     logits_r = h W_r              (T x V_r, kept in `dtype`),
 * the ranks' cross-entropy statistics are combined exactly as in
 * vocab_parallel_ce_fwd_bwd() (mean over the T positions), then
 *     dW_r = h^T dlogits_r          (its columns of dW, in place),
 *     dh   = sum_r dlogits_r W_r^T  (the shared hidden state's gradient,
 *                                    summed across the shards in rank order).
 * For TPR_BF16 the logits and dlogits are rounded to bf16 (as the CE entry
 * point's inputs and outputs are); products accumulate in fp32.
 *   h: T x d in `dtype`;  w: the head in `dtype`, d x V for TPR_W_MATH or the
 *   (V, d) weight of a d -> V linear layer for TPR_W_TORCH;
 *   labels: T int64 with 0 <= y < V (same contract as the CE entry point);
 *   loss: one fp32 on the device;  dh: fp32 T x d;  dw: fp32, same shape and
 *   layout as w.  T == 0 writes loss = 0 and zeroes dw.
 *   On return the workspace holds the logits (T x V in `dtype`, row-major)
 *   from its first byte and dlogits (T x V in `dtype`) from the next
 *   multiple of 256 bytes after them; the caller may read both once the
 *   stream has completed the call.
 * Errors: SHAPE, PARTITION, DTYPE (dtype or w_layout), NULLPTR, WORKSPACE, HIP.
 */
int vocab_parallel_head_ce_fwd_bwd(int parts, int dtype, int w_layout, int64_t T, int64_t d, int64_t V,
                                   const void* h, const void* w, const int64_t* labels,
                                   float* loss, float* dh, float* dw,
                                   void* ws, size_t ws_bytes, void* stream);

/* Message for the last non-zero status returned on the calling thread. */
const char* tprank_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* TPRANK_H */
