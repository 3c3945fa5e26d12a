"""Element-wise check of a cross-entropy gradient against the oracle's.

Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), 04 / VOCABULARY
SHARDS: the gradient of the mean loss is, per counted row,

    g_j = (p_j - q_j) / n,

with p the softmax over the vocabulary columns, q the target distribution
(one-hot, or (1 - eps) one-hot + eps / v_valid with label smoothing) and n the
number of counted rows.  The section's last paragraph asks that every case be
checked against the full-vocabulary reference's gradient.  A bound scaled by
max |g| cannot do that at a large vocabulary: there every p_j is far below 1
while the one-hot entry is 1, so the whole softmax part of a row sits below
2e-2 max |g| and could be zero, permuted or off by tens of percent unseen.
This check bounds every element on its own, from the arithmetic the kernels
perform.

Error model of a GPU gradient element:

    g_gpu = rnd( (p~ - q~) / n ),   p~ = p (1 + d) + a,   q~ = q (1 + d_q)

* rnd: round to nearest even in the output dtype, unit roundoff u_out
  (2^-8 for bf16, 2^-24 for fp32); 1/n and the scale factors are fp32, which
  adds 2^-22 relative to the rounded value.
* |d| <= r_p: bf16 logits -- the exponential exp(z - m') is kept in fp16
  between the sum pass and the gradient pass (unit roundoff 2^-11), plus
  2^-12 for the fp32 exponential, the fp32 row sum and the scale.  fp32
  logits -- exponentials and sums in fp32: the argument (z - m) log2(e) is
  rounded relative to |z| + |m|, which gives 2^-17 for the logit ranges of
  these tests (|z - m| below about 60).
* |a| <= a_p: bf16 logits -- an fp16 exponential below 2^-14 is subnormal
  with absolute spacing 2^-24, so its rounding error is at most 2^-25 before
  it is divided by s = 1 / max_j p_j; the exponent m' <= m of the part that
  was exponentiated against a partial maximum only shrinks it
  (exp(m' - m) <= 1).  Doubled: a_p = 2^-24 max_j p_j.  fp32: 2^-60 max p.
* |d_q| <= 2^-22: the smoothing share eps / (n v_valid) in fp32.

Hence, per element,

    n |g_gpu - g| <= (u_out + 2^-22) (|p - q| + r_p p + a_p) + r_p p + a_p
                     + 2^-22 q,

evaluated with the oracle's p and q.  With bf16 logits this is about 0.4 %
of |p - q| plus 0.07 % of p: a within-row permutation or a 5 % error of the
softmax part fails it (tests/test_ce_checks_cpu.py shows both on the CPU).
The target column keeps a bound of about 2^-8 of |p_y - 1|, what a bf16
gradient can hold there.
"""
import numpy as np

U_OUT = {"bf16": 2.0 ** -8, "f32": 2.0 ** -24}
R_P = {"bf16": 2.0 ** -11 + 2.0 ** -12, "f32": 2.0 ** -17}
A_P = {"bf16": 2.0 ** -24, "f32": 2.0 ** -60}
R_SCALE = 2.0 ** -22


def target_rows(labels, V, v_valid=None, eps=0.0, counted=None):
    """q per row (T x V fp64): the smoothed one-hot over the first v_valid
    columns; zero rows where ``counted`` is False."""
    labels = np.asarray(labels, dtype=np.int64)
    T = labels.shape[0]
    vv = V if v_valid is None else int(v_valid)
    q = np.zeros((T, V))
    c = np.ones(T, dtype=bool) if counted is None else np.asarray(counted, dtype=bool)
    q[c, :vv] = eps / vv
    rows = np.nonzero(c)[0]
    q[rows, labels[rows]] += 1.0 - eps
    return q


def grad_bound_ratio(g_gpu, g_ref, q, n, out_dtype):
    """Largest ratio of n |g_gpu - g_ref| to the per-element bound above
    (<= 1 passes), and the (row, column) where it occurs.

    ``g_gpu`` and ``g_ref`` are gradients of the same rows, T' x V (fp64);
    ``q`` the target distribution of those rows; ``n`` the mean's count.
    """
    g_gpu = np.asarray(g_gpu, dtype=np.float64)
    g_ref = np.asarray(g_ref, dtype=np.float64)
    assert g_gpu.shape == g_ref.shape == q.shape, (g_gpu.shape, g_ref.shape, q.shape)
    if g_ref.size == 0:
        return 0.0, (0, 0)
    p = n * g_ref + q
    np.maximum(p, 0.0, out=p)  # fp64 cancellation at the target can leave -1e-17
    a = A_P[out_dtype] * p.max(axis=1, keepdims=True)
    rp = R_P[out_dtype] * p
    bound = (U_OUT[out_dtype] + R_SCALE) * (np.abs(p - q) + rp + a) + rp + a + R_SCALE * q
    err = n * np.abs(g_gpu - g_ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(bound > 0, err / bound, np.where(err > 0, np.inf, 0.0))
    k = int(np.argmax(ratio))
    return float(ratio.flat[k]), np.unravel_index(k, ratio.shape)


def assert_grad_elementwise(g_gpu, g_ref, q, n, out_dtype, what=""):
    r, at = grad_bound_ratio(g_gpu, g_ref, q, n, out_dtype)
    assert r <= 1.0, (f"{what}: gradient element {tuple(int(i) for i in at)} off by {r:.3g} x its bound "
                      f"(gpu {np.asarray(g_gpu)[at]!r}, oracle {np.asarray(g_ref)[at]!r})")
    return r
