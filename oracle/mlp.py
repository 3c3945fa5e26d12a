"""Column-then-row tensor-parallel GELU MLP, forward and backward -- oracle
(test infrastructure only).

Sources:

* TP lesson page ("第 6 课：张量并行 TP"), section 2.A: the unsharded MLP is
  Y = sigma(X W1) W2 with X tokens x d, W1 d x 4d, W2 4d x d; W1 is split by
  output columns (column-parallel, step 2), the element-wise activation is
  applied to each rank's block locally (step 3), W2 is split by input rows
  (row-parallel, step 4) and one sum of the full-shape partials Z_r closes the
  block (step 5).  Its solution code uses torch's default GELU (exact erf) and
  the torch weight layout (out, in), Y = X W^T; no bias anywhere.
* Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), section
  "02 / BACKWARD": per rank G_H = G_Y W2_r^T, G_W2r = H_r^T G_Y,
  G_Z = G_H (.) sigma'(.), G_W1r = X^T G_Z and G_X = sum_r G_Z W1_r^T; the one
  replicated upstream G_Y is used once by every rank and never summed.  Its
  loss is L = sum(Y (.) G).  That page's demo uses tanh (sigma' = 1 - H^2);
  here sigma is the exact-erf GELU, so sigma' is GELU'(pre-activation).

The split reaches the unsharded MLP exactly (block-GEMM identity), so
``mlp_fwd_bwd`` -- the plain unsharded definition -- is the parity oracle and
``tp_mlp_fwd_bwd`` is the literal per-rank simulation.  Weight layouts:
"math" means w1 is d x f and w2 is f x d (Y = X W); "torch" means w1 is (f, d)
and w2 is (d, f) (Y = X W^T).  Gradients come back in the layout of their
weights.  Leading dimensions of x are flattened into tokens; the feature axis
stays last (the sharded GEMM page warns that a reshape must not move the
shard axis).
"""

import math

import numpy as np
from scipy.special import erfc

from .sharding import shard_ranges

_SQRT2 = math.sqrt(2.0)
_INV_SQRT_2PI = 1.0 / math.sqrt(2.0 * math.pi)


def _phi_cdf(x):
    # Standard normal CDF, Phi(x) = (1 + erf(x/sqrt2))/2, written with erfc so
    # that the negative tail keeps its relative precision.
    return 0.5 * erfc(-x / _SQRT2)


def gelu(x):
    """Exact GELU: x * Phi(x) with Phi the standard normal CDF."""
    x = np.asarray(x, dtype=np.float64)
    return x * _phi_cdf(x)


def gelu_prime(x):
    """d/dx [x Phi(x)] = Phi(x) + x phi(x), phi the standard normal density."""
    x = np.asarray(x, dtype=np.float64)
    return _phi_cdf(x) + x * np.exp(-0.5 * x * x) * _INV_SQRT_2PI


def to_math_layout(w1, w2, w_layout):
    """Return (W1 d x f, W2 f x d) as float64 from either layout."""
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    if w_layout == "math":
        W1, W2 = w1, w2
    elif w_layout == "torch":
        W1, W2 = w1.T, w2.T
    else:
        raise ValueError("layout")
    if W1.ndim != 2 or W2.ndim != 2 or W1.shape[1] != W2.shape[0] or W1.shape[0] != W2.shape[1]:
        raise ValueError("shape")
    return W1, W2


def _tokens(x, d):
    x = np.asarray(x, dtype=np.float64)
    if x.ndim < 1 or x.shape[-1] != d:
        raise ValueError("shape")
    return x.reshape(int(np.prod(x.shape[:-1])), d)


def _from_math(dW1, dW2, w_layout):
    return (dW1, dW2) if w_layout == "math" else (dW1.T, dW2.T)


def mlp_fwd_bwd(x, w1, w2, gy, w_layout="math"):
    """Unsharded MLP and the gradients of L = sum(y (.) gy).

    Returns (y, dx, dw1, dw2); y and dx have x's shape, dw1/dw2 the weights'.
    """
    W1, W2 = to_math_layout(w1, w2, w_layout)
    d = W1.shape[0]
    X = _tokens(x, d)
    G = _tokens(gy, d)
    if G.shape != X.shape:
        raise ValueError("shape")
    pre = X @ W1                      # pre-activation, tokens x f
    H = gelu(pre)
    Y = H @ W2
    GH = G @ W2.T                     # gradient at the activation output
    dW2 = H.T @ G
    GZ = GH * gelu_prime(pre)         # gradient at the pre-activation
    dW1 = X.T @ GZ
    dX = GZ @ W1.T
    dW1, dW2 = _from_math(dW1, dW2, w_layout)
    shape = np.shape(x)
    return Y.reshape(shape), dX.reshape(shape), dW1, dW2


def tp_mlp_fwd_bwd(x, w1, w2, gy, tp, w_layout="math", return_partials=False):
    """Literal simulation of ``tp`` ranks of the column-then-row MLP.

    Rank r owns hidden columns [lo, hi) of W1 and the same rows of W2
    (uneven/empty shards follow the shard-range rule).  Forward: local
    pre-activation, local GELU, a full-shape partial Z_r; y = sum_r Z_r.
    Backward: every rank uses the same gy once; dW1 and dW2 are each rank's
    slice; dx = sum_r dx_r.  With ``return_partials`` also returns the lists
    of Z_r and dx_r.
    """
    if type(tp) is not int or tp < 1:
        raise ValueError("partition")
    W1, W2 = to_math_layout(w1, w2, w_layout)
    d, f = W1.shape
    X = _tokens(x, d)
    G = _tokens(gy, d)
    if G.shape != X.shape:
        raise ValueError("shape")
    T = X.shape[0]
    Y = np.zeros((T, d))
    dX = np.zeros((T, d))
    dW1 = np.zeros((d, f))
    dW2 = np.zeros((f, d))
    Zs, dXs = [], []
    for lo, hi in shard_ranges(f, tp):
        W1r, W2r = W1[:, lo:hi], W2[lo:hi, :]
        pre_r = X @ W1r
        H_r = gelu(pre_r)
        Z_r = H_r @ W2r
        GH_r = G @ W2r.T
        dW2[lo:hi, :] = H_r.T @ G
        GZ_r = GH_r * gelu_prime(pre_r)
        dW1[:, lo:hi] = X.T @ GZ_r
        dX_r = GZ_r @ W1r.T
        Y += Z_r
        dX += dX_r
        Zs.append(Z_r)
        dXs.append(dX_r)
    dW1, dW2 = _from_math(dW1, dW2, w_layout)
    shape = np.shape(x)
    out = (Y.reshape(shape), dX.reshape(shape), dW1, dW2)
    if return_partials:
        return out + (Zs, dXs)
    return out


def mlp_sampled(x, w1, w2, gy, rows, cols, w_layout="math"):
    """Selected outputs of ``mlp_fwd_bwd`` computed one by one, for sizes too
    large for the full oracle.

    ``rows`` index tokens, ``cols`` index hidden units (0 <= c < f).  Returns a
    dict with y[rows], dx[rows] (tokens x d), dw1_cols = dW1[:, cols] (d x len)
    and dw2_rows = dW2[cols, :] (len x d), both in the math layout.
    """
    W1, W2 = to_math_layout(w1, w2, w_layout)
    d = W1.shape[0]
    X = _tokens(x, d)
    G = _tokens(gy, d)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)
    # token rows: y[t] = gelu(x[t] W1) W2 ; dx[t] = ((g[t] W2^T) (.) gelu'(x[t] W1)) W1^T
    pre_rows = X[rows] @ W1
    y_rows = gelu(pre_rows) @ W2
    dx_rows = ((G[rows] @ W2.T) * gelu_prime(pre_rows)) @ W1.T
    # hidden units: need the whole token column of the pre-activation
    pre_cols = X @ W1[:, cols]                 # T x len
    H_cols = gelu(pre_cols)
    GZ_cols = (G @ W2[cols, :].T) * gelu_prime(pre_cols)
    dw1_cols = X.T @ GZ_cols                   # d x len
    dw2_rows = H_cols.T @ G                    # len x d
    return dict(y=y_rows, dx=dx_rows, dw1_cols=dw1_cols, dw2_rows=dw2_rows)
