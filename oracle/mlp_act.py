"""Column-then-row tensor-parallel MLP with other activations and the gated
(gate / up) form, forward and backward -- oracle (test infrastructure only).

Sources:

* TP lesson page ("第 6 课：张量并行 TP"), section 2.A: Y = sigma(X W1) W2
  with an element-wise activation such as GeLU or SiLU applied to each rank's
  column block locally; its question 1 places the gate and up projections
  with the activation on the column-parallel side and the down projection on
  the row-parallel side.
* Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), section
  "02 / BACKWARD": G_H = G_Y W2_r^T, G_W2r = H_r^T G_Y, G_Z = G_H (.) sigma'
  (written there for tanh as 1 - H^2), G_W1r = X^T G_Z, G_X = sum_r G_Z W1_r^T.

Readings (the pages name the variants without formulas):

* activations: "gelu" is x Phi(x) (as in ``mlp.py``), "tanh" is tanh with
  sigma' = 1 - tanh^2 (the page's 1 - H^2), "silu" is x * s(x) with s the
  logistic sigmoid, sigma' = s (1 + x (1 - s));
* gated: a third weight W3 (the up projection, split by columns exactly like
  the gate W1) gives H = sigma(X W1) (.) (X W3); then G_A = G_H (.) (X W3)
  (.) sigma'(X W1), G_U = G_H (.) sigma(X W1), G_W1 = X^T G_A,
  G_W3 = X^T G_U and G_X = sum_r (G_A W1_r^T + G_U W3_r^T).

``mlp_act_fwd_bwd`` is the unsharded definition (the parity oracle);
``tp_mlp_act_fwd_bwd`` is the literal per-rank simulation.  Layouts as in
``mlp.py``: "math" has w1, w3 d x f and w2 f x d; "torch" has w1, w3 (f, d)
and w2 (d, f).  Returns (y, dx, dw1, dw2, dw3) with dw3 None when not gated.
"""

import numpy as np

from .mlp import gelu, gelu_prime, _tokens
from .sharding import shard_ranges

ACTS = ("gelu", "tanh", "silu")


def _sigmoid(x):
    # 1 / (1 + e^-x), written so that neither branch overflows.
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    ex = np.exp(x[~pos])
    out[~pos] = ex / (1.0 + ex)
    return out


def act(name, x):
    """The activation sigma(x)."""
    x = np.asarray(x, dtype=np.float64)
    if name == "gelu":
        return gelu(x)
    if name == "tanh":
        return np.tanh(x)
    if name == "silu":
        return x * _sigmoid(x)
    raise ValueError("activation")


def act_prime(name, x):
    """Its derivative sigma'(x)."""
    x = np.asarray(x, dtype=np.float64)
    if name == "gelu":
        return gelu_prime(x)
    if name == "tanh":
        return 1.0 - np.tanh(x) ** 2
    if name == "silu":
        s = _sigmoid(x)
        return s * (1.0 + x * (1.0 - s))
    raise ValueError("activation")


def _weights(w1, w2, w3, w_layout):
    w1 = np.asarray(w1, dtype=np.float64)
    w2 = np.asarray(w2, dtype=np.float64)
    w3 = None if w3 is None else np.asarray(w3, dtype=np.float64)
    if w_layout == "math":
        W1, W2, W3 = w1, w2, w3
    elif w_layout == "torch":
        W1, W2, W3 = w1.T, w2.T, None if w3 is None else w3.T
    else:
        raise ValueError("layout")
    if W1.ndim != 2 or W2.ndim != 2 or W1.shape[1] != W2.shape[0] or W1.shape[0] != W2.shape[1]:
        raise ValueError("shape")
    if W3 is not None and W3.shape != W1.shape:
        raise ValueError("shape")
    return W1, W2, W3


def _back(dw, w_layout):
    return None if dw is None else (dw if w_layout == "math" else dw.T)


def mlp_act_fwd_bwd(x, w1, w2, gy, act_name, w3=None, w_layout="math"):
    """Unsharded MLP (gated when w3 is given) and its gradients."""
    if act_name not in ACTS:
        raise ValueError("activation")
    W1, W2, W3 = _weights(w1, w2, w3, w_layout)
    d = W1.shape[0]
    X = _tokens(x, d)
    G = _tokens(gy, d)
    if G.shape != X.shape:
        raise ValueError("shape")
    A = X @ W1
    if W3 is None:
        H = act(act_name, A)
        dA = (G @ W2.T) * act_prime(act_name, A)
        dU = dW3 = None
        dX = dA @ W1.T
    else:
        U = X @ W3
        H = act(act_name, A) * U
        dH = G @ W2.T
        dA = dH * U * act_prime(act_name, A)
        dU = dH * act(act_name, A)
        dW3 = X.T @ dU
        dX = dA @ W1.T + dU @ W3.T
    Y = H @ W2
    dW2 = H.T @ G
    dW1 = X.T @ dA
    shape = np.shape(x)
    return (Y.reshape(shape), dX.reshape(shape), _back(dW1, w_layout), _back(dW2, w_layout), _back(dW3, w_layout))


def tp_mlp_act_fwd_bwd(x, w1, w2, gy, tp, act_name, w3=None, w_layout="math"):
    """Per-rank simulation: rank r holds columns f_r of W1 (and W3) and rows
    f_r of W2; y and dx are the rank-order sums of the ranks' partials."""
    if type(tp) is not int or tp < 1:
        raise ValueError("partition")
    if act_name not in ACTS:
        raise ValueError("activation")
    W1, W2, W3 = _weights(w1, w2, w3, w_layout)
    d, f = W1.shape
    X = _tokens(x, d)
    G = _tokens(gy, d)
    if G.shape != X.shape:
        raise ValueError("shape")
    Y = np.zeros_like(X)
    dX = np.zeros_like(X)
    dW1 = np.zeros_like(W1)
    dW2 = np.zeros_like(W2)
    dW3 = None if W3 is None else np.zeros_like(W3)
    for lo, hi in shard_ranges(f, tp):
        if hi == lo:
            continue
        A = X @ W1[:, lo:hi]
        dH = G @ W2[lo:hi].T
        if W3 is None:
            H = act(act_name, A)
            dA = dH * act_prime(act_name, A)
            dX_r = dA @ W1[:, lo:hi].T
        else:
            U = X @ W3[:, lo:hi]
            H = act(act_name, A) * U
            dA = dH * U * act_prime(act_name, A)
            dU = dH * act(act_name, A)
            dW3[:, lo:hi] = X.T @ dU
            dX_r = dA @ W1[:, lo:hi].T + dU @ W3[:, lo:hi].T
        Y += H @ W2[lo:hi]
        dX += dX_r
        dW1[:, lo:hi] = X.T @ dA
        dW2[lo:hi] = H.T @ G
    shape = np.shape(x)
    return (Y.reshape(shape), dX.reshape(shape), _back(dW1, w_layout), _back(dW2, w_layout), _back(dW3, w_layout))


def mlp_act_sampled(x, w1, w2, gy, act_name, rows, cols, w3=None, w_layout="math"):
    """Selected outputs of ``mlp_act_fwd_bwd`` computed one by one, for sizes
    too large for the full oracle.

    ``rows`` index tokens, ``cols`` index hidden units (0 <= c < f).  Returns
    a dict with y[rows], dx[rows], dw1_cols = dW1[:, cols], dw2_rows =
    dW2[cols, :] and (gated) dw3_cols = dW3[:, cols], in the math layout.
    """
    if act_name not in ACTS:
        raise ValueError("activation")
    W1, W2, W3 = _weights(w1, w2, w3, w_layout)
    d = W1.shape[0]
    X = _tokens(x, d)
    G = _tokens(gy, d)
    rows = np.asarray(rows, dtype=np.int64)
    cols = np.asarray(cols, dtype=np.int64)

    def block(Xs, Gs, c1, c2, c3):
        # A, (U), H and the two pre-activation gradients for tokens Xs and
        # hidden units given by the column blocks c1 (W1), c2 (W2 rows), c3 (W3)
        A = Xs @ c1
        dH = Gs @ c2.T
        if c3 is None:
            return act(act_name, A), dH * act_prime(act_name, A), None
        U = Xs @ c3
        return act(act_name, A) * U, dH * U * act_prime(act_name, A), dH * act(act_name, A)

    H, dA, dU = block(X[rows], G[rows], W1, W2, W3)
    out = dict(y=H @ W2, dx=dA @ W1.T + (0.0 if W3 is None else dU @ W3.T))
    Hc, dAc, dUc = block(X, G, W1[:, cols], W2[cols, :], None if W3 is None else W3[:, cols])
    out["dw1_cols"] = X.T @ dAc
    out["dw2_rows"] = Hc.T @ G
    if W3 is not None:
        out["dw3_cols"] = X.T @ dUc
    return out
