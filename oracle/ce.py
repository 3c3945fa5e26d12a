"""Vocabulary-parallel cross-entropy, forward and backward -- oracle
(test infrastructure only).

Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), section
"04 / VOCABULARY SHARDS": for one supervised position with logits z over a
vocabulary split into shards V_r and target y,

    m_r = max over V_r of z,            m = max over r of m_r,
    s_r = sum over V_r of exp(z - m),   s = sum over r of s_r,
    t_r = [y in V_r] (z_y - m),         L = log s - sum over r of t_r,
    dL/dz_j = exp(z_j - m) / s - [j = y].

The same section notes that shifting every logit by one constant changes
neither the loss nor the probabilities.  The workload applies this to T
positions and returns the mean loss, so each row's gradient carries a 1/T
factor (the gradient of the returned scalar); no label smoothing, no ignored
labels.

The shard procedure reaches the plain definition L = logsumexp(z) - z_y
exactly, so ``cross_entropy`` (the definition) is the parity oracle for loss
and gradient and ``vocab_parallel_ce`` is the literal per-shard procedure,
also used for the per-shard statistics (m_r, s_r, t_r).  Rows are processed in
blocks to bound host memory.
"""

import numpy as np

from .sharding import shard_ranges

_BLOCK = 64


def _check(logits, labels):
    logits = np.asarray(logits)
    labels = np.asarray(labels)
    if logits.ndim != 2 or labels.shape != (logits.shape[0],):
        raise ValueError("shape")
    V = logits.shape[1]
    if labels.size and (labels.min() < 0 or labels.max() >= V):
        raise ValueError("label")
    return logits, labels.astype(np.int64)


def cross_entropy(logits, labels, grad_rows=None):
    """Mean cross-entropy over rows, its per-row losses and its gradient.

    Returns (loss, row_loss[T], dlogits) where dlogits holds every row, or
    only ``grad_rows`` (in that order) when given.
    """
    logits, labels = _check(logits, labels)
    T, V = logits.shape
    row_loss = np.zeros(T)
    want = np.arange(T) if grad_rows is None else np.asarray(grad_rows, dtype=np.int64)
    pos = {int(t): i for i, t in enumerate(want)}
    grad = np.zeros((len(want), V))
    for lo in range(0, T, _BLOCK):
        hi = min(T, lo + _BLOCK)
        z = np.asarray(logits[lo:hi], dtype=np.float64)
        y = labels[lo:hi]
        m = z.max(axis=1, keepdims=True)
        e = np.exp(z - m)
        s = e.sum(axis=1, keepdims=True)
        idx = np.arange(hi - lo)
        row_loss[lo:hi] = np.log(s[:, 0]) + m[:, 0] - z[idx, y]
        for t in range(lo, hi):
            if t in pos:
                g = e[t - lo] / s[t - lo, 0]
                g[y[t - lo]] -= 1.0
                grad[pos[t]] = g / T
    loss = row_loss.mean() if T else 0.0
    return loss, row_loss, grad


def vocab_parallel_ce(logits, labels, parts):
    """Literal per-shard procedure; returns (loss, row_loss, dlogits, stats).

    ``stats`` is T x parts x 3 holding (m_r, s_r, t_r) per row and shard, with
    m_r = -inf and s_r = 0 for an empty shard.
    """
    if type(parts) is not int or parts < 1:
        raise ValueError("partition")
    logits, labels = _check(logits, labels)
    T, V = logits.shape
    ranges = shard_ranges(V, parts)
    stats = np.zeros((T, parts, 3))
    row_loss = np.zeros(T)
    grad = np.zeros((T, V))
    for t in range(T):
        z = np.asarray(logits[t], dtype=np.float64)
        y = int(labels[t])
        m_r = np.array([z[lo:hi].max() if hi > lo else -np.inf for lo, hi in ranges])
        m = m_r.max()
        s_r = np.array([np.exp(z[lo:hi] - m).sum() for lo, hi in ranges])
        t_r = np.array([(z[y] - m) if lo <= y < hi else 0.0 for lo, hi in ranges])
        s = s_r.sum()
        row_loss[t] = np.log(s) - t_r.sum()
        g = np.exp(z - m) / s
        g[y] -= 1.0
        grad[t] = g / T
        stats[t, :, 0], stats[t, :, 1], stats[t, :, 2] = m_r, s_r, t_r
    loss = row_loss.mean() if T else 0.0
    return loss, row_loss, grad, stats
