"""Cross-entropy with a padded vocabulary, ignored positions and label
smoothing -- oracle (test infrastructure only).

Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), end of section
"04 / VOCABULARY SHARDS": the worked example is the plain loss; the page lists
vocabulary padding, an ignore index and label smoothing as what a real
implementation must also handle, and asks that every such edge be checked
against the loss, gradient and normalisation of an unsharded full-vocabulary
reference.  The readings taken here (the pages give no formulas for them):

* padding: the logits rows have V columns of which only the first ``v_valid``
  are vocabulary entries; the padding columns take no part in the softmax and
  receive a zero gradient, so a padded row gives exactly the unpadded result;
* ignore index: positions whose label equals ``ignore_index`` add no loss and
  get a zero gradient row, and the mean is over the n counted positions (for
  n = 0 the mean is 0/0: the loss is NaN and every gradient is zero);
* label smoothing eps: the target distribution of a counted row is
  q = (1 - eps) onehot(y) + eps / v_valid over the vocabulary entries, the
  row loss is the cross-entropy -sum_j q_j log p_j with p the softmax over the
  vocabulary entries, and dL/dz_j = (p_j - q_j) / n.

``cross_entropy_opts`` is that definition written out;
``vocab_parallel_ce_opts`` is the page's per-shard procedure (m_r, s_r, t_r)
extended by one more per-shard sum u_r (the sum of the shard's vocabulary
logits) that the smoothing term needs, combined across shards in rank order.
"""

import numpy as np

from .sharding import shard_ranges

_BLOCK = 64


def _check(logits, labels, v_valid, ignore_index, label_smoothing):
    logits = np.asarray(logits)
    labels = np.asarray(labels)
    if logits.ndim != 2 or labels.shape != (logits.shape[0],):
        raise ValueError("shape")
    V = logits.shape[1]
    vv = V if v_valid is None else int(v_valid)
    if vv < 1 or vv > V:
        raise ValueError("v_valid")
    eps = float(label_smoothing)
    if not 0.0 <= eps <= 1.0:
        raise ValueError("label_smoothing")
    labels = labels.astype(np.int64)
    counted = np.ones(labels.shape, dtype=bool) if ignore_index is None else labels != int(ignore_index)
    y = labels[counted]
    if y.size and (y.min() < 0 or y.max() >= vv):
        raise ValueError("label")
    return logits, labels, vv, counted, eps


def cross_entropy_opts(logits, labels, v_valid=None, ignore_index=None, label_smoothing=0.0, grad_rows=None):
    """The definition.  Returns (loss, row_loss[T], dlogits, n).

    row_loss is 0 for ignored rows; dlogits holds every row, or only
    ``grad_rows`` (in that order) when given.
    """
    logits, labels, vv, counted, eps = _check(logits, labels, v_valid, ignore_index, label_smoothing)
    T, V = logits.shape
    n = int(counted.sum())
    row_loss = np.zeros(T)
    want = np.arange(T) if grad_rows is None else np.asarray(grad_rows, dtype=np.int64)
    pos = {int(t): i for i, t in enumerate(want)}
    grad = np.zeros((len(want), V))
    for lo in range(0, T, _BLOCK):
        hi = min(T, lo + _BLOCK)
        z = np.asarray(logits[lo:hi, :vv], dtype=np.float64)
        zmax = z.max(axis=1, keepdims=True)
        logp = z - zmax - np.log(np.exp(z - zmax).sum(axis=1, keepdims=True))
        for t in range(lo, hi):
            if not counted[t]:
                continue
            q = np.full(vv, eps / vv)
            q[labels[t]] += 1.0 - eps
            row_loss[t] = -(q * logp[t - lo]).sum()
            if t in pos:
                grad[pos[t], :vv] = (np.exp(logp[t - lo]) - q) / n
    loss = row_loss.sum() / n if n else float("nan")
    return loss, row_loss, grad, n


def vocab_parallel_ce_opts(logits, labels, parts, v_valid=None, ignore_index=None, label_smoothing=0.0):
    """Per-shard procedure over ``parts`` shards of the padded width V.

    Returns (loss, row_loss, dlogits, stats, n); ``stats`` is T x parts x 3
    holding (m_r, s_r, t_r) over the vocabulary entries of each shard (m_r =
    -inf and s_r = 0 for a shard with none; t_r = 0 for an ignored row).
    """
    if type(parts) is not int or parts < 1:
        raise ValueError("partition")
    logits, labels, vv, counted, eps = _check(logits, labels, v_valid, ignore_index, label_smoothing)
    T, V = logits.shape
    ranges = [(lo, min(hi, vv)) for lo, hi in shard_ranges(V, parts)]
    n = int(counted.sum())
    stats = np.zeros((T, parts, 3))
    row_loss = np.zeros(T)
    grad = np.zeros((T, V))
    for t in range(T):
        z = np.asarray(logits[t], dtype=np.float64)
        y = int(labels[t])
        c = bool(counted[t])
        m_r = np.array([z[lo:hi].max() if hi > lo else -np.inf for lo, hi in ranges])
        m = m_r.max()
        s_r = np.array([np.exp(z[lo:hi] - m).sum() if hi > lo else 0.0 for lo, hi in ranges])
        t_r = np.array([(z[y] - m) if c and lo <= y < hi else 0.0 for lo, hi in ranges])
        u_r = np.array([z[lo:hi].sum() if hi > lo else 0.0 for lo, hi in ranges])
        stats[t, :, 0], stats[t, :, 1], stats[t, :, 2] = m_r, s_r, t_r
        if not c:
            continue
        s = s_r.sum()
        # -sum_j q_j (z_j - m - log s) with q = (1-eps) onehot + eps / vv
        row_loss[t] = np.log(s) - (1.0 - eps) * t_r.sum() - eps * (u_r.sum() / vv - m)
        for lo, hi in ranges:
            grad[t, lo:hi] = (np.exp(z[lo:hi] - m) / s - eps / vv) / n
        grad[t, y] -= (1.0 - eps) / n
    loss = row_loss.sum() / n if n else float("nan")
    return loss, row_loss, grad, stats, n
