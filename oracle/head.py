"""Vocabulary-parallel output head with cross-entropy, forward and backward --
oracle (test infrastructure only).

Multi-card tensor page ("多卡张量：拆开计算，再合回同一结果"), section
"04 / VOCABULARY SHARDS" and the paragraph after its tables: the output head
is split by vocabulary columns, rank r holding W_r (the columns V_r of the
d x V head matrix W).  With hidden states h (T x d) shared by every rank,

    logits_r = h W_r                      (stays on rank r),
    cross-entropy over the shards          (section 04, see ``ce.py``),
    dW_r = h^T dlogits_r                   (stays on rank r),
    dh = sum over r of dlogits_r W_r^T     (the shared hidden state's gradient
                                            is summed across the output shards).

The loss is the mean over the T positions, so dlogits carries 1/T (as in
``ce.py``).  ``w_layout`` "math" takes W as d x V; "torch" takes the
nn.Linear(d, V) weight, V x d, whose transpose is W.

The shard procedure reaches the plain definition exactly (the column blocks
of h W are h W_r, and the sum over r of dlogits_r W_r^T is dlogits W^T), so
``head_ce`` (the definition) is the parity oracle and ``vocab_parallel_head_ce``
is the literal per-rank procedure kept beside it.
"""

import numpy as np

from .ce import cross_entropy, vocab_parallel_ce
from .sharding import shard_ranges


def _as_math(w, w_layout):
    if w_layout == "math":
        return w
    if w_layout == "torch":
        return w.T
    raise ValueError("layout")


def _check(h, w, labels, w_layout):
    h = np.asarray(h, dtype=np.float64)
    W = _as_math(np.asarray(w, dtype=np.float64), w_layout)
    labels = np.asarray(labels)
    if h.ndim != 2 or W.ndim != 2 or h.shape[1] != W.shape[0] or labels.shape != (h.shape[0],):
        raise ValueError("shape")
    return h, W, labels


def head_ce(h, w, labels, w_layout="math"):
    """Plain definition: returns (loss, dh, dw) with dw in ``w_layout``."""
    h, W, labels = _check(h, w, labels, w_layout)
    logits = h @ W
    loss, _, dlogits = cross_entropy(logits, labels)
    dh = dlogits @ W.T
    dW = h.T @ dlogits
    return loss, dh, (dW if w_layout == "math" else dW.T)


def vocab_parallel_head_ce(h, w, labels, parts, w_layout="math", skip_rank=None):
    """Literal per-rank procedure; returns (loss, dh, dw).

    Rank r computes its logits block, the shards combine their cross-entropy
    statistics (``vocab_parallel_ce``), rank r forms dW_r and its partial
    dh_r, and dh is the sum of the partials in rank order.  ``skip_rank``
    leaves one rank's partial out of that sum (tests use it to show the sum
    is needed).
    """
    if type(parts) is not int or parts < 1:
        raise ValueError("partition")
    h, W, labels = _check(h, w, labels, w_layout)
    T, d = h.shape
    V = W.shape[1]
    ranges = shard_ranges(V, parts)
    blocks = [h @ W[:, lo:hi] for lo, hi in ranges]
    logits = np.concatenate(blocks, axis=1) if blocks else np.zeros((T, 0))
    loss, _, dlogits, _ = vocab_parallel_ce(logits, labels, parts)
    dW = np.zeros((d, V))
    dh = np.zeros((T, d))
    for r, (lo, hi) in enumerate(ranges):
        dW[:, lo:hi] = h.T @ dlogits[:, lo:hi]
        if r != skip_rank:
            dh += dlogits[:, lo:hi] @ W[:, lo:hi].T
    return loss, dh, (dW if w_layout == "math" else dW.T)
