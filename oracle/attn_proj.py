"""Tensor-parallel attention-block projections, forward and backward --
oracle (test infrastructure only).  The attention core between them (scores,
softmax, context) is not part of this: its output (the context) and its
input gradients (dQ, dK, dV) are given.

TP lesson page ("第 6 课：张量并行 TP"), section 2.B (the attention block,
figure 6-2) and section 3's architectural constraints:

* the QKV projection is column-parallel: W_Q, W_K, W_V are split along the
  output head dimension, each of `tp` ranks owning H/tp heads and computing
  its heads' Q, K, V from the replicated input X with no communication;
* the output projection W_O is row-parallel: split along its input (head)
  rows, each rank multiplies its local context by its rows, and one sum of
  the full-shape partials closes the block; the backward mirrors this (the
  input gradient is the one summed quantity);
* the head count must divide by tp; with grouped-query attention the KV head
  count must too (the page's Llama-3-8B example: 32 query and 8 KV heads give
  4 and 1 per rank at tp = 8, while tp = 16 leaves KV heads that cannot be
  divided, which needs replication -- out of scope here).

Readings: weights in the math layout are W_Q d x (Hq dh), W_K and W_V
d x (Hkv dh), W_O (Hq dh) x d; head h owns columns [h dh, (h+1) dh).  The
library takes the three QKV weights fused, with one contiguous column block
per rank holding that rank's Q heads, then its K heads, then its V heads
(``fuse_qkv``); QKV outputs and their gradients use the same column order.
Forward outputs Q, K, V (and backward dctx) are what the attention core
consumes; y and dx are the block's reduced outputs.
"""

import numpy as np

from .sharding import shard_ranges


def check_heads(tp, n_q_heads, n_kv_heads):
    """Heads per rank (q, kv), or ValueError('partition' / 'shape')."""
    if type(tp) is not int or tp < 1:
        raise ValueError("partition")
    if n_q_heads < 1 or n_kv_heads < 1 or n_q_heads % n_kv_heads:
        raise ValueError("shape")
    if n_q_heads % tp or n_kv_heads % tp:
        raise ValueError("partition")
    return n_q_heads // tp, n_kv_heads // tp


def fuse_qkv(wq, wk, wv, tp, n_q_heads, n_kv_heads, head_dim):
    """Math-layout Q, K, V weights (or any arrays with those column counts)
    -> one array whose rank-r column block is [Q heads of r | K heads of r |
    V heads of r]."""
    qh, kh = check_heads(tp, n_q_heads, n_kv_heads)
    blocks = []
    for r in range(tp):
        blocks.append(wq[:, r * qh * head_dim:(r + 1) * qh * head_dim])
        blocks.append(wk[:, r * kh * head_dim:(r + 1) * kh * head_dim])
        blocks.append(wv[:, r * kh * head_dim:(r + 1) * kh * head_dim])
    return np.concatenate(blocks, axis=1)


def split_qkv(fused, tp, n_q_heads, n_kv_heads, head_dim):
    """Inverse of ``fuse_qkv``: (Q part, K part, V part)."""
    qh, kh = check_heads(tp, n_q_heads, n_kv_heads)
    w = (qh + 2 * kh) * head_dim
    q, k, v = [], [], []
    for r in range(tp):
        b = fused[:, r * w:(r + 1) * w]
        q.append(b[:, :qh * head_dim])
        k.append(b[:, qh * head_dim:(qh + kh) * head_dim])
        v.append(b[:, (qh + kh) * head_dim:])
    return np.concatenate(q, axis=1), np.concatenate(k, axis=1), np.concatenate(v, axis=1)


def attn_proj_fwd_bwd(x, wq, wk, wv, wo, ctx, gy, dq, dk, dv):
    """Unsharded projections and their gradients (math layout, fp64).

    Forward: Q = X W_Q, K = X W_K, V = X W_V, y = ctx W_O.  Backward with the
    core's gradients dQ, dK, dV and the block's output gradient gy:
    dctx = gy W_O^T, dW_O = ctx^T gy, dW_Q = X^T dQ (likewise K, V),
    dX = dQ W_Q^T + dK W_K^T + dV W_V^T.
    Returns dict(q, k, v, y, dctx, dx, dwq, dwk, dwv, dwo).
    """
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, wq, wk, wv, wo, ctx, gy, dq, dk, dv = map(f, (x, wq, wk, wv, wo, ctx, gy, dq, dk, dv))
    if wo.shape[0] != wq.shape[1] or wo.shape[1] != x.shape[1] or ctx.shape != (x.shape[0], wq.shape[1]):
        raise ValueError("shape")
    return dict(q=x @ wq, k=x @ wk, v=x @ wv, y=ctx @ wo, dctx=gy @ wo.T, dx=dq @ wq.T + dk @ wk.T + dv @ wv.T,
                dwq=x.T @ dq, dwk=x.T @ dk, dwv=x.T @ dv, dwo=ctx.T @ gy)


def tp_attn_proj_fwd_bwd(x, wq, wk, wv, wo, ctx, gy, dq, dk, dv, tp, n_q_heads, n_kv_heads, head_dim):
    """Per-rank simulation: rank r owns Q heads [r qh, (r+1) qh) and KV heads
    [r kh, (r+1) kh) of the column-parallel projection and the matching rows
    of W_O; y and dx are the rank-order sums of the ranks' partials, every
    other output is the concatenation of the ranks' slices."""
    qh, kh = check_heads(tp, n_q_heads, n_kv_heads)
    f = lambda a: np.asarray(a, dtype=np.float64)
    x, wq, wk, wv, wo, ctx, gy, dq, dk, dv = map(f, (x, wq, wk, wv, wo, ctx, gy, dq, dk, dv))
    T, d = x.shape
    if wq.shape != (d, n_q_heads * head_dim) or wk.shape != (d, n_kv_heads * head_dim) or wv.shape != wk.shape:
        raise ValueError("shape")
    out = dict(q=np.zeros((T, wq.shape[1])), k=np.zeros((T, wk.shape[1])), v=np.zeros((T, wv.shape[1])),
               y=np.zeros((T, d)), dctx=np.zeros_like(ctx), dx=np.zeros((T, d)), dwq=np.zeros_like(wq),
               dwk=np.zeros_like(wk), dwv=np.zeros_like(wv), dwo=np.zeros_like(wo))
    qr = shard_ranges(n_q_heads * head_dim, tp)
    kr = shard_ranges(n_kv_heads * head_dim, tp)
    for r in range(tp):
        (q0, q1), (k0, k1) = qr[r], kr[r]
        assert q1 - q0 == qh * head_dim and k1 - k0 == kh * head_dim
        out["q"][:, q0:q1] = x @ wq[:, q0:q1]
        out["k"][:, k0:k1] = x @ wk[:, k0:k1]
        out["v"][:, k0:k1] = x @ wv[:, k0:k1]
        out["y"] += ctx[:, q0:q1] @ wo[q0:q1]
        out["dctx"][:, q0:q1] = gy @ wo[q0:q1].T
        out["dwo"][q0:q1] = ctx[:, q0:q1].T @ gy
        out["dwq"][:, q0:q1] = x.T @ dq[:, q0:q1]
        out["dwk"][:, k0:k1] = x.T @ dk[:, k0:k1]
        out["dwv"][:, k0:k1] = x.T @ dv[:, k0:k1]
        out["dx"] += dq[:, q0:q1] @ wq[:, q0:q1].T + dk[:, k0:k1] @ wk[:, k0:k1].T + dv[:, k0:k1] @ wv[:, k0:k1].T
    return out
