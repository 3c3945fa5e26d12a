"""Sharded matrix multiply forward and backward -- oracle (test infrastructure only).

Sharded GEMM page ("Sharded GEMM与Backprop：行、列、内维三种切分"):

* section "题意与假设": A is M x K, B is K x N, the upstream gradient G is M x N
  and the loss is the Frobenius inner product L = <G, AB>;
* section "解题路线", step 1: the unsharded gradients are dA = G B^T and
  dB = A^T G;
* step 2 (rows): A and G are split by rows; each rank computes Y_r = A_r B and
  dA_r = G_r B^T (stacked by rows) and a local dB_r = A_r^T G_r that must be
  summed over ranks, never concatenated;
* step 3 (columns): B and G are split by columns; Y_r = A B_r and
  dB_r = A^T G_r are stacked by columns and dA_r = G_r B_r^T is summed;
* step 4 (inner): A is split by columns and B by rows along K; the partial
  products A_r B_r are summed to form Y, and dA_r = G B_r^T, dB_r = A_r^T G are
  stacked along K;
* the reference code's contract raises ValueError('shape') for non-2-D
  operands or mismatched shapes and ValueError('partition') for a bad part
  count or axis name.

The split method reaches the unsharded products exactly (block-GEMM identity,
TP lesson page section 2.A, step 1), so ``matmul_grads`` -- the plain
definition -- is what the GPU path is compared with; ``sharded_matmul`` is the
literal per-rank simulation that the tests show equal to it.
"""

import numpy as np

from .sharding import shard_ranges

AXES = ("rows", "columns", "inner")


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def check_matmul_args(a, b, g, parts, axis):
    """Raise the sharded GEMM page's errors; return (M, K, N)."""
    a, b, g = (np.asarray(t) for t in (a, b, g))
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0] or g.shape != (a.shape[0], b.shape[1]):
        raise ValueError("shape")
    if type(parts) is not int or parts < 1 or axis not in AXES:
        raise ValueError("partition")
    return a.shape[0], a.shape[1], b.shape[1]


def matmul_grads(a, b, g):
    """Plain definition: Y = A B, dA = G B^T, dB = A^T G (all float64)."""
    a, b, g = _f64(a), _f64(b), _f64(g)
    if a.ndim != 2 or b.ndim != 2 or a.shape[1] != b.shape[0] or g.shape != (a.shape[0], b.shape[1]):
        raise ValueError("shape")
    return a @ b, g @ b.T, a.T @ g


def sharded_matmul_partials(a, b, g, parts, axis):
    """Per-rank pieces of the literal simulation.

    Returns a list, one entry per rank, of dicts with the rank's index range
    ``rng`` on the split dimension and its three local results ``y``, ``da``,
    ``db``.  Which of them are slices of the global result and which are
    partial sums depends on the axis (see the module docstring).
    """
    M, K, N = check_matmul_args(a, b, g, parts, axis)
    a, b, g = _f64(a), _f64(b), _f64(g)
    out = []
    if axis == "rows":
        for lo, hi in shard_ranges(M, parts):
            a_r, g_r = a[lo:hi, :], g[lo:hi, :]
            out.append(dict(rng=(lo, hi), y=a_r @ b, da=g_r @ b.T, db=a_r.T @ g_r))
    elif axis == "columns":
        for lo, hi in shard_ranges(N, parts):
            b_r, g_r = b[:, lo:hi], g[:, lo:hi]
            out.append(dict(rng=(lo, hi), y=a @ b_r, da=g_r @ b_r.T, db=a.T @ g_r))
    else:
        for lo, hi in shard_ranges(K, parts):
            a_r, b_r = a[:, lo:hi], b[lo:hi, :]
            out.append(dict(rng=(lo, hi), y=a_r @ b_r, da=g @ b_r.T, db=a_r.T @ g))
    return out


def sharded_matmul(a, b, g, parts, axis, skip_rank=None):
    """Literal simulation of ``parts`` ranks on one axis; returns (Y, dA, dB).

    Stacked results are assembled by writing each rank's slice; summed results
    start from a float64 zero accumulator and add every rank's partial (an
    empty rank adds nothing; an inner-axis rank with no K indices adds the
    zero M x N product).  ``skip_rank`` leaves one rank's partial out of the
    sums -- the page's warning that a missing forward sum loses the other
    shards' contribution -- and exists only for negative tests.
    """
    M, K, N = check_matmul_args(a, b, g, parts, axis)
    y = np.zeros((M, N))
    da = np.zeros((M, K))
    db = np.zeros((K, N))
    for r, p in enumerate(sharded_matmul_partials(a, b, g, parts, axis)):
        lo, hi = p["rng"]
        keep = r != skip_rank
        if axis == "rows":
            y[lo:hi, :] = p["y"]
            da[lo:hi, :] = p["da"]
            if keep:
                db += p["db"]
        elif axis == "columns":
            y[:, lo:hi] = p["y"]
            db[:, lo:hi] = p["db"]
            if keep:
                da += p["da"]
        else:
            da[:, lo:hi] = p["da"]
            db[lo:hi, :] = p["db"]
            if keep:
                y += p["y"]
    return y, da, db
