"""Pins for the oracle's sharded matmul forward/backward (CPU only)."""
import itertools

import numpy as np
import pytest
import torch

import oracle


def brute(a, b, g):
    M, K = len(a), len(a[0])
    N = len(b[0])
    y = [[sum(a[i][k] * b[k][j] for k in range(K)) for j in range(N)] for i in range(M)]
    da = [[sum(g[i][j] * b[k][j] for j in range(N)) for k in range(K)] for i in range(M)]
    db = [[sum(a[i][k] * g[i][j] for i in range(M)) for j in range(N)] for k in range(K)]
    return np.array(y).reshape(M, N), np.array(da).reshape(M, K), np.array(db).reshape(K, N)


def rand(rng, *shape):
    return rng.uniform(-1, 1, size=shape)


@pytest.mark.parametrize("M,K,N", [(1, 1, 1), (3, 5, 4), (2, 6, 3), (6, 1, 5), (4, 4, 4)])
def test_definition_matches_brute_force(M, K, N):
    rng = np.random.default_rng(M * 100 + K * 10 + N)
    a, b, g = rand(rng, M, K), rand(rng, K, N), rand(rng, M, N)
    want = brute(a.tolist(), b.tolist(), g.tolist())
    got = oracle.matmul_grads(a, b, g)
    for w, o in zip(want, got):
        np.testing.assert_allclose(o, w, rtol=1e-13, atol=1e-13)


def test_definition_matches_autograd():
    # L = <G, A B>; torch autograd in float64 differentiates it independently.
    rng = np.random.default_rng(7)
    for M, K, N in [(3, 5, 4), (7, 2, 9), (1, 12, 1), (10, 10, 3)]:
        a, b, g = rand(rng, M, K), rand(rng, K, N), rand(rng, M, N)
        ta = torch.tensor(a, requires_grad=True)
        tb = torch.tensor(b, requires_grad=True)
        y = ta @ tb
        (y * torch.tensor(g)).sum().backward()
        oy, oda, odb = oracle.matmul_grads(a, b, g)
        np.testing.assert_allclose(oy, y.detach().numpy(), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(oda, ta.grad.numpy(), rtol=1e-13, atol=1e-14)
        np.testing.assert_allclose(odb, tb.grad.numpy(), rtol=1e-13, atol=1e-14)


def test_definition_matches_central_differences():
    # L is bilinear, so a central difference is exact up to rounding.
    rng = np.random.default_rng(3)
    a, b, g = rand(rng, 3, 5), rand(rng, 5, 4), rand(rng, 3, 4)
    _, da, db = oracle.matmul_grads(a, b, g)
    h = 1e-3
    L = lambda a_, b_: float((g * (a_ @ b_)).sum())
    for i, k in itertools.product(range(3), range(5)):
        e = np.zeros_like(a); e[i, k] = h
        assert abs((L(a + e, b) - L(a - e, b)) / (2 * h) - da[i, k]) < 1e-11
    for k, j in itertools.product(range(5), range(4)):
        e = np.zeros_like(b); e[k, j] = h
        assert abs((L(a, b + e) - L(a, b - e)) / (2 * h) - db[k, j]) < 1e-11


def test_sharded_equals_unsharded_1000_random_sizes():
    # Sharded GEMM page walk-through: 1000 random sizes on all three axes,
    # part counts above the dimension (empty shards) included.
    rng = np.random.default_rng(0)
    for _ in range(1000):
        M, K, N = (int(v) for v in rng.integers(1, 13, size=3))
        parts = int(rng.integers(1, 17))
        a, b, g = rand(rng, M, K), rand(rng, K, N), rand(rng, M, N)
        want = oracle.matmul_grads(a, b, g)
        for axis in oracle.AXES:
            got = oracle.sharded_matmul(a, b, g, parts, axis)
            for w, o in zip(want, got):
                assert o.shape == w.shape
                np.testing.assert_allclose(o, w, rtol=1e-12, atol=1e-12)


def test_walkthrough_shapes_all_axes_parts_2_and_7():
    rng = np.random.default_rng(0)
    a, b, g = rand(rng, 3, 5), rand(rng, 5, 4), rand(rng, 3, 4)
    want = oracle.matmul_grads(a, b, g)
    for parts, axis in itertools.product((2, 7), oracle.AXES):
        got = oracle.sharded_matmul(a, b, g, parts, axis)
        for w, o in zip(want, got):
            np.testing.assert_allclose(o, w, rtol=1e-12, atol=1e-12)
    pieces = oracle.sharded_matmul_partials(a, b, g, 2, "inner")
    assert [p["rng"] for p in pieces] == [(0, 3), (3, 5)]
    assert pieces[0]["da"].shape == (3, 3) and pieces[1]["db"].shape == (2, 4)


@pytest.mark.parametrize("axis,field", [("rows", 2), ("columns", 1), ("inner", 0)])
def test_dropping_one_partial_breaks_the_sum(axis, field):
    # The summed output of each axis (dB, dA, Y) needs every rank's partial.
    rng = np.random.default_rng(11)
    a, b, g = rand(rng, 6, 6, ), rand(rng, 6, 6), rand(rng, 6, 6)
    want = oracle.matmul_grads(a, b, g)
    for r in range(3):
        got = oracle.sharded_matmul(a, b, g, 3, axis, skip_rank=r)
        assert np.abs(got[field] - want[field]).max() > 1e-3
        for i in range(3):
            if i != field:
                np.testing.assert_allclose(got[i], want[i], rtol=1e-12, atol=1e-12)


def test_inner_empty_shard_contributes_zero():
    a, b, g = np.ones((2, 2)), np.ones((2, 3)), np.ones((2, 3))
    pieces = oracle.sharded_matmul_partials(a, b, g, 4, "inner")
    assert [p["rng"] for p in pieces] == [(0, 1), (1, 2), (2, 2), (2, 2)]
    assert pieces[3]["y"].shape == (2, 3) and not pieces[3]["y"].any()


@pytest.mark.parametrize("args", [
    (np.ones((2, 3)), np.ones((4, 2)), np.ones((2, 2))),   # K mismatch
    (np.ones((2, 3)), np.ones((3, 2)), np.ones((3, 2))),   # G shape
    (np.ones(3), np.ones((3, 2)), np.ones((1, 2))),        # ndim
])
def test_shape_errors(args):
    with pytest.raises(ValueError, match="shape"):
        oracle.sharded_matmul(*args, 2, "rows")


@pytest.mark.parametrize("parts,axis", [(0, "rows"), (2.0, "rows"), (2, "diag"), (-1, "inner")])
def test_partition_errors(parts, axis):
    with pytest.raises(ValueError, match="partition"):
        oracle.sharded_matmul(np.ones((2, 2)), np.ones((2, 2)), np.ones((2, 2)), parts, axis)
