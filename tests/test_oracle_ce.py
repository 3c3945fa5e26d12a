"""Pins for the oracle's vocabulary-parallel cross-entropy (CPU only)."""
import json
import math
import os

import mpmath
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def demo_logits():
    return np.array(json.load(open(os.path.join(GOLDEN, "ce_demo.json")))["logits"])


def test_demo_logits_against_arbitrary_precision():
    # The page prints only the inputs; the expected values come from mpmath at
    # 50 digits (an independent evaluation of log-sum-exp and softmax).
    z = demo_logits()
    mpmath.mp.dps = 50
    ez = [mpmath.e ** mpmath.mpf(float(v)) for v in z]
    S = mpmath.fsum(ez)
    for y in range(6):
        for parts in range(1, 8):
            loss, row, grad, stats = oracle.vocab_parallel_ce(z[None, :], np.array([y]), parts)
            want = float(mpmath.log(S) - mpmath.mpf(float(z[y])))
            assert loss == pytest.approx(want, rel=1e-14)
            p = np.array([float(e / S) for e in ez])
            p[y] -= 1.0
            np.testing.assert_allclose(grad[0], p, rtol=1e-13, atol=1e-15)
        loss2, _, g2 = oracle.cross_entropy(z[None, :], np.array([y]))
        assert loss2 == pytest.approx(float(mpmath.log(S) - mpmath.mpf(float(z[y]))), rel=1e-14)


def test_demo_global_max_and_shard_stats():
    z = demo_logits()
    for parts in range(1, 8):
        _, _, _, st = oracle.vocab_parallel_ce(z[None, :], np.array([0]), parts)
        m_r, s_r, t_r = st[0, :, 0], st[0, :, 1], st[0, :, 2]
        for r, (lo, hi) in enumerate(oracle.shard_ranges(6, parts)):
            if hi > lo:
                assert m_r[r] == z[lo:hi].max()
                # s_r / s is the shard's probability mass (scipy softmax)
                assert s_r[r] / s_r.sum() == pytest.approx(scipy.special.softmax(z)[lo:hi].sum(), rel=1e-13)
            else:
                assert m_r[r] == -np.inf and s_r[r] == 0.0
        assert max(m_r) == 2.0
        # log s + m is the log-sum-exp of the row (scipy)
        assert math.log(s_r.sum()) + 2.0 == pytest.approx(scipy.special.logsumexp(z), rel=1e-15)
        # only the shard holding the target (index 0) has a target term, z_0 - m
        assert np.count_nonzero(t_r) == 1 and t_r[0] == pytest.approx(1.2 - 2.0, rel=1e-15)


def test_closed_form_log_integer_logits():
    # z_j = ln c_j makes softmax exactly c_j / sum(c) and the loss ln(sum c / c_y).
    c = np.array([1.0, 2.0, 3.0, 4.0, 10.0])
    z = np.log(c)
    for y in range(5):
        for parts in (1, 2, 3, 6):
            loss, _, grad, _ = oracle.vocab_parallel_ce(z[None, :], np.array([y]), parts)
            assert loss == pytest.approx(math.log(20.0 / c[y]), rel=1e-14)
            want = c / 20.0
            want[y] -= 1
            np.testing.assert_allclose(grad[0], want, atol=1e-15)


def test_uniform_logits_loss_is_log_vocab():
    for V in (1, 2, 7, 1000):
        loss, _, grad = oracle.cross_entropy(np.full((3, V), 0.37), np.zeros(3, dtype=np.int64))
        assert loss == pytest.approx(math.log(V), abs=1e-14)


def test_shift_invariance():
    # The section notes that a common shift of every logit changes neither the
    # loss nor the probabilities.
    rng = np.random.default_rng(0)
    z = rng.normal(0, 2, size=(5, 40))
    y = rng.integers(0, 40, size=5)
    base = oracle.vocab_parallel_ce(z, y, 3)
    for c in (-100.0, -3.5, 7.25, 500.0):
        sh = oracle.vocab_parallel_ce(z + c, y, 3)
        assert sh[0] == pytest.approx(base[0], rel=1e-12)
        np.testing.assert_allclose(sh[2], base[2], atol=1e-14)


def test_matches_torch_cross_entropy_mean_and_autograd():
    rng = np.random.default_rng(1)
    T, V = 33, 257
    z = rng.normal(0, 2, size=(T, V))
    y = rng.integers(0, V, size=T)
    tz = torch.tensor(z, requires_grad=True)
    L = F.cross_entropy(tz, torch.tensor(y), reduction="mean")
    L.backward()
    for parts in (1, 2, 5, 8, 300):
        loss, row, grad, _ = oracle.vocab_parallel_ce(z, y, parts)
        assert loss == pytest.approx(L.item(), rel=1e-13)
        np.testing.assert_allclose(grad, tz.grad.numpy(), rtol=1e-11, atol=1e-16)
    loss, row, grad = oracle.cross_entropy(z, y)
    assert loss == pytest.approx(L.item(), rel=1e-13)
    np.testing.assert_allclose(grad, tz.grad.numpy(), rtol=1e-11, atol=1e-16)
    np.testing.assert_allclose(row, F.cross_entropy(torch.tensor(z), torch.tensor(y), reduction="none").numpy(), rtol=1e-13)


def test_gradient_invariants_and_finite_differences():
    rng = np.random.default_rng(2)
    T, V = 4, 30
    z = rng.normal(0, 2, size=(T, V))
    y = rng.integers(0, V, size=T)
    loss, _, grad = oracle.cross_entropy(z, y)
    np.testing.assert_allclose(grad.sum(axis=1), 0.0, atol=1e-16)
    assert (grad >= -1.0 / T).all() and (grad <= 1.0 / T).all()
    h = 1e-6
    for t in range(T):
        for j in (0, 7, int(y[t]), V - 1):
            e = np.zeros_like(z); e[t, j] = h
            fd = (oracle.cross_entropy(z + e, y)[0] - oracle.cross_entropy(z - e, y)[0]) / (2 * h)
            assert abs(fd - grad[t, j]) < 1e-9


def test_sharded_equals_unsharded_all_part_counts():
    rng = np.random.default_rng(3)
    T, V = 6, 50
    z = rng.normal(0, 2, size=(T, V))
    y = rng.integers(0, V, size=T)
    want = oracle.cross_entropy(z, y)
    for parts in range(1, 60):
        got = oracle.vocab_parallel_ce(z, y, parts)
        assert got[0] == pytest.approx(want[0], rel=1e-13)
        np.testing.assert_allclose(got[1], want[1], rtol=1e-13)
        np.testing.assert_allclose(got[2], want[2], rtol=1e-12, atol=1e-17)


def test_grad_rows_subset_and_blocking():
    rng = np.random.default_rng(4)
    T, V = 150, 20   # spans several row blocks
    z = rng.normal(0, 2, size=(T, V))
    y = rng.integers(0, V, size=T)
    loss, row, grad = oracle.cross_entropy(z, y)
    rows = [149, 0, 63, 64, 65]
    loss2, row2, g2 = oracle.cross_entropy(z, y, grad_rows=rows)
    assert loss2 == loss
    np.testing.assert_array_equal(g2, grad[rows])
    assert grad.shape == (T, V)


def test_label_out_of_range_raises():
    with pytest.raises(ValueError, match="label"):
        oracle.cross_entropy(np.zeros((2, 5)), np.array([0, 5]))
    with pytest.raises(ValueError, match="label"):
        oracle.vocab_parallel_ce(np.zeros((2, 5)), np.array([-1, 0]), 2)
