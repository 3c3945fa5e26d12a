"""Pins for the oracle's cross-entropy with vocabulary padding, ignored
positions and label smoothing (CPU only)."""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle.ce_options import cross_entropy_opts, vocab_parallel_ce_opts

IGN = -100


def _case(T, V, vv, seed, ignore_frac=0.25, scale=2.0):
    rng = np.random.default_rng(seed)
    z = scale * rng.standard_normal((T, V))
    y = rng.integers(0, vv, size=T)
    y[rng.random(T) < ignore_frac] = IGN
    return z, y


def _torch_ref(z, y, vv, eps):
    zt = torch.tensor(z[:, :vv], dtype=torch.float64, requires_grad=True)
    loss = F.cross_entropy(zt, torch.tensor(y), ignore_index=IGN, label_smoothing=eps)
    loss.backward()
    g = np.zeros_like(z)
    g[:, :vv] = zt.grad.numpy()
    return loss.item(), g


@pytest.mark.parametrize("eps", [0.0, 0.1, 0.5, 1.0])
@pytest.mark.parametrize("T,V,vv", [(9, 13, 13), (9, 16, 11), (6, 40, 37), (1, 8, 1)])
def test_against_torch_cross_entropy(T, V, vv, eps):
    # torch's cross_entropy (fp64) on the unpadded columns, with its own
    # ignore_index and label_smoothing: loss and autograd gradient.
    z, y = _case(T, V, vv, seed=T * 100 + V)
    if (y != IGN).sum() == 0:
        y[0] = 0
    want_l, want_g = _torch_ref(z, y, vv, eps)
    for fn in (lambda: cross_entropy_opts(z, y, vv, IGN, eps)[:3:2],
               lambda: vocab_parallel_ce_opts(z, y, 3, vv, IGN, eps)[:3:2]):
        loss, g = fn()
        assert loss == pytest.approx(want_l, rel=1e-13)
        np.testing.assert_allclose(g, want_g, rtol=1e-12, atol=1e-16)


def test_plain_case_reduces_to_plain_ce():
    # No padding, nothing ignored, eps = 0: the plain loss of the worked example.
    z, y = _case(7, 10, 10, seed=3, ignore_frac=0.0)
    l0, r0, g0 = oracle.cross_entropy(z, y)
    l1, r1, g1, n = cross_entropy_opts(z, y)
    assert n == 7 and l1 == pytest.approx(l0, rel=1e-14)
    np.testing.assert_allclose(g1, g0, rtol=1e-13, atol=1e-17)
    np.testing.assert_allclose(r1, scipy.special.logsumexp(z, axis=1) - z[np.arange(7), y], rtol=1e-13)


@pytest.mark.parametrize("eps", [0.0, 0.3, 1.0])
def test_uniform_logits_give_log_vocab(eps):
    # Equal logits: p is uniform over the vocabulary entries, so the loss is
    # log v_valid for any target distribution q.
    z = np.full((5, 12), 0.7)
    z[:, 9:] = 50.0  # padding must not count
    y = np.array([0, IGN, 8, 3, 1])
    for loss in (cross_entropy_opts(z, y, 9, IGN, eps)[0], vocab_parallel_ce_opts(z, y, 4, 9, IGN, eps)[0]):
        assert loss == pytest.approx(math.log(9), rel=1e-14)


def test_full_smoothing_closed_form():
    # eps = 1: q is uniform, the row loss is logsumexp(z) - mean(z).
    z, y = _case(6, 20, 17, seed=4)
    y[0] = 2
    c = y != IGN
    want = (scipy.special.logsumexp(z[:, :17], axis=1) - z[:, :17].mean(axis=1))[c].mean()
    assert cross_entropy_opts(z, y, 17, IGN, 1.0)[0] == pytest.approx(want, rel=1e-13)
    assert vocab_parallel_ce_opts(z, y, 5, 17, IGN, 1.0)[0] == pytest.approx(want, rel=1e-13)


def test_all_ignored_is_nan_with_zero_gradient():
    z, _ = _case(4, 9, 9, seed=5)
    y = np.full(4, IGN)
    for loss, g in (cross_entropy_opts(z, y, 9, IGN, 0.1)[:3:2], vocab_parallel_ce_opts(z, y, 2, 9, IGN, 0.1)[:3:2]):
        assert math.isnan(loss)
        assert not g.any()


def test_ignoring_a_row_equals_dropping_it():
    z, y = _case(8, 15, 15, seed=6, ignore_frac=0.0)
    y[[1, 4, 5]] = IGN
    keep = y != IGN
    l, rl, g, n = cross_entropy_opts(z, y, None, IGN, 0.2)
    l2, rl2, g2, n2 = cross_entropy_opts(z[keep], y[keep], None, None, 0.2)
    assert n == n2 == 5 and l == pytest.approx(l2, rel=1e-14)
    np.testing.assert_array_equal(g[~keep], 0.0)
    np.testing.assert_allclose(g[keep], g2, rtol=1e-14)
    np.testing.assert_array_equal(rl[~keep], 0.0)


def test_padding_values_do_not_matter():
    z, y = _case(5, 24, 19, seed=7)
    y[0] = 18
    l, _, g, _ = cross_entropy_opts(z, y, 19, IGN, 0.1)
    z2 = z.copy()
    z2[:, 19:] = np.array([1e30, -1e30, np.nan, 3.0, 0.0])
    for fn in (lambda zz: cross_entropy_opts(zz, y, 19, IGN, 0.1)[:3:2],
               lambda zz: vocab_parallel_ce_opts(zz, y, 6, 19, IGN, 0.1)[:3:2]):
        l2, g2 = fn(z2)
        assert l2 == pytest.approx(l, rel=1e-14)
        np.testing.assert_allclose(g2, g, rtol=1e-13, atol=1e-16)
        np.testing.assert_array_equal(g2[:, 19:], 0.0)


@pytest.mark.parametrize("parts", [1, 2, 3, 5, 8, 9, 30])
def test_sharded_equals_unsharded(parts):
    # Includes shards that hold only padding (parts 8, 9 on 24 columns of
    # which 14 are vocabulary) and empty shards (parts 30 > 24).
    z, y = _case(11, 24, 14, seed=parts)
    y[0] = 13
    l0, r0, g0, n0 = cross_entropy_opts(z, y, 14, IGN, 0.15)
    l1, r1, g1, st, n1 = vocab_parallel_ce_opts(z, y, parts, 14, IGN, 0.15)
    assert n0 == n1 and l1 == pytest.approx(l0, rel=1e-13)
    np.testing.assert_allclose(r1, r0, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(g1, g0, rtol=1e-12, atol=1e-17)
    for r, (lo, hi) in enumerate(oracle.shard_ranges(24, parts)):
        hi = min(hi, 14)
        if hi <= lo:
            assert np.all(st[:, r, 0] == -np.inf) and not st[:, r, 1].any()


def test_gradient_rows_sum_to_zero():
    z, y = _case(10, 30, 27, seed=9)
    y[0] = 1
    _, _, g, _ = cross_entropy_opts(z, y, 27, IGN, 0.25)
    np.testing.assert_allclose(g.sum(axis=1), 0.0, atol=1e-15)


def test_finite_differences():
    z, y = _case(4, 9, 7, seed=10, ignore_frac=0.0)
    y[2] = IGN
    _, _, g, _ = cross_entropy_opts(z, y, 7, IGN, 0.3)
    h = 1e-6
    for t in range(4):
        for j in range(9):
            zp, zm = z.copy(), z.copy()
            zp[t, j] += h
            zm[t, j] -= h
            fd = (cross_entropy_opts(zp, y, 7, IGN, 0.3)[0] - cross_entropy_opts(zm, y, 7, IGN, 0.3)[0]) / (2 * h)
            assert fd == pytest.approx(g[t, j], abs=1e-8)


def test_ignore_index_inside_the_vocabulary():
    # An ignore index may be a vocabulary id (a padding token): rows with it
    # are ignored, other rows may not use it as a target.
    z, _ = _case(4, 6, 6, seed=11)
    y = np.array([0, 3, 0, 5])
    l, _, g, n = cross_entropy_opts(z, y, None, 0, 0.0)
    assert n == 2
    want = (scipy.special.logsumexp(z[[1, 3]], axis=1) - z[[1, 3], [3, 5]]).mean()
    assert l == pytest.approx(want, rel=1e-14)
    assert not g[[0, 2]].any()


def test_errors():
    z, y = _case(3, 8, 6, seed=12, ignore_frac=0.0)
    with pytest.raises(ValueError, match="v_valid"):
        cross_entropy_opts(z, y, 9)
    with pytest.raises(ValueError, match="v_valid"):
        cross_entropy_opts(z, y, 0)
    with pytest.raises(ValueError, match="label_smoothing"):
        cross_entropy_opts(z, y, 6, IGN, 1.5)
    with pytest.raises(ValueError, match="label"):
        cross_entropy_opts(z, np.array([0, 6, 1]), 6)  # target in the padding
    with pytest.raises(ValueError, match="label"):
        cross_entropy_opts(z, np.array([0, -1, 1]), 6, IGN)
    with pytest.raises(ValueError, match="partition"):
        vocab_parallel_ce_opts(z, y, 0, 6)
