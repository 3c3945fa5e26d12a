"""Pins for the oracle's vocabulary-parallel output head + cross-entropy (CPU only)."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def _inputs(T, d, V, seed, layout="math"):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((T, d))
    W = rng.standard_normal((d, V)) * 0.5
    y = rng.integers(0, V, size=T)
    return h, (W if layout == "math" else W.T.copy()), y


@pytest.mark.parametrize("layout", ["math", "torch"])
def test_head_against_torch_autograd(layout):
    # The unsharded definition against torch's own cross-entropy and autograd (fp64).
    h, w, y = _inputs(7, 5, 11, seed=1, layout=layout)
    ht = torch.tensor(h, requires_grad=True)
    wt = torch.tensor(w, requires_grad=True)
    logits = ht @ (wt if layout == "math" else wt.T)
    loss = F.cross_entropy(logits, torch.tensor(y))
    loss.backward()
    l, dh, dw = oracle.head_ce(h, w, y, layout)
    assert l == pytest.approx(loss.item(), rel=1e-13)
    np.testing.assert_allclose(dh, ht.grad.numpy(), rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_head_finite_differences():
    h, w, y = _inputs(3, 4, 6, seed=2)
    _, dh, dw = oracle.head_ce(h, w, y)
    eps = 1e-6
    for arr, grad in ((h, dh), (w, dw)):
        for idx in np.ndindex(arr.shape):
            keep = arr[idx]
            arr[idx] = keep + eps
            lp = oracle.head_ce(h, w, y)[0]
            arr[idx] = keep - eps
            lm = oracle.head_ce(h, w, y)[0]
            arr[idx] = keep
            assert (lp - lm) / (2 * eps) == pytest.approx(grad[idx], rel=1e-6, abs=1e-9)


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("V,parts", [(11, 1), (11, 2), (11, 3), (11, 7), (5, 7), (16, 4), (1, 3)])
def test_sharded_equals_unsharded(V, parts, layout):
    # The multi-card page's claim: the per-shard procedure (logits per shard,
    # combined statistics, dh summed over shards) reaches the unsharded result.
    h, w, y = _inputs(6, 4, V, seed=V * 10 + parts, layout=layout)
    l0, dh0, dw0 = oracle.head_ce(h, w, y, layout)
    l1, dh1, dw1 = oracle.vocab_parallel_head_ce(h, w, y, parts, layout)
    assert l1 == pytest.approx(l0, rel=1e-13)
    np.testing.assert_allclose(dh1, dh0, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dw1, dw0, rtol=1e-12, atol=1e-14)


def test_dh_needs_every_shard():
    # Leaving one shard's partial out of the sum changes dh (the sum across
    # the output shards is required); dW is untouched.
    h, w, y = _inputs(5, 3, 12, seed=4)
    _, dh0, dw0 = oracle.vocab_parallel_head_ce(h, w, y, 3)
    for r in range(3):
        _, dh1, dw1 = oracle.vocab_parallel_head_ce(h, w, y, 3, skip_rank=r)
        assert np.abs(dh1 - dh0).max() > 1e-3
        np.testing.assert_array_equal(dw1, dw0)


def test_zero_hidden_closed_form():
    # h = 0: every logit is 0, so the loss is log V, dW = h^T dlogits = 0 and
    # dh = (1/V - onehot)/T W^T.
    T, d, V = 4, 3, 9
    _, w, y = _inputs(T, d, V, seed=5)
    h = np.zeros((T, d))
    l, dh, dw = oracle.head_ce(h, w, y)
    assert l == pytest.approx(math.log(V), rel=1e-15)
    np.testing.assert_array_equal(dw, np.zeros_like(dw))
    g = np.full((T, V), 1.0 / V)
    g[np.arange(T), y] -= 1.0
    np.testing.assert_allclose(dh, (g / T) @ w.T, rtol=1e-14, atol=1e-16)


def test_layouts_are_transposes():
    h, w, y = _inputs(4, 5, 7, seed=6)
    l0, dh0, dw0 = oracle.head_ce(h, w, y, "math")
    l1, dh1, dw1 = oracle.head_ce(h, w.T.copy(), y, "torch")
    assert l1 == l0
    np.testing.assert_array_equal(dh1, dh0)
    np.testing.assert_array_equal(dw1, dw0.T)


def test_errors():
    h, w, y = _inputs(3, 4, 5, seed=7)
    with pytest.raises(ValueError, match="shape"):
        oracle.head_ce(h[:, :3], w, y)
    with pytest.raises(ValueError, match="layout"):
        oracle.head_ce(h, w, y, "other")
    with pytest.raises(ValueError, match="partition"):
        oracle.vocab_parallel_head_ce(h, w, y, 0)
    with pytest.raises(ValueError, match="label"):
        oracle.head_ce(h, w, np.array([0, 1, 5]))
