"""Pins for the oracle's MLP with tanh / SiLU activations and the gated
(gate / up) form (CPU only)."""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle.mlp_act import ACTS, act, act_prime, mlp_act_fwd_bwd, tp_mlp_act_fwd_bwd

TORCH_ACT = {"gelu": F.gelu, "tanh": torch.tanh, "silu": F.silu}


def _inputs(T, d, f, seed, gated, layout="math"):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((d, f)) / np.sqrt(d)
    w3 = rng.standard_normal((d, f)) / np.sqrt(d) if gated else None
    w2 = rng.standard_normal((f, d)) / np.sqrt(f)
    gy = rng.standard_normal((T, d))
    if layout == "torch":
        w1, w2 = w1.T.copy(), w2.T.copy()
        w3 = None if w3 is None else w3.T.copy()
    return x, w1, w2, gy, w3


def _torch(x, w1, w2, gy, name, w3, layout):
    t = lambda a: torch.tensor(a, dtype=torch.float64, requires_grad=True)
    X, W1, W2 = t(x), t(w1), t(w2)
    W3 = None if w3 is None else t(w3)
    mm = (lambda a, w: a @ w) if layout == "math" else (lambda a, w: a @ w.T)
    H = TORCH_ACT[name](mm(X, W1))
    if W3 is not None:
        H = H * mm(X, W3)
    Y = mm(H, W2)
    (Y * torch.tensor(gy)).sum().backward()
    g = lambda a: None if a is None else a.grad.numpy()
    return Y.detach().numpy(), g(X), g(W1), g(W2), g(W3)


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("name", ACTS)
def test_against_torch_autograd(name, gated, layout):
    # torch's own GELU / tanh / SiLU and autograd on L = sum(Y * G).
    x, w1, w2, gy, w3 = _inputs(7, 6, 10, seed=4 * ACTS.index(name) + 2 * gated + (layout == "torch"), gated=gated, layout=layout)
    want = _torch(x, w1, w2, gy, name, w3, layout)
    for got in (mlp_act_fwd_bwd(x, w1, w2, gy, name, w3, layout),
                tp_mlp_act_fwd_bwd(x, w1, w2, gy, 3, name, w3, layout)):
        for g, w in zip(got, want):
            if w is None:
                assert g is None
            else:
                np.testing.assert_allclose(g, w, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("name", ACTS)
def test_activation_values_and_derivatives(name):
    x = np.linspace(-9.0, 9.0, 181)
    xt = torch.tensor(x, requires_grad=True)
    y = TORCH_ACT[name](xt)
    y.sum().backward()
    # (torch's erf-based GELU loses the far negative tail below 1e-15; the
    # oracle's erfc keeps it)
    np.testing.assert_allclose(act(name, x), y.detach().numpy(), rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(act_prime(name, x), xt.grad.numpy(), rtol=1e-12, atol=1e-15)


def test_closed_forms():
    assert act("silu", np.array([0.0]))[0] == 0.0 and act_prime("silu", np.array([0.0]))[0] == 0.5
    assert act_prime("tanh", np.array([0.0]))[0] == 1.0
    x = np.array([-50.0, -3.0, 0.5, 4.0, 60.0])
    np.testing.assert_allclose(act("silu", x), x * scipy.special.expit(x), rtol=1e-15)
    # tanh' is the page's 1 - H^2 with H = tanh
    np.testing.assert_allclose(act_prime("tanh", x), 1.0 - np.tanh(x) ** 2, rtol=0, atol=0)
    # GELU is the function of the plain MLP oracle
    np.testing.assert_array_equal(act("gelu", x), oracle.gelu(x))


@pytest.mark.parametrize("name", ACTS)
def test_finite_differences(name):
    x, w1, w2, gy, w3 = _inputs(3, 4, 5, seed=11, gated=True)
    got = mlp_act_fwd_bwd(x, w1, w2, gy, name, w3)
    loss = lambda xx, a, b, c: float((mlp_act_fwd_bwd(xx, a, b, gy, name, c)[0] * gy).sum())
    h = 1e-6
    args = [x, w1, w2, w3]
    grads = [got[1], got[2], got[3], got[4]]
    for i, (a, g) in enumerate(zip(args, grads)):
        for idx in [(0, 0), (1, 2), (a.shape[0] - 1, a.shape[1] - 1)]:
            p = [v.copy() for v in args]
            m = [v.copy() for v in args]
            p[i][idx] += h
            m[i][idx] -= h
            fd = (loss(*p) - loss(*m)) / (2 * h)
            assert fd == pytest.approx(g[idx], abs=1e-7, rel=1e-6)


@pytest.mark.parametrize("tp", [1, 2, 3, 4, 7, 13])
@pytest.mark.parametrize("gated", [False, True])
def test_sharded_equals_unsharded(tp, gated):
    # tp = 13 > f = 10 leaves ranks without columns.
    x, w1, w2, gy, w3 = _inputs(6, 8, 10, seed=tp, gated=gated)
    for name in ACTS:
        a = mlp_act_fwd_bwd(x, w1, w2, gy, name, w3)
        b = tp_mlp_act_fwd_bwd(x, w1, w2, gy, tp, name, w3)
        for u, v in zip(a, b):
            if u is None:
                assert v is None
            else:
                np.testing.assert_allclose(v, u, rtol=1e-12, atol=1e-14)


def test_gelu_equals_plain_mlp():
    x, w1, w2, gy, _ = _inputs(5, 6, 9, seed=3, gated=False)
    a = mlp_act_fwd_bwd(x, w1, w2, gy, "gelu")
    b = oracle.mlp_fwd_bwd(x, w1, w2, gy, "math")
    for u, v in zip(a[:4], b):
        np.testing.assert_allclose(u, v, rtol=1e-14, atol=1e-15)


def test_gate_with_unit_up_projection_is_plain():
    # If X W3 is all ones (x has a constant column of ones and W3 picks it),
    # the gated MLP is the plain one: same y, dx-through-W1, dW1, dW2.
    x, w1, w2, gy, _ = _inputs(6, 5, 7, seed=4, gated=False)
    x[:, 0] = 1.0
    w3 = np.zeros_like(w1)
    w3[0, :] = 1.0
    for name in ACTS:
        g = mlp_act_fwd_bwd(x, w1, w2, gy, name, w3)
        p = mlp_act_fwd_bwd(x, w1, w2, gy, name)
        np.testing.assert_allclose(g[0], p[0], rtol=1e-13)
        np.testing.assert_allclose(g[2], p[2], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(g[3], p[3], rtol=1e-13, atol=1e-15)
        # dx differs only in column 0, through the up projection
        np.testing.assert_allclose(g[1][:, 1:], p[1][:, 1:], rtol=1e-13, atol=1e-15)


def test_activation_before_the_sum_matters():
    # The activation acts on each rank's block; applying it to a sum of
    # partial pre-activations (a wrong split) gives another result.
    x, w1, w2, gy, _ = _inputs(4, 6, 8, seed=5, gated=False)
    for name in ("tanh", "silu"):
        y = mlp_act_fwd_bwd(x, w1, w2, gy, name)[0]
        wrong = act(name, x[:, :3] @ w1[:3] + 0) @ w2 + act(name, x[:, 3:] @ w1[3:]) @ w2
        assert np.abs(y - wrong).max() > 1e-3


def test_errors():
    x, w1, w2, gy, w3 = _inputs(3, 4, 5, seed=6, gated=True)
    with pytest.raises(ValueError, match="activation"):
        mlp_act_fwd_bwd(x, w1, w2, gy, "relu")
    with pytest.raises(ValueError, match="shape"):
        mlp_act_fwd_bwd(x, w1, w2, gy, "silu", w3[:, :4])
    with pytest.raises(ValueError, match="layout"):
        mlp_act_fwd_bwd(x, w1, w2, gy, "silu", w3, "other")
    with pytest.raises(ValueError, match="partition"):
        tp_mlp_act_fwd_bwd(x, w1, w2, gy, 0, "silu", w3)


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("layout", ["math", "torch"])
def test_sampled_matches_full(gated, layout):
    from oracle.mlp_act import mlp_act_sampled
    x, w1, w2, gy, w3 = _inputs(9, 7, 11, seed=12, gated=gated, layout=layout)
    rows, cols = np.array([0, 4, 8]), np.array([1, 5, 10])
    for name in ACTS:
        y, dx, dw1, dw2, dw3 = mlp_act_fwd_bwd(x, w1, w2, gy, name, w3, layout)
        s = mlp_act_sampled(x, w1, w2, gy, name, rows, cols, w3, layout)
        m = (lambda w: w) if layout == "math" else (lambda w: w.T)
        np.testing.assert_allclose(s["y"], y[rows], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(s["dx"], dx[rows], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(s["dw1_cols"], m(dw1)[:, cols], rtol=1e-13, atol=1e-15)
        np.testing.assert_allclose(s["dw2_rows"], m(dw2)[cols, :], rtol=1e-13, atol=1e-15)
        if gated:
            np.testing.assert_allclose(s["dw3_cols"], m(dw3)[:, cols], rtol=1e-13, atol=1e-15)
        else:
            assert "dw3_cols" not in s
