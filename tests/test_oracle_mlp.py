"""Pins for the oracle's GELU, MLP forward/backward and its TP simulation (CPU only)."""
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- GELU

def test_gelu_textbook_values():
    # Phi(1) and Phi(-1) from the normal CDF (scipy), GELU(0)=0, GELU'(0)=1/2.
    assert oracle.gelu(1.0) == pytest.approx(scipy.stats.norm.cdf(1.0), rel=1e-15)
    assert oracle.gelu(-1.0) == pytest.approx(-scipy.stats.norm.cdf(-1.0), rel=1e-14)
    assert oracle.gelu(0.0) == 0.0
    assert oracle.gelu_prime(0.0) == pytest.approx(0.5, rel=1e-15)


def test_gelu_matches_library_exact_gelu():
    x = np.linspace(-12, 12, 4001)
    # x * ndtr(x): scipy's normal CDF keeps relative precision in the tail.
    np.testing.assert_allclose(oracle.gelu(x), x * scipy.special.ndtr(x), rtol=1e-13, atol=0)
    # torch's exact GELU (absolute agreement; torch loses the far negative tail)
    want = F.gelu(torch.tensor(x), approximate="none").numpy()
    np.testing.assert_allclose(oracle.gelu(x), want, rtol=1e-13, atol=1e-15)


def test_gelu_odd_part_identity():
    # Phi(x) + Phi(-x) = 1 gives GELU(x) - GELU(-x) = x.
    x = np.linspace(-8, 8, 1001)
    np.testing.assert_allclose(oracle.gelu(x) - oracle.gelu(-x), x, rtol=0, atol=1e-14)


def test_gelu_prime_matches_autograd_and_differences():
    x = torch.linspace(-9, 9, 2001, dtype=torch.float64, requires_grad=True)
    F.gelu(x).sum().backward()
    np.testing.assert_allclose(oracle.gelu_prime(x.detach().numpy()), x.grad.numpy(), rtol=1e-13, atol=1e-15)
    xs = np.linspace(-6, 6, 241)
    h = 1e-5
    fd = (oracle.gelu(xs + h) - oracle.gelu(xs - h)) / (2 * h)
    np.testing.assert_allclose(oracle.gelu_prime(xs), fd, rtol=1e-8, atol=1e-9)


# ---------------------------------------------------------------- MLP

def _torch_mlp_grads(x, w1, w2, gy, layout):
    tx = torch.tensor(x, requires_grad=True)
    t1 = torch.tensor(w1, requires_grad=True)
    t2 = torch.tensor(w2, requires_grad=True)
    if layout == "math":
        y = F.gelu(tx @ t1) @ t2
    else:
        y = F.gelu(tx @ t1.T) @ t2.T
    (y * torch.tensor(gy)).sum().backward()
    return y.detach().numpy(), tx.grad.numpy(), t1.grad.numpy(), t2.grad.numpy()


@pytest.mark.parametrize("layout", ["math", "torch"])
def test_mlp_matches_torch_autograd(layout):
    rng = np.random.default_rng(5)
    T, d, f = 16, 12, 20
    x = rng.normal(size=(T, d))
    w1 = rng.normal(size=(d, f) if layout == "math" else (f, d)) * 0.5
    w2 = rng.normal(size=(f, d) if layout == "math" else (d, f)) * 0.5
    gy = rng.normal(size=(T, d))
    want = _torch_mlp_grads(x, w1, w2, gy, layout)
    got = oracle.mlp_fwd_bwd(x, w1, w2, gy, layout)
    for w, o in zip(want, got):
        assert o.shape == w.shape
        np.testing.assert_allclose(o, w, rtol=1e-12, atol=1e-12)


def test_mlp_demo_inputs_finite_differences():
    # Multi-card tensor page demo: X and G are printed, the weights are not;
    # every weight and input gradient is checked by finite differences.
    g = json.load(open(os.path.join(GOLDEN, "mlp_demo.json")))
    X, G = np.array(g["X"]), np.array(g["G"])
    rng = np.random.default_rng(2)
    W1, W2 = rng.normal(size=(2, 4)), rng.normal(size=(4, 2))
    y, dx, dw1, dw2 = oracle.mlp_fwd_bwd(X, W1, W2, G, "math")
    L = lambda x_, a_, b_: float((oracle.mlp_fwd_bwd(x_, a_, b_, G, "math")[0] * G).sum())
    h = 1e-6
    for arr, grad, which in [(X, dx, 0), (W1, dw1, 1), (W2, dw2, 2)]:
        for idx in np.ndindex(arr.shape):
            e = np.zeros_like(arr); e[idx] = h
            args_p = [X, W1, W2]; args_m = [X, W1, W2]
            args_p[which] = arr + e; args_m[which] = arr - e
            fd = (L(*args_p) - L(*args_m)) / (2 * h)
            assert abs(fd - grad[idx]) < 1e-7 * max(1.0, abs(fd))


@pytest.mark.parametrize("tp", [1, 2, 3, 4, 5, 7, 25])
@pytest.mark.parametrize("layout", ["math", "torch"])
def test_tp_simulation_equals_unsharded(tp, layout):
    # TP lesson page 2.A: column-then-row with one final sum equals the full MLP,
    # including uneven and (tp > f) empty shards.
    rng = np.random.default_rng(tp)
    T, d, f = 6, 8, 20
    x = rng.normal(size=(2, 3, d))
    w1 = rng.normal(size=(d, f) if layout == "math" else (f, d))
    w2 = rng.normal(size=(f, d) if layout == "math" else (d, f))
    gy = rng.normal(size=(2, 3, d))
    want = oracle.mlp_fwd_bwd(x, w1, w2, gy, layout)
    got = oracle.tp_mlp_fwd_bwd(x, w1, w2, gy, tp, layout)
    for w, o in zip(want, got):
        assert o.shape == w.shape
        np.testing.assert_allclose(o, w, rtol=1e-12, atol=1e-11)


def test_activation_before_sum_is_not_the_mlp():
    # Applying GELU to each partial and then summing is a different function.
    rng = np.random.default_rng(4)
    x = rng.normal(size=(4, 8))
    w1, w2 = rng.normal(size=(8, 12)), rng.normal(size=(12, 8))
    ranges = oracle.shard_ranges(8, 2)
    partial = [x[:, lo:hi] @ w1[lo:hi, :] for lo, hi in ranges]       # row-parallel first layer
    wrong = sum(oracle.gelu(p) for p in partial) @ w2
    right = oracle.gelu(sum(partial)) @ w2
    assert np.abs(wrong - right).max() > 1e-2
    np.testing.assert_allclose(right, oracle.mlp_fwd_bwd(x, w1, w2, np.zeros((4, 8)))[0], rtol=1e-12, atol=1e-12)


def test_partials_sum_and_shapes():
    rng = np.random.default_rng(9)
    x, w1, w2, gy = rng.normal(size=(5, 6)), rng.normal(size=(6, 10)), rng.normal(size=(10, 6)), rng.normal(size=(5, 6))
    y, dx, _, _, Zs, dXs = oracle.tp_mlp_fwd_bwd(x, w1, w2, gy, 4, "math", return_partials=True)
    assert len(Zs) == 4 and all(z.shape == (5, 6) for z in Zs)
    np.testing.assert_allclose(sum(Zs), y, rtol=1e-13, atol=1e-13)
    np.testing.assert_allclose(sum(dXs), dx, rtol=1e-13, atol=1e-13)
    # dropping one rank's partial loses its contribution
    assert np.abs(sum(Zs[1:]) - y).max() > 1e-3


def test_lesson_selftest_shapes_within_its_tolerances():
    # TP lesson self-test shapes, simulated in fp32 with torch: the oracle's
    # fp64 answer sits within the page's fp32 tolerances of an fp32 run.
    g = json.load(open(os.path.join(GOLDEN, "tp_lesson_selftest.json")))
    torch.manual_seed(0)
    x = torch.randn(*g["x"]); w1 = torch.randn(*g["w1"]); w2 = torch.randn(*g["w2"])
    y32 = F.gelu(x @ w1.T) @ w2.T
    y64 = oracle.mlp_fwd_bwd(x.numpy(), w1.numpy(), w2.numpy(), np.zeros(g["x"]), "torch")[0]
    tol = g["tp_mlp"]
    torch.testing.assert_close(torch.tensor(y64, dtype=torch.float32), y32, atol=tol["atol"], rtol=tol["rtol"])


@pytest.mark.parametrize("layout", ["math", "torch"])
def test_sampled_matches_full(layout):
    rng = np.random.default_rng(12)
    T, d, f = 9, 7, 11
    x = rng.normal(size=(T, d))
    w1 = rng.normal(size=(d, f) if layout == "math" else (f, d))
    w2 = rng.normal(size=(f, d) if layout == "math" else (d, f))
    gy = rng.normal(size=(T, d))
    y, dx, dw1, dw2 = oracle.mlp_fwd_bwd(x, w1, w2, gy, layout)
    if layout == "torch":
        dw1, dw2 = dw1.T, dw2.T
    rows, cols = [0, 4, 8, 4], [10, 0, 3]
    s = oracle.mlp_sampled(x, w1, w2, gy, rows, cols, layout)
    np.testing.assert_allclose(s["y"], y[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["dx"], dx[rows], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["dw1_cols"], dw1[:, cols], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(s["dw2_rows"], dw2[cols, :], rtol=1e-12, atol=1e-12)


def test_mlp_shape_errors():
    with pytest.raises(ValueError):
        oracle.mlp_fwd_bwd(np.ones((2, 3)), np.ones((4, 5)), np.ones((5, 4)), np.ones((2, 3)))
    with pytest.raises(ValueError, match="partition"):
        oracle.tp_mlp_fwd_bwd(np.ones((2, 3)), np.ones((3, 5)), np.ones((5, 3)), np.ones((2, 3)), 0)


def test_mlp_empty_feature_and_token_dims():
    # zero tokens, zero hidden units or zero features: shapes are kept and empty
    # contractions give exact zeros
    for T, d, f in ((0, 3, 4), (5, 3, 0), (5, 0, 4)):
        x, w1, w2, gy = np.ones((T, d)), np.ones((d, f)), np.ones((f, d)), np.ones((T, d))
        y, dx, dw1, dw2 = oracle.mlp_fwd_bwd(x, w1, w2, gy)
        assert y.shape == (T, d) and dx.shape == (T, d) and dw1.shape == (d, f) and dw2.shape == (f, d)
        for t in (y, dx, dw1, dw2):
            assert not t.any()
