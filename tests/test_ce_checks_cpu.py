"""The element-wise cross-entropy gradient check (ce_checks.py), on the CPU.

A gradient formed with the kernels' roundings (exponentials kept in fp16,
gradient rounded to bf16 at the end; fp32 throughout for fp32 logits) passes
it.  The same gradient with its softmax part permuted within each row, scaled
by 1.05, or zeroed fails it -- while all three pass the contract check
max |g - g_ref| <= 2e-2 max |g_ref| at the configured vocabulary, which is
why the GPU tests run both.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from ce_checks import grad_bound_ratio, target_rows
from oracle.ce_options import cross_entropy_opts


def contract_err(got, want):
    return float(np.abs(got - want).max() / np.abs(want).max())


def to_bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).double().numpy()


def kernel_like_grad(z, q, n, vv, out_dtype):
    """(p~ - q) / n with the GPU path's roundings: exp(z - m) kept in fp16
    (bf16 logits) or fp32, divided by the fp32-accurate row sum, the result
    rounded to the output dtype."""
    zv = z[:, :vv]
    m = zv.max(axis=1, keepdims=True)
    e = np.exp(zv - m)
    s = e.sum(axis=1, keepdims=True)
    kept = e.astype(np.float16).astype(np.float64) if out_dtype == "bf16" else e.astype(np.float32).astype(np.float64)
    g = np.zeros_like(z)
    g[:, :vv] = kept / s / n
    g -= q / n
    return to_bf16(g) if out_dtype == "bf16" else g.astype(np.float32).astype(np.float64)


@pytest.fixture(scope="module")
def full_vocab_rows():
    # Rows of the configured workload: bf16 logits ~ N(0, 2) over 128256
    # entries; the mean is over the configured 4096 positions.
    logits, labels = workloads.vocab_ce(T=6, V=128256, seed=11)
    z = logits.double().numpy()
    y = labels.numpy()
    _, _, g_ref = oracle.cross_entropy(z, y)
    T_full = 4096
    g_ref = g_ref * z.shape[0] / T_full
    q = target_rows(y, z.shape[1])
    return z, y, g_ref, q, T_full


def test_kernel_like_gradient_passes(full_vocab_rows):
    z, y, g_ref, q, n = full_vocab_rows
    g = kernel_like_grad(z, q, n, z.shape[1], "bf16")
    r, _ = grad_bound_ratio(g, g_ref, q, n, "bf16")
    assert r <= 1.0, r
    assert contract_err(g, g_ref) <= 2e-2


def test_softmax_part_is_below_the_contract_scale(full_vocab_rows):
    # the premise: every softmax term is below 2e-2 of the largest |g|
    z, y, g_ref, q, n = full_vocab_rows
    p = n * g_ref + q
    p[np.arange(len(y)), y] = 0.0
    assert (p / n).max() < 2e-2 * np.abs(g_ref).max()


@pytest.mark.parametrize("defect", ["permuted", "scaled_1.05", "zeroed"])
def test_softmax_defects_fail_elementwise_but_pass_the_contract(full_vocab_rows, defect):
    z, y, g_ref, q, n = full_vocab_rows
    g = kernel_like_grad(z, q, n, z.shape[1], "bf16")
    rng = np.random.default_rng(0)
    bad = g.copy()
    for t in range(len(y)):
        cols = np.delete(np.arange(z.shape[1]), y[t])
        if defect == "permuted":
            bad[t, cols] = g[t, rng.permutation(cols)]
        elif defect == "scaled_1.05":
            bad[t, cols] = to_bf16(g[t, cols] * 1.05)
        else:
            bad[t, cols] = 0.0
    assert contract_err(bad, g_ref) <= 2e-2            # the old check accepts it
    r, _ = grad_bound_ratio(bad, g_ref, q, n, "bf16")
    assert r > 1.0, (defect, r)                         # the element-wise check does not


def test_options_smoothing_padding_ignored_rows():
    # The measured options case: 128000 of 128256 columns, eps 0.1, ignored rows.
    T, V, vv, eps, ign = 8, 128256, 128000, 0.1, -100
    logits, labels = workloads.vocab_ce_opts(T, V, vv, seed=4, ignore_frac=0.3)
    z, y = logits.double().numpy(), labels.numpy()
    counted = y != ign
    _, _, g_ref, n = cross_entropy_opts(z, y, vv, ign, eps)
    q = target_rows(np.where(counted, y, 0), V, vv, eps, counted)
    g = kernel_like_grad(z, q, n, vv, "bf16")
    g[~counted] = 0.0
    r, _ = grad_bound_ratio(g, g_ref, q, n, "bf16")
    assert r <= 1.0, r
    bad = g.copy()
    k = np.nonzero(counted)[0][0]
    cols = np.delete(np.arange(vv), y[k])
    bad[k, cols] = to_bf16(g[k, cols] * 1.05)
    assert grad_bound_ratio(bad, g_ref, q, n, "bf16")[0] > 1.0


def test_fp32_logits():
    logits, labels = workloads.vocab_ce(T=4, V=40000, seed=5, dtype=torch.float32)
    z, y = logits.double().numpy(), labels.numpy()
    _, _, g_ref = oracle.cross_entropy(z, y)
    q = target_rows(y, z.shape[1])
    g = kernel_like_grad(z, q, len(y), z.shape[1], "f32")
    assert grad_bound_ratio(g, g_ref, q, len(y), "f32")[0] <= 1.0
    bad = g * (1 + 1e-4)
    assert grad_bound_ratio(bad, g_ref, q, len(y), "f32")[0] > 1.0
