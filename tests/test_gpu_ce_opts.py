"""GPU parity of the cross-entropy options (vocabulary padding, ignored
positions, label smoothing) through the C ABI, against the fp64 oracle.

Same tolerances as the plain cross-entropy: the loss within 1e-5 relative,
dlogits within 1e-5 (fp32 logits) or 2e-2 (bf16 logits) of max |oracle| and
element by element against the oracle's (p - q) / n (ce_checks.py), padding
columns and ignored rows exactly zero, maxima exact.
"""
import math
import sys

import numpy as np
import pytest
import torch

import workloads
from ce_checks import assert_grad_elementwise, target_rows
from oracle.ce_options import cross_entropy_opts, vocab_parallel_ce_opts

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
IGN = -100


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, want):
    scale = float(np.abs(want).max()) if want.size else 0.0
    diff = float(np.abs(got - want).max()) if want.size else 0.0
    return diff / scale if scale > 0 else diff


def tol_of(dtype):
    return 1e-5 if dtype == torch.float32 else 2e-2


@pytest.fixture(scope="module")
def tpr():
    import megatron_mlp_fwd_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


def check(tpr, logits, labels, parts, vv, ign, eps, stats=False):
    loss, dl, st = tpr.vocab_parallel_ce_opts_fwd_bwd(parts, logits, labels, v_valid=vv, ignore_index=ign,
                                                      label_smoothing=eps, shard_stats=stats)
    torch.cuda.synchronize()
    z, y = f64(logits), labels.cpu().numpy()
    wl, _, wg, wst, n = vocab_parallel_ce_opts(z, y, parts, vv, ign, eps)
    tol = tol_of(logits.dtype)
    if n == 0:
        assert math.isnan(loss.item())
    else:
        assert abs(loss.item() - wl) <= 1e-5 * abs(wl) + 1e-6, (loss.item(), wl)
    g = f64(dl)
    assert rel_err(g, wg) <= tol
    V = logits.shape[1]
    counted = np.ones(len(y), dtype=bool) if ign is None else y != ign
    q = target_rows(np.where(counted, y, 0), V, vv, eps, counted)
    assert_grad_elementwise(g, wg, q, max(n, 1), "f32" if logits.dtype == torch.float32 else "bf16", "dlogits")
    assert not g[:, vv:].any()                              # padding columns
    if ign is not None:
        assert not g[y == ign].any()                        # ignored rows
    if stats:
        gst = f64(st)
        np.testing.assert_array_equal(gst[:, :, 0], wst[:, :, 0])
        np.testing.assert_allclose(gst[:, :, 1], wst[:, :, 1], rtol=1e-5, atol=1e-30)
        np.testing.assert_allclose(gst[:, :, 2], wst[:, :, 2], rtol=1e-6, atol=1e-6)
    return loss, dl


@pytest.mark.parametrize("parts", [1, 3, 8])
@pytest.mark.parametrize("eps", [0.0, 0.1, 1.0])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,V,vv", [(37, 1000, 1000), (37, 1000, 997), (16, 4104, 4099), (5, 24, 17), (9, 8, 1),
                                    (6, 40000, 39993)])
def test_ce_opts_small(tpr, T, V, vv, dtype, eps, parts):
    say("CE options", T, V, vv, dtype, eps, parts)
    logits, labels = workloads.vocab_ce_opts(T, V, vv, seed=T + V + parts, device=DEV, dtype=dtype, ignore_frac=0.25)
    labels[0] = vv - 1  # a target in the last vocabulary column (the partial vector when vv % 8 != 0)
    check(tpr, logits, labels, parts, vv, IGN, eps)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("parts", [1, 5, 8])
def test_ce_opts_shard_stats(tpr, dtype, parts):
    say("CE options with shard statistics", dtype, parts)
    T, V, vv = 11, 2048, 1500   # shards 5..7 of 8 hold only padding
    logits, labels = workloads.vocab_ce_opts(T, V, vv, seed=parts, device=DEV, dtype=dtype, ignore_frac=0.3)
    check(tpr, logits, labels, parts, vv, IGN, 0.2, stats=True)


# Paired kernel: vocabulary vectors split between registers (22 x 512) and
# LDS (up to 4864), with the partial last vector and whole padding vectors.
@pytest.mark.parametrize("V,pad", [(8 * 11264, 3), (8 * 11264 + 8, 1), (8 * 11265, 8), (8 * 11364, 11),
                                   (8 * (11264 + 4864), 7), (8 * (11264 + 4864), 64)])
def test_ce_opts_row_split_edges(tpr, V, pad):
    say("CE options bf16 row split, V =", V, "padding", pad)
    T, vv = 6, V - pad
    logits, labels = workloads.vocab_ce_opts(T, V, vv, seed=V + pad, device=DEV)
    labels[0] = vv - 1
    labels[1] = 0
    labels[2] = IGN
    labels[3] = (vv // 8) * 8 - 1   # last column of the last whole vector
    check(tpr, logits, labels, 4, vv, IGN, 0.1)


def test_ce_opts_all_ignored(tpr):
    for dtype in (torch.bfloat16, torch.float32):
        say("CE options, every row ignored", dtype)
        logits, labels = workloads.vocab_ce_opts(4, 64, 60, seed=1, device=DEV, dtype=dtype)
        labels[:] = IGN
        loss, dl = check(tpr, logits, labels, 2, 60, IGN, 0.1)
        assert math.isnan(loss.item()) and not dl.any()


def test_ce_opts_ignore_index_in_vocabulary(tpr):
    say("CE options, ignore_index = 0")
    logits, labels = workloads.vocab_ce_opts(20, 1024, 1024, seed=2, device=DEV, ignore_frac=0.0)
    labels[::3] = 0
    check(tpr, logits, labels, 8, 1024, 0, 0.0)


def test_ce_opts_without_options_matches_plain(tpr):
    say("CE options off == plain CE")
    logits, labels = workloads.vocab_ce(T=64, V=128256, seed=3, device=DEV)
    a = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels)
    b = tpr.vocab_parallel_ce_opts_fwd_bwd(8, logits, labels, ignore_index=None)
    torch.cuda.synchronize()
    assert abs(a[0].item() - b[0].item()) <= 1e-6 * abs(a[0].item())
    assert torch.equal(a[1], b[1])


def test_ce_opts_zero_rows(tpr):
    say("CE options T=0")
    logits = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    labels = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, dl, _ = tpr.vocab_parallel_ce_opts_fwd_bwd(2, logits, labels, v_valid=12)
    torch.cuda.synchronize()
    assert math.isnan(loss.item()) and dl.shape == (0, 16)


def test_ce_opts_full_config(tpr):
    # The measured case: 4096 x 128256 bf16 logits of a 128000-entry
    # vocabulary, 8 shards, label smoothing 0.1, one position in eight
    # ignored; every row against the oracle, in row blocks.
    say("CE options 4096 x 128256 (128000 vocabulary), eps 0.1, 1/8 ignored, every row")
    T, V, vv, P, eps = 4096, 128256, 128000, 8, 0.1
    logits, labels = workloads.vocab_ce_opts(T, V, vv, seed=0, device=DEV)
    out = (torch.empty((), device=DEV), torch.full((T, V), float("nan"), dtype=torch.bfloat16, device=DEV), None)
    loss, dl, _ = tpr.vocab_parallel_ce_opts_fwd_bwd(P, logits, labels, v_valid=vv, ignore_index=IGN,
                                                     label_smoothing=eps, out=out)
    torch.cuda.synchronize()
    y = labels.cpu().numpy()
    counted = y != IGN
    n = int(counted.sum())
    rowsum = dl.float().sum(dim=1)
    assert rowsum.abs().max().item() <= 2.0 ** -7 / n
    assert not dl[:, vv:].any()
    assert not dl[torch.as_tensor(~counted, device=DEV)].any()
    z = logits.float().cpu().numpy()
    total = diff = scale = worst = 0.0
    for lo in range(0, T, 256):
        hi = min(T, lo + 256)
        _, rl, g, nb = cross_entropy_opts(z[lo:hi], y[lo:hi], vv, IGN, eps)
        total += rl.sum()
        g *= nb / n                           # the block's mean -> the mean over all counted rows
        got = f64(dl[lo:hi])
        assert not np.isnan(got).any(), lo
        diff = max(diff, float(np.abs(got - g).max()))
        scale = max(scale, float(np.abs(g).max()))
        c = counted[lo:hi]
        q = target_rows(np.where(c, y[lo:hi], 0), V, vv, eps, c)
        worst = max(worst, assert_grad_elementwise(got, g, q, n, "bf16", f"rows {lo}..{hi}"))
    wl = total / n
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl)
    assert diff <= 2e-2 * scale
    say("worst element / bound", round(worst, 3), "max-scaled error", diff / scale)
