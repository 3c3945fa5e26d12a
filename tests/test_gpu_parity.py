"""GPU parity: libtprank (through its C ABI) against the fp64 oracle.

Tolerances (max |gpu - oracle| over an output tensor, relative to max |oracle|):
1e-5 for fp32 inputs and 2e-2 for bf16 inputs; shard ranges and shapes are
bit-exact.  Cross-entropy gradients are also checked element by element
(ce_checks.py: every softmax term against a bound derived from the kernels'
roundings), since at a large vocabulary the max-scaled bound cannot see the
softmax part.  The oracle sees exactly the values the GPU sees (bf16 widened
to fp64) and rounds no intermediate.  Full-size workloads are compared on
every output element (outputs pre-filled with NaN, so a tile never written
fails), the oracle working through them in row blocks.
"""
import sys

import math

import numpy as np
import pytest
import torch

import oracle
import workloads
from ce_checks import assert_grad_elementwise, target_rows

pytestmark = pytest.mark.gpu

TOL_F32 = 1e-5
TOL_BF16 = 2e-2


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, want):
    want = np.asarray(want, dtype=np.float64)
    got = np.asarray(got, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    if want.size == 0:
        return 0.0
    scale = float(np.abs(want).max())
    diff = float(np.abs(got - want).max())
    return diff / scale if scale > 0 else diff


def tol_of(dtype):
    return TOL_F32 if dtype == torch.float32 else TOL_BF16


def out_kind(dtype):
    return "f32" if dtype == torch.float32 else "bf16"


@pytest.fixture(scope="module")
def tpr():
    import megatron_mlp_fwd_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


DEV = "cuda:0"


# ---------------------------------------------------------------- sharded GEMM

@pytest.mark.parametrize("parts", [2, 7])
@pytest.mark.parametrize("axis", ["rows", "columns", "inner"])
def test_walkthrough_fp32(tpr, axis, parts):
    say("walkthrough M3K5N4", axis, parts)
    a, b, g = workloads.sharded_gemm_tiny(seed=0, device=DEV)
    got = tpr.sharded_matmul_fwd_bwd(axis, parts, a, b, g)
    torch.cuda.synchronize()
    want = oracle.matmul_grads(f64(a), f64(b), f64(g))
    for w, o in zip(want, got):
        assert rel_err(f64(o), w) <= TOL_F32


def test_random_sizes_fp32_sweep(tpr):
    # 1000 random sizes on all three axes, part counts above the dimension
    # included (sizes 1..12, parts 1..16, seed 0).
    rng = np.random.default_rng(0)
    say("random fp32 sweep, 1000 sizes x 3 axes")
    worst = 0.0
    for i in range(1000):
        M, K, N = (int(v) for v in rng.integers(1, 13, size=3))
        parts = int(rng.integers(1, 17))
        a = rng.uniform(-1, 1, (M, K)).astype(np.float32)
        b = rng.uniform(-1, 1, (K, N)).astype(np.float32)
        g = rng.uniform(-1, 1, (M, N)).astype(np.float32)
        ta, tb, tg = (torch.from_numpy(x).to(DEV) for x in (a, b, g))
        want = oracle.matmul_grads(a, b, g)
        for axis in ("rows", "columns", "inner"):
            got = tpr.sharded_matmul_fwd_bwd(axis, parts, ta, tb, tg)
            for w, o in zip(want, got):
                e = rel_err(f64(o), w)
                worst = max(worst, e)
                assert e <= TOL_F32, (i, M, K, N, parts, axis, e)
    say("worst rel err", worst)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("shape", [(0, 5, 4), (3, 0, 4), (3, 5, 0), (0, 0, 0)])
@pytest.mark.parametrize("axis", ["rows", "columns", "inner"])
def test_zero_sizes(tpr, axis, shape, dtype):
    say("zero sizes", axis, shape, dtype)
    M, K, N = shape
    a = torch.randn(M, K, device=DEV).to(dtype)
    b = torch.randn(K, N, device=DEV).to(dtype)
    g = torch.randn(M, N, device=DEV).to(dtype)
    out = tuple(torch.full(s, float("nan"), device=DEV) for s in ((M, N), (M, K), (K, N)))
    got = tpr.sharded_matmul_fwd_bwd(axis, 3, a, b, g, out=out)
    torch.cuda.synchronize()
    want = oracle.matmul_grads(f64(a), f64(b), f64(g))
    for w, o in zip(want, got):
        np.testing.assert_array_equal(f64(o), w)  # empty contractions give exact zeros


BF16_GEMM_SHAPES = [(512, 256, 512), (300, 136, 520), (264, 72, 40), (1000, 1000, 24), (7, 9, 11), (520, 96, 264),
                    (256, 1024, 768)]


@pytest.fixture(params=["auto", "staged"])
def gemm_path(request, monkeypatch):
    # "auto" lets the library pick the direct-to-LDS kernel where eligible;
    # "staged" forces the register-staged kernel on the same shapes.
    if request.param == "staged":
        monkeypatch.setenv("TPRANK_GEMM_PATH", "staged")
    else:
        monkeypatch.delenv("TPRANK_GEMM_PATH", raising=False)
    return request.param


@pytest.mark.parametrize("parts", [1, 3, 8])
@pytest.mark.parametrize("shape", BF16_GEMM_SHAPES)
@pytest.mark.parametrize("axis", ["rows", "columns", "inner"])
def test_bf16_gemm_tiles_and_tails(tpr, axis, shape, parts, gemm_path):
    say("bf16 sharded GEMM", axis, shape, parts, gemm_path)
    M, K, N = shape
    a, b, g = workloads.inner_gemm(M, K, N, seed=M + K + N + parts, device=DEV, b_std=1.0)
    got = tpr.sharded_matmul_fwd_bwd(axis, parts, a, b, g)
    torch.cuda.synchronize()
    want = oracle.matmul_grads(f64(a), f64(b), f64(g))
    for name, w, o in zip(("Y", "dA", "dB"), want, got):
        e = rel_err(f64(o), w)
        # inputs are exact in bf16 and products accumulate in fp32: far below the contract
        assert e <= 1e-4, (name, e)


def test_bf16_gemm_more_parts_than_rows(tpr):
    say("bf16 sharded GEMM, empty shards")
    a, b, g = workloads.inner_gemm(5, 6, 7, seed=3, device=DEV, b_std=1.0)
    want = oracle.matmul_grads(f64(a), f64(b), f64(g))
    for axis in ("rows", "columns", "inner"):
        for parts in (8, 13, 17):
            got = tpr.sharded_matmul_fwd_bwd(axis, parts, a, b, g)
            for w, o in zip(want, got):
                assert rel_err(f64(o), w) <= 1e-4


def _nan_out(*shapes):
    return tuple(torch.full(sh, float("nan"), device=DEV) for sh in shapes)


def test_inner_gemm_70b_rank_full(tpr):
    # One TP=8 rank's inner-axis shard of the 70B MLP: M=8192, K_r=1024,
    # N=8192, every element of Y, dA and dB at 1 and 8 parts.  bf16 inputs are
    # exact in the oracle and products accumulate in fp32, so beside the 2e-2
    # contract the results sit within 1e-4 of max |oracle|.
    say("inner GEMM 8192x1024x8192 bf16, every element, parts 1 and 8")
    M, K, N = 8192, 1024, 8192
    a, b, g = workloads.inner_gemm(M, K, N, seed=5, device=DEV)
    want = oracle.matmul_grads(f64(a), f64(b), f64(g))
    first = None
    for parts in (1, 8):
        got = tpr.sharded_matmul_fwd_bwd("inner", parts, a, b, g, out=_nan_out((M, N), (M, K), (K, N)))
        torch.cuda.synchronize()
        for name, w, o in zip(("Y", "dA", "dB"), want, got):
            e = rel_err(f64(o), w)
            say("parts", parts, name, "rel err", e)
            assert e <= 1e-4, (parts, name, e)
        if first is None:
            first = got
        else:  # stacked outputs do not depend on the split; Y only through its sum
            assert torch.equal(got[1], first[1]) and torch.equal(got[2], first[2])
        del got
    del first
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K", [32736, 32768])
def test_bf16_gemm_operand_size_limit(tpr, K):
    # The direct-to-LDS kernel addresses each operand with 32-bit byte offsets
    # and takes operands below 1 GiB: at M = 16384 an A of K = 32736 columns
    # (1023 MiB, K a multiple of 32) runs there with its largest offsets in
    # every product, K = 32768 (1 GiB) sends the products reading A to the
    # register-staged kernel.  Both checked on sampled rows and columns.
    M, N = 16384, 64
    say("bf16 inner GEMM at the 1 GiB operand limit: M, K, N =", M, K, N)
    a, b, g = workloads.inner_gemm(M, K, N, seed=K, device=DEV)
    Y, dA, dB = tpr.sharded_matmul_fwd_bwd("inner", 1, a, b, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(K)
    rows = np.sort(np.concatenate([rng.choice(M, 6, replace=False), [0, M - 1]]))
    krows = np.sort(np.concatenate([rng.choice(K, 6, replace=False), [0, K - 1]]))
    ri, ki = torch.from_numpy(rows).to(DEV), torch.from_numpy(krows).to(DEV)
    B, G = f64(b), f64(g)
    assert rel_err(f64(Y[ri]), f64(a[ri]) @ B) <= 1e-4
    assert rel_err(f64(dA[ri]), f64(g[ri]) @ B.T) <= 1e-4
    assert rel_err(f64(dB[ki]), f64(a[:, ki]).T @ G) <= 1e-4
    del Y, dA, dB, a, b, g
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- partial sum

def _slot_order_sum(p):
    # the definition evaluated in the library's order: fp32 adds, slot by slot
    acc = p[0].copy()
    for r in range(1, p.shape[0]):
        acc = (acc + p[r]).astype(np.float32)
    return acc


@pytest.mark.parametrize("nslots,n", [(1, 1000), (2, 4096), (3, 4099), (8, 1 << 20), (9, 5000), (17, 4096),
                                      (8, 8192 * 8192)])
def test_partial_sum(tpr, nslots, n):
    # Cross-rank partial sum through tprank_partial_sum: the same bits as
    # fp32 adds in slot order, within fp32 rounding of the fp64 sum.
    say("partial sum", nslots, n)
    g = torch.Generator(device=DEV)
    g.manual_seed(nslots * 7 + n % 1000)
    parts = torch.randn(nslots, n, generator=g, device=DEV)
    out = torch.full((n,), float("nan"), device=DEV)
    got = tpr.partial_sum(parts, out=out)
    torch.cuda.synchronize()
    p = parts.cpu().numpy()
    np.testing.assert_array_equal(got.cpu().numpy(), _slot_order_sum(p))
    want = p.astype(np.float64).sum(axis=0)
    assert np.abs(got.cpu().numpy() - want).max() <= nslots * 2.0 ** -23 * np.abs(p).sum(axis=0).max()
    del parts, out, got
    torch.cuda.empty_cache()


def test_partial_sum_strided_and_edges(tpr):
    import ctypes
    lib = tpr.load_library()
    stream = torch.cuda.current_stream().cuda_stream
    nslots, n, stride = 5, 1000, 1024      # slots 1024 floats apart, 1000 used
    g = torch.Generator(device=DEV)
    g.manual_seed(3)
    buf = torch.randn(nslots, stride, generator=g, device=DEV)
    out = torch.full((n + 8,), float("nan"), device=DEV)
    assert lib.tprank_partial_sum(nslots, n, buf.data_ptr(), stride, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    np.testing.assert_array_equal(out[:n].cpu().numpy(), _slot_order_sum(buf[:, :n].cpu().numpy()))
    assert torch.isnan(out[n:]).all()      # nothing past the n outputs
    # no slots: the empty sum is zero
    assert lib.tprank_partial_sum(0, n, None, n, out.data_ptr(), stream) == 0
    torch.cuda.synchronize()
    assert not out[:n].any() and torch.isnan(out[n:]).all()
    # rejected before any launch
    assert lib.tprank_partial_sum(2, 10, buf.data_ptr(), 5, out.data_ptr(), stream) == tpr.binding.TPR_ERR_SHAPE
    assert lib.tprank_partial_sum(2, 10, buf.data_ptr(), 16, buf.data_ptr() + 8, stream) == \
        tpr.binding.TPR_ERR_VALUE
    assert lib.tprank_partial_sum(2, 10, None, 16, out.data_ptr(), stream) == tpr.binding.TPR_ERR_NULLPTR


# ---------------------------------------------------------------- TP MLP

def test_mlp_lesson_selftest_fp32(tpr):
    # The TP lesson's self-test: tp=4, x (2,8,64), w1 (256,64), w2 (64,256), torch layout.
    say("TP MLP fp32 tp=4 x(2,8,64)")
    x, w1, w2, gy = workloads.tp_mlp_tiny(seed=0, device=DEV)
    got = tpr.tp_mlp_fwd_bwd(4, x, w1, w2, gy, "torch")
    torch.cuda.synchronize()
    want = oracle.mlp_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), "torch")
    for name, w, o in zip(("y", "dx", "dw1", "dw2"), want, got):
        assert o.shape == torch.Size(w.shape)
        assert rel_err(f64(o), w) <= TOL_F32, name
    # and within the page's own fp32 tolerances
    torch.testing.assert_close(got[0].cpu(), torch.tensor(want[0], dtype=torch.float32), atol=3e-4, rtol=1e-5)


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("tp", [1, 2, 3, 5, 7, 300])
def test_mlp_fp32_uneven_and_empty_ranks(tpr, tp, layout):
    say("TP MLP fp32", tp, layout)
    T, d, f = 10, 24, 20
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=tp, device=DEV, dtype=torch.float32, w_std=0.3)
    if layout == "torch":
        w1, w2 = w1.t().contiguous(), w2.t().contiguous()
    got = tpr.tp_mlp_fwd_bwd(tp, x, w1, w2, gy, layout)
    torch.cuda.synchronize()
    want = oracle.mlp_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), layout)
    for name, w, o in zip(("y", "dx", "dw1", "dw2"), want, got):
        assert rel_err(f64(o), w) <= TOL_F32, name


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("tp", [1, 2, 3])
@pytest.mark.parametrize("shape", [(512, 256, 256), (300, 264, 200), (64, 40, 24), (96, 512, 768), (272, 320, 448),
                                   (256, 256, 232)])
def test_mlp_bf16_tiles_and_tails(tpr, shape, tp, layout, gemm_path):
    say("TP MLP bf16", shape, tp, layout, gemm_path)
    T, d, f = shape
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=T + tp, device=DEV, w_std=0.05)
    if layout == "torch":
        w1, w2 = w1.t().contiguous(), w2.t().contiguous()
    got = tpr.tp_mlp_fwd_bwd(tp, x, w1, w2, gy, layout)
    torch.cuda.synchronize()
    want = oracle.mlp_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), layout)
    for name, w, o in zip(("y", "dx", "dw1", "dw2"), want, got):
        e = rel_err(f64(o), w)
        assert e <= TOL_BF16, (name, e)


@pytest.mark.parametrize("tp,shape", [(5, (300, 264, 200)), (8, (256, 128, 512)), (8, (96, 64, 40)),
                                      (13, (130, 72, 9))])
def test_mlp_bf16_many_ranks(tpr, tp, shape):
    # More ranks than one grouped launch holds problems (16): the backward
    # products of all ranks are then split over several launches, and with
    # f < tp some ranks hold no hidden units.  Outputs start as NaN, so a
    # product that no launch ran fails.
    T, d, f = shape
    say("TP MLP bf16 many ranks", tp, shape)
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=tp * 31 + T, device=DEV, w_std=0.05)
    out = _nan_out((T, d), (T, d), (d, f), (f, d))
    got = tpr.tp_mlp_fwd_bwd(tp, x, w1, w2, gy, "math", out=out)
    torch.cuda.synchronize()
    want = oracle.mlp_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), "math")
    for name, w, o in zip(("y", "dx", "dw1", "dw2"), want, got):
        e = rel_err(f64(o), w)
        assert e <= TOL_BF16, (name, e)


def test_mlp_zero_sizes(tpr):
    for T, d, f in ((0, 8, 8), (8, 8, 0), (8, 0, 8)):
        for dtype in (torch.float32, torch.bfloat16):
            say("TP MLP zero sizes", T, d, f, dtype)
            x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=1, device=DEV, dtype=dtype)
            out = (torch.full((T, d), float("nan"), device=DEV), torch.full((T, d), float("nan"), device=DEV),
                   torch.full((d, f), float("nan"), device=DEV), torch.full((f, d), float("nan"), device=DEV))
            got = tpr.tp_mlp_fwd_bwd(2, x, w1, w2, gy, "math", out=out)
            torch.cuda.synchronize()
            want = oracle.mlp_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), "math")
            for w, o in zip(want, got):
                np.testing.assert_array_equal(f64(o), w)


def _mlp_rank_full(tpr, T, d, f, seed):
    # Every element of y, dx, dw1 and dw2 against the fp64 oracle; the
    # outputs start as NaN so that a tile the launches never write fails.
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=seed, device=DEV)
    out = _nan_out((T, d), (T, d), (d, f), (f, d))
    got = tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy, "math", out=out)
    torch.cuda.synchronize()
    want = oracle.mlp_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), "math")
    errs = {}
    for name, w, o in zip(("y", "dx", "dw1", "dw2"), want, got):
        h = f64(o)
        assert not np.isnan(h).any(), name
        errs[name] = rel_err(h, w)
    say("rel errs", errs)
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)


def test_mlp_llama3_8b_tp8_rank_full(tpr):
    say("Llama-3-8B TP=8 rank MLP T=4096 d=4096 f=1792, every element")
    _mlp_rank_full(tpr, 4096, 4096, 1792, seed=8)


def test_mlp_llama3_70b_tp8_rank_full(tpr):
    say("Llama-3-70B TP=8 rank MLP T=8192 d=8192 f=3584, every element")
    _mlp_rank_full(tpr, 8192, 8192, 3584, seed=70)
    torch.cuda.empty_cache()


# ---------------------------------------------------------------- vocab CE

@pytest.mark.parametrize("stats", [True, False])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("V,parts", [(8, 1), (8, 3), (1001, 3), (4096, 8), (4096, 17), (40000, 8), (100, 5000),
                                     (128256, 8)])
def test_ce_small(tpr, V, parts, dtype, stats):
    say("vocab CE", V, parts, dtype, "stats" if stats else "no stats")
    T = 5
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=V + parts, device=DEV, dtype=dtype)
    loss, dl, st = tpr.vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=stats)
    torch.cuda.synchronize()
    z, y = f64(logits), labels.cpu().numpy()
    wl, _, wg, wst = oracle.vocab_parallel_ce(z, y, parts)
    tol = tol_of(dtype)
    assert abs(loss.item() - wl) <= tol * abs(wl)
    assert rel_err(f64(dl), wg) <= tol
    assert_grad_elementwise(f64(dl), wg, target_rows(y, V), T, out_kind(dtype), "dlogits")
    if not stats:
        assert st is None
        return
    gst = f64(st)
    np.testing.assert_array_equal(gst[:, :, 0], wst[:, :, 0])           # maxima are exact
    np.testing.assert_allclose(gst[:, :, 1], wst[:, :, 1], rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(gst[:, :, 2], wst[:, :, 2], rtol=1e-6, atol=1e-6)


# Rows held partly in registers (22 x 512 vectors of 8 logits) and partly in
# LDS (up to 4864 vectors): empty, single-vector, ragged and full LDS parts,
# and one vector past the capacity (served by the single-row kernel).
@pytest.mark.parametrize("V", [8 * 11264, 8 * 11265, 8 * 11364, 8 * (11264 + 4864), 8 * (11264 + 4864) + 8])
def test_ce_bf16_row_split_edges(tpr, V):
    say("vocab CE bf16, no stats, V =", V)
    T = 4
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=V, device=DEV)
    labels[0] = V - 1   # target in the last vector
    labels[1] = 0
    loss, dl, _ = tpr.vocab_parallel_ce_fwd_bwd(4, logits, labels)
    torch.cuda.synchronize()
    z, y = f64(logits), labels.cpu().numpy()
    wl, _, wg = oracle.cross_entropy(z, y, grad_rows=np.arange(T))
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl)
    assert rel_err(f64(dl), wg) <= TOL_BF16
    # every element, the LDS-resident part of the row included
    assert_grad_elementwise(f64(dl), wg, target_rows(y, V), T, "bf16", "dlogits")


# Per-shard statistics in the paired kernel: equal shards of >= 64 vectors of
# 8 logits, boundaries inside a wave's group of 64 vectors (vps not a
# multiple of 64), rows with and without an LDS part, 1 to 16 shards; checked
# against the oracle, and against the one-row (or three-pass) kernel on the
# same inputs.
@pytest.mark.parametrize("vps,parts", [(64, 1), (64, 3), (100, 5), (700, 7), (2004, 8), (1500, 10), (1000, 16)])
def test_ce_bf16_shard_stats_paired(tpr, vps, parts, monkeypatch):
    V, T = 8 * vps * parts, 6
    say("vocab CE bf16 with shard stats, paired kernel: V =", V, "parts =", parts)
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=vps + parts, device=DEV)
    labels[0], labels[1], labels[2] = V - 1, 0, min(8 * vps, V - 1)  # last column; first column of shard 1
    monkeypatch.delenv("TPRANK_CE_STATS_PATH", raising=False)
    loss, dl, st = tpr.vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=True)
    monkeypatch.setenv("TPRANK_CE_STATS_PATH", "onerow")
    loss1, dl1, st1 = tpr.vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=True)
    torch.cuda.synchronize()
    z, y = f64(logits), labels.cpu().numpy()
    wl, _, wg, wst = oracle.vocab_parallel_ce(z, y, parts)
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl)
    assert rel_err(f64(dl), wg) <= TOL_BF16
    q = target_rows(y, V)
    assert_grad_elementwise(f64(dl), wg, q, T, "bf16", "dlogits (paired kernel)")
    assert_grad_elementwise(f64(dl1), wg, q, T, "bf16", "dlogits (one-row kernel)")
    gst = f64(st)
    np.testing.assert_array_equal(gst[:, :, 0], wst[:, :, 0])           # maxima are exact
    np.testing.assert_allclose(gst[:, :, 1], wst[:, :, 1], rtol=1e-5, atol=1e-30)
    np.testing.assert_allclose(gst[:, :, 2], wst[:, :, 2], rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(gst[:, :, 0], f64(st1)[:, :, 0])
    np.testing.assert_allclose(gst[:, :, 1], f64(st1)[:, :, 1], rtol=1e-5)
    assert abs(loss.item() - loss1.item()) <= 1e-5 * abs(loss1.item())


def test_ce_zero_rows(tpr):
    say("vocab CE T=0")
    logits = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    labels = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, dl, _ = tpr.vocab_parallel_ce_fwd_bwd(2, logits, labels)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and dl.shape == (0, 16)


def _ce_check_all_rows(dl, z, y, loss, what, block=256):
    """Every row of a full-size CE result against the oracle, in row blocks:
    the loss within 1e-5, dlogits within 2e-2 max |oracle| over the whole
    tensor and element by element (ce_checks.py)."""
    T, V = z.shape
    row_loss = np.empty(T)
    diff = scale = worst = 0.0
    for lo in range(0, T, block):
        hi = min(T, lo + block)
        _, rl, g = oracle.cross_entropy(z[lo:hi], y[lo:hi])
        row_loss[lo:hi] = rl
        g *= (hi - lo) / T            # the block's mean -> the mean over all T rows
        got = f64(dl[lo:hi])
        assert not np.isnan(got).any(), (what, lo)
        diff = max(diff, float(np.abs(got - g).max()))
        scale = max(scale, float(np.abs(g).max()))
        worst = max(worst, assert_grad_elementwise(got, g, target_rows(y[lo:hi], V), T, "bf16",
                                                   f"{what}, rows {lo}..{hi}"))
    wl = row_loss.mean()
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl), (loss.item(), wl)
    assert diff <= TOL_BF16 * scale, (diff, scale)
    say(what, "worst element / bound", round(worst, 3), "max-scaled error", diff / scale)
    return row_loss


def test_ce_full_config(tpr):
    # 4096 positions x vocab 128256, 8 contiguous shards of 16032, bf16 ~ N(0, 2).
    say("vocab CE 4096 x 128256 bf16, 8 shards, every row")
    T, V, P = 4096, 128256, 8
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=0, device=DEV)
    out = (torch.empty((), device=DEV), torch.full((T, V), float("nan"), dtype=torch.bfloat16, device=DEV),
           torch.full((T, P, 3), float("nan"), device=DEV))
    loss, dl, st = tpr.vocab_parallel_ce_fwd_bwd(P, logits, labels, shard_stats=True, out=out)
    torch.cuda.synchronize()
    # every row's gradient sums to 0 (softmax minus one-hot); rounding each term
    # to bf16 (unit roundoff 2^-8) over sum_j |g_j| = 2 (1 - p_y) / T bounds the
    # row sum by 2^-7 / T
    rowsum = dl.float().sum(dim=1)
    assert rowsum.abs().max().item() <= 2.0 ** -7 / T
    z = logits.float().cpu().numpy()
    y = labels.cpu().numpy()
    rl = _ce_check_all_rows(dl, z, y, loss, "CE with shard stats")
    _, _, _, wst = oracle.vocab_parallel_ce(z[:64], y[:64], P)
    gst = f64(st)
    assert not np.isnan(gst).any()
    np.testing.assert_array_equal(gst[:64, :, 0], wst[:, :, 0])
    np.testing.assert_allclose(gst[:64, :, 1], wst[:, :, 1], rtol=1e-5)
    np.testing.assert_allclose(gst[:64, :, 2], wst[:, :, 2], rtol=1e-6, atol=1e-6)
    # the rest of the rows: the statistics combine to the row's loss and max
    m = gst[:, :, 0].max(axis=1)
    np.testing.assert_array_equal(m, z.max(axis=1))
    lse = np.log(gst[:, :, 1].sum(axis=1)) + m
    zy = z[np.arange(T), y]
    np.testing.assert_allclose(gst[:, :, 2].sum(axis=1), zy - m, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(lse - zy, rl, rtol=2e-6, atol=1e-6)


def test_ce_full_config_no_stats(tpr):
    # The benchmarked call: 4096 x 128256, 8 shards, no per-shard statistics.
    say("vocab CE 4096 x 128256 bf16, 8 shards, no stats, every row")
    T, V, P = 4096, 128256, 8
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=0, device=DEV)
    out = (torch.empty((), device=DEV), torch.full((T, V), float("nan"), dtype=torch.bfloat16, device=DEV), None)
    loss, dl, st = tpr.vocab_parallel_ce_fwd_bwd(P, logits, labels, out=out)
    torch.cuda.synchronize()
    assert st is None
    rowsum = dl.float().sum(dim=1)
    assert rowsum.abs().max().item() <= 2.0 ** -7 / T
    _ce_check_all_rows(dl, logits.float().cpu().numpy(), labels.cpu().numpy(), loss, "CE without shard stats")


def test_determinism(tpr):
    say("determinism: repeated calls are bitwise identical")
    logits, labels = workloads.vocab_ce(T=64, V=128256, seed=9, device=DEV)
    a = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels)
    b = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    a = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels, shard_stats=True)
    b = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels, shard_stats=True)
    for p, q in zip(a, b):
        assert torch.equal(p, q)
    x, w1, w2, gy = workloads.rank_mlp(300, 264, 200, seed=4, device=DEV)
    r1 = tpr.tp_mlp_fwd_bwd(3, x, w1, w2, gy)
    r2 = tpr.tp_mlp_fwd_bwd(3, x, w1, w2, gy)
    for p, q in zip(r1, r2):
        assert torch.equal(p, q)


# ---------------------------------------------------------------- vocab head + CE

U24 = 2.0 ** -24


def _head_stages(tpr, h, w, y, parts, layout):
    """Run the head and return (loss, dh, dw, logits, dlogits): the last two
    read from the workspace, where the entry point leaves them (logits at
    byte 0, dlogits at the next 256-byte boundary)."""
    T, d = h.shape
    V = w.shape[1] if layout == "math" else w.shape[0]
    nb = tpr.vocab_parallel_head_ce_workspace_bytes(parts, h.dtype, T, d, V)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device=DEV)  # NaN in bf16 and fp32
    loss, dh, dw = tpr.vocab_parallel_head_ce_fwd_bwd(parts, h, w, y, w_layout=layout, workspace=ws)
    torch.cuda.synchronize()
    tv = T * V * h.element_size()
    off = (tv + 255) // 256 * 256
    logits = ws[:tv].view(h.dtype).view(T, V)
    dl = ws[off:off + tv].view(h.dtype).view(T, V)
    return loss, dh, dw, logits, dl


def _check_head_stages(h, w, y, layout, parts, loss, dh, dw, logits, dl, dtype):
    """Each stage against the oracle on that stage's exact inputs, element
    by element: logits = h W (rounded once to the compute dtype, fp32
    accumulation over d: |err| <= u |z| + d 2^-24 (|h| |W|)); dlogits =
    the CE gradient of the GPU's own logits (ce_checks.py); dh = dlogits W^T
    and dW = h^T dlogits of the GPU's own dlogits (fp32 accumulation over V,
    plus the rank-order sum of the parts: (V + parts) 2^-24 (|dl| |W|^T))."""
    H, Wm = f64(h), f64(w if layout == "math" else w.t())
    T, d = H.shape
    V = Wm.shape[1]
    u = U24 if dtype == torch.float32 else 2.0 ** -8
    z_ref = H @ Wm
    z = f64(logits)
    assert not np.isnan(z).any()
    bound = u * np.abs(z_ref) + d * U24 * (np.abs(H) @ np.abs(Wm))
    assert (np.abs(z - z_ref) <= bound).all(), float((np.abs(z - z_ref) / bound).max())
    yy = y.cpu().numpy()
    wl, _, g_ref = oracle.cross_entropy(z, yy)
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl) + 1e-7
    G = f64(dl)
    assert_grad_elementwise(G, g_ref, target_rows(yy, V), T, out_kind(dtype), "head dlogits")
    dh_ref = G @ Wm.T
    bh = (V + parts) * U24 * (np.abs(G) @ np.abs(Wm.T))
    assert (np.abs(f64(dh) - dh_ref) <= bh).all(), float((np.abs(f64(dh) - dh_ref) / bh).max())
    dw_ref = H.T @ G
    bw = (T + 1) * U24 * (np.abs(H.T) @ np.abs(G))
    got_dw = f64(dw if layout == "math" else dw.t())
    assert (np.abs(got_dw - dw_ref) <= bw).all(), float((np.abs(got_dw - dw_ref) / bw).max())


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("parts", [1, 3, 8])
@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,d,V", [(37, 64, 1003), (256, 264, 4096), (5, 8, 3)])
def test_head_ce(tpr, T, d, V, dtype, parts, layout):
    say("vocab head + CE", T, d, V, dtype, parts, layout)
    # Logits of standard deviation 2, like the CE workload: with bf16 logits
    # the probabilities carry a relative error of about |z| 2^-9.
    h, w, y = workloads.vocab_head(T, d, V, seed=T + d + V + parts, device=DEV, dtype=dtype,
                                   w_std=2.0 / math.sqrt(d), w_layout=layout)
    loss, dh, dw, logits, dl = _head_stages(tpr, h, w, y, parts, layout)
    wl, wdh, wdw = oracle.head_ce(f64(h), f64(w), y.cpu().numpy(), layout)
    tol = tol_of(dtype)
    assert abs(loss.item() - wl) <= tol * abs(wl)
    assert rel_err(f64(dh), wdh) <= tol
    assert rel_err(f64(dw), wdw) <= tol
    _check_head_stages(h, w, y, layout, parts, loss, dh, dw, logits, dl, dtype)


def test_head_ce_zero_rows(tpr):
    say("vocab head + CE, T = 0")
    h = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    w = torch.randn(16, 40, device=DEV).to(torch.bfloat16)
    y = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, dh, dw = tpr.vocab_parallel_head_ce_fwd_bwd(4, h, w, y)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and dh.shape == (0, 16)
    assert torch.count_nonzero(dw).item() == 0


def test_head_ce_llama3_8b_sized(tpr):
    # Llama-3-8B hidden size with a 32000-entry vocabulary, 8 shards (the
    # full 128256 vocabulary is the benchmark's; the fp64 oracle of a smaller
    # vocabulary keeps the test in seconds), bf16, every element of every stage.
    say("vocab head + CE T=512 d=4096 V=32000 bf16, 8 shards")
    T, d, V = 512, 4096, 32000
    h, w, y = workloads.vocab_head(T, d, V, seed=3, device=DEV, w_std=2.0 / math.sqrt(d))
    loss, dh, dw, logits, dl = _head_stages(tpr, h, w, y, 8, "math")
    wl, wdh, wdw = oracle.head_ce(f64(h), f64(w), y.cpu().numpy())
    assert abs(loss.item() - wl) <= TOL_BF16 * abs(wl)
    assert rel_err(f64(dh), wdh) <= TOL_BF16
    assert rel_err(f64(dw), wdw) <= TOL_BF16
    _check_head_stages(h, w, y, "math", 8, loss, dh, dw, logits, dl, torch.bfloat16)
