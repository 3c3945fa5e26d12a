"""GPU parity: libtprank (through its C ABI) against the fp64 oracle.

Tolerances (max |gpu - oracle| over an output tensor, relative to max |oracle|):
1e-5 for fp32 inputs and 2e-2 for bf16 inputs; shard ranges and shapes are
bit-exact.  The oracle sees exactly the values the GPU sees (bf16 widened to
fp64) and rounds no intermediate.  Full-size workloads are checked on sampled
outputs that the oracle computes one by one, plus properties that hold at any
size.
"""
import sys

import math

import numpy as np
import pytest
import torch

import oracle
import workloads

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


def test_inner_gemm_70b_rank_sampled(tpr):
    # One TP=8 rank's inner-axis shard of the 70B MLP: M=8192, K_r=1024, N=8192.
    say("inner GEMM 8192x1024x8192 bf16, sampled")
    M, K, N = 8192, 1024, 8192
    a, b, g = workloads.inner_gemm(M, K, N, seed=5, device=DEV)
    Y, dA, dB = tpr.sharded_matmul_fwd_bwd("inner", 1, a, b, g)
    torch.cuda.synchronize()
    rng = np.random.default_rng(1)
    rows = np.sort(rng.choice(M, 12, replace=False))
    cols = np.sort(rng.choice(N, 12, replace=False))
    A, B, G = f64(a), f64(b), f64(g)
    assert rel_err(f64(Y[rows]), A[rows] @ B) <= TOL_BF16
    assert rel_err(f64(dA[rows]), G[rows] @ B.T) <= TOL_BF16
    assert rel_err(f64(dB[:, cols]), A.T @ G[:, cols]) <= TOL_BF16
    # the same rank split 8 ways again must agree with itself
    Y8, dA8, dB8 = tpr.sharded_matmul_fwd_bwd("inner", 8, a, b, g)
    torch.cuda.synchronize()
    assert rel_err(f64(Y8[rows]), A[rows] @ B) <= TOL_BF16
    assert torch.equal(dA8, dA) and torch.equal(dB8, dB)


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


def _mlp_rank_sampled(tpr, T, d, f, seed):
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=seed, device=DEV)
    y, dx, dw1, dw2 = tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy, "math")
    torch.cuda.synchronize()
    rng = np.random.default_rng(seed)
    rows = np.sort(rng.choice(T, 8, replace=False))
    cols = np.sort(rng.choice(f, 8, replace=False))
    s = oracle.mlp_sampled(f64(x), f64(w1), f64(w2), f64(gy), rows, cols, "math")
    errs = dict(y=rel_err(f64(y[rows]), s["y"]), dx=rel_err(f64(dx[rows]), s["dx"]),
                dw1=rel_err(f64(dw1[:, cols]), s["dw1_cols"]), dw2=rel_err(f64(dw2[cols]), s["dw2_rows"]))
    say("sampled rel errs", errs)
    for k, e in errs.items():
        assert e <= TOL_BF16, (k, e)
    # properties at full size: finite everywhere
    for t in (y, dx, dw1, dw2):
        assert torch.isfinite(t).all()


def test_mlp_llama3_8b_tp8_rank_sampled(tpr):
    say("Llama-3-8B TP=8 rank MLP T=4096 d=4096 f=1792, sampled")
    _mlp_rank_sampled(tpr, 4096, 4096, 1792, seed=8)


def test_mlp_llama3_70b_tp8_rank_sampled(tpr):
    say("Llama-3-70B TP=8 rank MLP T=8192 d=8192 f=3584, sampled")
    _mlp_rank_sampled(tpr, 8192, 8192, 3584, seed=70)


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


def test_ce_full_config(tpr):
    # 4096 positions x vocab 128256, 8 contiguous shards of 16032, bf16 ~ N(0, 2).
    say("vocab CE 4096 x 128256 bf16, 8 shards")
    T, V, P = 4096, 128256, 8
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=0, device=DEV)
    loss, dl, st = tpr.vocab_parallel_ce_fwd_bwd(P, logits, labels, shard_stats=True)
    torch.cuda.synchronize()
    # every row's gradient sums to 0 (softmax minus one-hot); rounding each term
    # to bf16 (unit roundoff 2^-8) over sum_j |g_j| = 2 (1 - p_y) / T bounds the
    # row sum by 2^-7 / T
    rowsum = dl.float().sum(dim=1)
    assert rowsum.abs().max().item() <= 2.0 ** -7 / T
    z = logits.float().cpu().numpy()
    y = labels.cpu().numpy()
    rows = np.sort(np.random.default_rng(0).choice(T, 16, replace=False))
    wl, _, wg = oracle.cross_entropy(z, y, grad_rows=rows)
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl)
    assert rel_err(f64(dl[rows]), wg) <= TOL_BF16
    _, _, _, wst = oracle.vocab_parallel_ce(z[rows], y[rows], P)
    gst = f64(st[rows])
    np.testing.assert_array_equal(gst[:, :, 0], wst[:, :, 0])
    np.testing.assert_allclose(gst[:, :, 1], wst[:, :, 1], rtol=1e-5)
    np.testing.assert_allclose(gst[:, :, 2], wst[:, :, 2], rtol=1e-6, atol=1e-6)


def test_ce_full_config_no_stats(tpr):
    # The benchmarked call: 4096 x 128256, 8 shards, no per-shard statistics.
    say("vocab CE 4096 x 128256 bf16, 8 shards, no stats")
    T, V, P = 4096, 128256, 8
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=0, device=DEV)
    loss, dl, st = tpr.vocab_parallel_ce_fwd_bwd(P, logits, labels)
    torch.cuda.synchronize()
    assert st is None
    rowsum = dl.float().sum(dim=1)
    assert rowsum.abs().max().item() <= 2.0 ** -7 / T
    z = logits.float().cpu().numpy()
    y = labels.cpu().numpy()
    rows = np.sort(np.random.default_rng(1).choice(T, 16, replace=False))
    wl, _, wg = oracle.cross_entropy(z, y, grad_rows=rows)
    assert abs(loss.item() - wl) <= 1e-5 * abs(wl)
    assert rel_err(f64(dl[rows]), wg) <= TOL_BF16


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
    loss, dh, dw = tpr.vocab_parallel_head_ce_fwd_bwd(parts, h, w, y, w_layout=layout)
    torch.cuda.synchronize()
    wl, wdh, wdw = oracle.head_ce(f64(h), f64(w), y.cpu().numpy(), layout)
    tol = tol_of(dtype)
    assert abs(loss.item() - wl) <= tol * abs(wl)
    assert rel_err(f64(dh), wdh) <= tol
    assert rel_err(f64(dw), wdw) <= tol


def test_head_ce_zero_rows(tpr):
    say("vocab head + CE, T = 0")
    h = torch.empty(0, 16, dtype=torch.bfloat16, device=DEV)
    w = torch.randn(16, 40, device=DEV).to(torch.bfloat16)
    y = torch.empty(0, dtype=torch.int64, device=DEV)
    loss, dh, dw = tpr.vocab_parallel_head_ce_fwd_bwd(4, h, w, y)
    torch.cuda.synchronize()
    assert loss.item() == 0.0 and dh.shape == (0, 16)
    assert torch.count_nonzero(dw).item() == 0


def test_head_ce_llama3_8b_sized_sampled(tpr):
    # Llama-3-8B hidden size with a 32000-entry vocabulary, 8 shards (the
    # full 128256 vocabulary is the benchmark's; the fp64 oracle of a smaller
    # vocabulary keeps the test in seconds), bf16.
    say("vocab head + CE T=512 d=4096 V=32000 bf16, 8 shards")
    T, d, V = 512, 4096, 32000
    h, w, y = workloads.vocab_head(T, d, V, seed=3, device=DEV, w_std=2.0 / math.sqrt(d))
    loss, dh, dw = tpr.vocab_parallel_head_ce_fwd_bwd(8, h, w, y)
    torch.cuda.synchronize()
    wl, wdh, wdw = oracle.head_ce(f64(h), f64(w), y.cpu().numpy())
    assert abs(loss.item() - wl) <= TOL_BF16 * abs(wl)
    assert rel_err(f64(dh), wdh) <= TOL_BF16
    assert rel_err(f64(dw), wdw) <= TOL_BF16
