"""Calls on a caller's stream, and writes that stay inside their outputs.

Side stream: the binding allocates the workspace and the outputs on the
stream the kernels run on, so memory that the default stream allocates and
overwrites while they run cannot be the workspace of the running call.

Guard bands: every output is a view into a larger buffer whose other bytes
hold a sentinel; after uneven splits, empty shards and empty ranks each
sentinel byte must be unchanged, so no kernel writes outside its output
(a write past a rank's stacked slice into a neighbour's would otherwise be
hidden by the neighbour's own later write).
"""
import sys

import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
GUARD = 4096              # bytes of sentinel on each side of an output
SENTINEL = 0x5A           # byte pattern: a finite value in every dtype, never written by the library


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tpr():
    import megatron_mlp_fwd_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


# ---------------------------------------------------------------- side stream

def test_side_stream_workspace_not_reused_by_default_stream(tpr):
    say("MLP and CE launched on a side stream while the default stream allocates and overwrites memory")
    T, d, f = 4096, 4096, 1792
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=21, device=DEV)
    logits, labels = workloads.vocab_ce(T=512, V=128256, seed=22, device=DEV)
    ref = tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy)
    ref_ce = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels)
    torch.cuda.synchronize()
    ws_mlp = tpr.tp_mlp_workspace_bytes(1, torch.bfloat16, T, d, f)
    side = torch.cuda.Stream(device=DEV)
    side.wait_stream(torch.cuda.current_stream())
    for trial in range(3):
        got = tpr.tp_mlp_fwd_bwd(1, x, w1, w2, gy, stream=side)
        got_ce = tpr.vocab_parallel_ce_fwd_bwd(8, logits, labels, stream=side)
        # the default stream now allocates blocks of the workspace's size and fills them
        junk = [torch.full((ws_mlp // 4,), float("nan"), device=DEV) for _ in range(3)]
        junk += [torch.full((512,), float("nan"), device=DEV) for _ in range(8)]
        side.synchronize()
        torch.cuda.synchronize()
        for a, b in zip(got, ref):
            assert torch.equal(a, b), trial
        assert torch.equal(got_ce[0], ref_ce[0]) and torch.equal(got_ce[1], ref_ce[1]), trial
        del junk, got, got_ce


# ---------------------------------------------------------------- guard bands

def _guarded(shape, dtype):
    """(buffer, view): a contiguous view of `shape` inside a sentinel-filled
    byte buffer with GUARD bytes on each side."""
    n = int(np.prod(shape)) * torch.tensor([], dtype=dtype).element_size()
    buf = torch.full((n + 2 * GUARD,), SENTINEL, dtype=torch.uint8, device=DEV)
    view = buf[GUARD:GUARD + n].view(dtype).view(shape)
    return buf, view


def _check_guards(bufs):
    torch.cuda.synchronize()
    for i, b in enumerate(bufs):
        lo, hi = b[:GUARD], b[b.numel() - GUARD:]
        assert bool((lo == SENTINEL).all()) and bool((hi == SENTINEL).all()), f"output {i}: a guard byte changed"


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("axis", ["rows", "columns", "inner"])
@pytest.mark.parametrize("shape,parts", [((5, 6, 7), 8), ((300, 136, 520), 3), ((264, 72, 40), 7),
                                         ((7, 9, 11), 13)])
def test_sharded_gemm_guard_bands(tpr, axis, shape, parts, dtype):
    say("guard bands, sharded GEMM", axis, shape, parts, dtype)
    M, K, N = shape
    a, b, g = workloads.inner_gemm(M, K, N, seed=M + parts, device=DEV, dtype=dtype, b_std=1.0)
    bufs, outs = zip(*(_guarded(s, torch.float32) for s in ((M, N), (M, K), (K, N))))
    got = tpr.sharded_matmul_fwd_bwd(axis, parts, a, b, g, out=outs)
    _check_guards(bufs)
    ref = tpr.sharded_matmul_fwd_bwd(axis, parts, a, b, g)
    for x, y in zip(got, ref):
        assert torch.equal(x, y)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("T,d,f,tp", [(10, 24, 20, 7), (300, 264, 200, 3), (272, 320, 448, 2), (64, 40, 24, 300)])
def test_mlp_guard_bands(tpr, T, d, f, tp, dtype):
    say("guard bands, MLP", (T, d, f), tp, dtype)
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=T + tp, device=DEV, dtype=dtype, w_std=0.05)
    bufs, outs = zip(*(_guarded(s, torch.float32) for s in ((T, d), (T, d), (d, f), (f, d))))
    nb = tpr.tp_mlp_workspace_bytes(tp, dtype, T, d, f)
    wbuf, ws = _guarded((max(nb, 1),), torch.uint8)
    got = tpr.tp_mlp_fwd_bwd(tp, x, w1, w2, gy, out=outs, workspace=ws)
    _check_guards(bufs + (wbuf,))
    ref = tpr.tp_mlp_fwd_bwd(tp, x, w1, w2, gy)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("gated", [False, True])
def test_mlp_act_guard_bands(tpr, gated):
    say("guard bands, SiLU MLP", "gated" if gated else "plain")
    T, d, f, tp = 272, 320, 264, 3
    x, w1, w2, gy = workloads.rank_mlp(T, d, f, seed=9, device=DEV, w_std=0.05)
    w3 = (w1.float() * 0.5).bfloat16() if gated else None
    shapes = [(T, d), (T, d), (d, f), (f, d)] + ([(d, f)] if gated else [])
    bufs, outs = zip(*(_guarded(s, torch.float32) for s in shapes))
    outs = tuple(outs) + (() if gated else (None,))
    nb = tpr.tp_mlp_act_workspace_bytes(tp, torch.bfloat16, gated, T, d, f)
    wbuf, ws = _guarded((nb,), torch.uint8)
    got = tpr.tp_mlp_act_fwd_bwd(tp, x, w1, w2, gy, act="silu", w3=w3, out=outs, workspace=ws)
    _check_guards(bufs + (wbuf,))
    ref = tpr.tp_mlp_act_fwd_bwd(tp, x, w1, w2, gy, act="silu", w3=w3)
    for a, b in zip(got, ref):
        if a is not None:
            assert torch.equal(a, b)


@pytest.mark.parametrize("stats", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("T,V,parts", [(5, 1001, 3), (6, 128256, 8), (3, 8 * 11264 + 24, 4), (4, 100, 300)])
def test_ce_guard_bands(tpr, T, V, parts, dtype, stats):
    say("guard bands, vocab CE", T, V, parts, dtype, stats)
    logits, labels = workloads.vocab_ce(T=T, V=V, seed=V + parts, device=DEV, dtype=dtype)
    shapes = [((), torch.float32), ((T, V), dtype)] + ([((T, parts, 3), torch.float32)] if stats else [])
    bufs, outs = zip(*(_guarded(s, dt) for s, dt in shapes))
    outs = tuple(outs) + (() if stats else (None,))
    wbuf, ws = _guarded((tpr.vocab_parallel_ce_workspace_bytes(parts, T, V),), torch.uint8)
    got = tpr.vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=stats, out=outs, workspace=ws)
    _check_guards(bufs + (wbuf,))
    ref = tpr.vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=stats)
    for a, b in zip(got, ref):
        if a is not None:
            assert torch.equal(a, b)


@pytest.mark.parametrize("T,V,vv,eps", [(37, 1000, 997, 0.1), (6, 8 * 11364, 8 * 11364 - 11, 0.0)])
def test_ce_opts_guard_bands(tpr, T, V, vv, eps):
    say("guard bands, CE options", T, V, vv, eps)
    logits, labels = workloads.vocab_ce_opts(T, V, vv, seed=T, device=DEV, ignore_frac=0.25)
    bufs, outs = zip(*(_guarded(s, dt) for s, dt in (((), torch.float32), ((T, V), torch.bfloat16))))
    wbuf, ws = _guarded((tpr.vocab_parallel_ce_opts_workspace_bytes(8, T, V),), torch.uint8)
    got = tpr.vocab_parallel_ce_opts_fwd_bwd(8, logits, labels, v_valid=vv, label_smoothing=eps,
                                             out=tuple(outs) + (None,), workspace=ws)
    _check_guards(bufs + (wbuf,))
    ref = tpr.vocab_parallel_ce_opts_fwd_bwd(8, logits, labels, v_valid=vv, label_smoothing=eps)
    assert torch.equal(got[1], ref[1])


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("parts", [3, 8, 2000])
def test_head_guard_bands(tpr, parts, layout):
    say("guard bands, vocab head + CE", parts, layout)
    T, d, V = 37, 64, 1003
    h, w, y = workloads.vocab_head(T, d, V, seed=parts, device=DEV, w_std=0.25, w_layout=layout)
    wshape = (d, V) if layout == "math" else (V, d)
    bufs, outs = zip(*(_guarded(s, torch.float32) for s in ((), (T, d), wshape)))
    nb = tpr.vocab_parallel_head_ce_workspace_bytes(parts, torch.bfloat16, T, d, V)
    wbuf, ws = _guarded((nb,), torch.uint8)
    got = tpr.vocab_parallel_head_ce_fwd_bwd(parts, h, w, y, w_layout=layout, out=outs, workspace=ws)
    _check_guards(bufs + (wbuf,))
    ref = tpr.vocab_parallel_head_ce_fwd_bwd(parts, h, w, y, w_layout=layout)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)


@pytest.mark.parametrize("tp,hq,hkv,dh", [(2, 8, 2, 16), (3, 6, 3, 12)])
def test_attn_proj_guard_bands(tpr, tp, hq, hkv, dh):
    say("guard bands, attention projections", tp, hq, hkv, dh)
    T, d = 272, 320
    g = torch.Generator(device=DEV)
    g.manual_seed(tp)
    nq, nkv = hq * dh, hkv * dh
    nqkv = nq + 2 * nkv
    mk = lambda shape, std: (torch.randn(shape, generator=g, device=DEV) * std).bfloat16()
    x, gy, ctx, dqkv = mk((T, d), 1), mk((T, d), 1), mk((T, nq), 1), mk((T, nqkv), 1)
    wq, wo = mk((d, nqkv), 0.05), mk((nq, d), 0.05)
    shapes = [((T, nqkv), torch.bfloat16), ((T, d), torch.float32), ((T, nq), torch.bfloat16),
              ((T, d), torch.float32), ((d, nqkv), torch.float32), ((nq, d), torch.float32)]
    bufs, outs = zip(*(_guarded(s, dt) for s, dt in shapes))
    nb = tpr.tp_attn_proj_workspace_bytes(tp, torch.bfloat16, T, d, hq, hkv, dh)
    wbuf, ws = _guarded((nb,), torch.uint8)
    got = tpr.tp_attn_proj_fwd_bwd(tp, x, wq, wo, ctx, gy, dqkv, hq, hkv, dh, out=outs, workspace=ws)
    _check_guards(bufs + (wbuf,))
    ref = tpr.tp_attn_proj_fwd_bwd(tp, x, wq, wo, ctx, gy, dqkv, hq, hkv, dh)
    for a, b in zip(got, ref):
        assert torch.equal(a, b)
