"""GPU parity of the MLP with tanh / SiLU activations and of the gated
(gate / up) MLP through the C ABI, against the fp64 oracle.

Tolerances as for the GELU MLP: max |gpu - oracle| per output tensor within
1e-5 (fp32 inputs) or 2e-2 (bf16 inputs) of max |oracle|.  With bf16 inputs
the GPU rounds the GEMM operands it produces (H, the pre-activation
gradients, and for the gated MLP also A and U) to bf16; the oracle rounds
nothing.
"""
import sys

import numpy as np
import pytest
import torch

import workloads
from oracle.mlp_act import mlp_act_fwd_bwd

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, want):
    scale = float(np.abs(want).max()) if want.size else 0.0
    diff = float(np.abs(got - want).max()) if want.size else 0.0
    return diff / scale if scale > 0 else diff


@pytest.fixture(scope="module")
def tpr():
    import megatron_mlp_fwd_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


def _weights(d, f, seed, dtype, layout, gated, std):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    mk = lambda shape: (torch.randn(shape, generator=g, device=DEV) * std).to(dtype)
    w1 = mk((d, f) if layout == "math" else (f, d))
    w3 = mk((d, f) if layout == "math" else (f, d)) if gated else None
    w2 = mk((f, d) if layout == "math" else (d, f))
    return w1, w2, w3


@pytest.mark.parametrize("tp", [1, 3])
@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("act", ["gelu", "tanh", "silu"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_mlp_act(tpr, dtype, act, gated, layout, tp):
    # bf16: several 256 x 256 tiles with ragged edges; fp32: the TP lesson's
    # self-test sizes.
    T, d, f = (272, 320, 264) if dtype == torch.bfloat16 else (16, 64, 256)
    say("MLP", act, "gated" if gated else "plain", dtype, layout, "tp", tp, (T, d, f))
    x, _, _, gy = workloads.rank_mlp(T, d, 8, seed=T + tp, device=DEV, dtype=dtype)
    std = 1.0 / d ** 0.5 if dtype == torch.float32 else 0.05
    w1, w2, w3 = _weights(d, f, seed=7 * tp + gated, dtype=dtype, layout=layout, gated=gated, std=std)
    got = tpr.tp_mlp_act_fwd_bwd(tp, x, w1, w2, gy, act=act, w3=w3, w_layout=layout)
    torch.cuda.synchronize()
    want = mlp_act_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), act, None if w3 is None else f64(w3), layout)
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    for name, g, w in zip(("y", "dx", "dw1", "dw2", "dw3"), got, want):
        if w is None:
            assert g is None
            continue
        e = rel_err(f64(g), w)
        assert e <= tol, (name, e)


@pytest.mark.parametrize("tp", [1, 3])
@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("act", ["gelu", "tanh", "silu"])
def test_mlp_act_bf16_fc1_fills_the_chip(tpr, act, layout, tp):
    # T = 1024, f = 16384: fc1 alone fills whole rounds of the 256 compute
    # units (tp 1: 4 x 64 = 256 tiles; tp 3: 4 x 66 = 264 tiles, whose second
    # round leaves room for 3 of dH's 4 row blocks only), so dH does not join
    # the fc1 launch: fc1 takes the activation epilogue (sigma and sigma' from
    # the accumulator) and dH the multiplying one.  The smaller shapes above
    # take the other schedule (fp32 P and dH, then one element-wise pass).
    T, d, f = 1024, 128, 16384
    say("MLP bf16, fc1 fills the chip", act, layout, "tp", tp, (T, d, f))
    x, _, _, gy = workloads.rank_mlp(T, d, 8, seed=T + tp, device=DEV, dtype=torch.bfloat16)
    w1, w2, w3 = _weights(d, f, seed=11 * tp, dtype=torch.bfloat16, layout=layout, gated=False, std=0.05)
    got = tpr.tp_mlp_act_fwd_bwd(tp, x, w1, w2, gy, act=act, w_layout=layout)
    torch.cuda.synchronize()
    want = mlp_act_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), act, None, layout)
    for name, g, w in zip(("y", "dx", "dw1", "dw2"), got, want):
        e = rel_err(f64(g), w)
        assert e <= 2e-2, (name, e)


def test_gelu_act_matches_plain_entry_point(tpr):
    say("tp_mlp_act gelu == tp_mlp_fwd_bwd")
    x, w1, w2, gy = workloads.rank_mlp(300, 264, 200, seed=4, device=DEV)
    a = tpr.tp_mlp_fwd_bwd(3, x, w1, w2, gy)
    b = tpr.tp_mlp_act_fwd_bwd(3, x, w1, w2, gy, act="gelu")
    torch.cuda.synchronize()
    for p, q in zip(a, b[:4]):
        assert torch.equal(p, q)
    assert b[4] is None


def test_mlp_act_empty_shards(tpr):
    # tp = 5 > f = 3: two ranks hold no hidden units.
    say("gated SiLU MLP with empty ranks")
    x, _, _, gy = workloads.rank_mlp(40, 64, 8, seed=1, device=DEV, dtype=torch.float32)
    w1, w2, w3 = _weights(64, 3, seed=2, dtype=torch.float32, layout="math", gated=True, std=0.125)
    got = tpr.tp_mlp_act_fwd_bwd(5, x, w1, w2, gy, act="silu", w3=w3)
    torch.cuda.synchronize()
    want = mlp_act_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), "silu", f64(w3))
    for g, w in zip(got, want):
        assert rel_err(f64(g), w) <= 1e-5


@pytest.mark.parametrize("size", ["8b", "70b"])
def test_gated_silu_rank_full(tpr, size):
    # The Llama-3 rank MLP shapes (gate / up / down with SiLU at TP = 8),
    # every element of every output against the fp64 oracle (outputs start
    # as NaN, so a tile never written fails).
    T, d, f = (4096, 4096, 1792) if size == "8b" else (8192, 8192, 3584)
    say("gated SiLU rank MLP, every element", (T, d, f))
    x, _, _, gy = workloads.rank_mlp(T, d, 8, seed=5, device=DEV)
    w1, w2, w3 = _weights(d, f, seed=6, dtype=torch.bfloat16, layout="math", gated=True, std=0.02)
    nan = lambda *sh: torch.full(sh, float("nan"), device=DEV)
    out = (nan(T, d), nan(T, d), nan(d, f), nan(f, d), nan(d, f))
    got = tpr.tp_mlp_act_fwd_bwd(1, x, w1, w2, gy, act="silu", w3=w3, out=out)
    torch.cuda.synchronize()
    want = mlp_act_fwd_bwd(f64(x), f64(w1), f64(w2), f64(gy), "silu", f64(w3))
    for name, w, o in zip(("y", "dx", "dw1", "dw2", "dw3"), want, got):
        h = f64(o)
        assert not np.isnan(h).any(), name
        e = rel_err(h, w)
        say(name, "rel err", e)
        assert e <= 2e-2, (name, e)
    del got, out
    torch.cuda.empty_cache()