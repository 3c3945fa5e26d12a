"""GPU parity of the tensor-parallel attention-block projections through the
C ABI, against the fp64 oracle.  Tolerances as for the sharded GEMM: max
|gpu - oracle| per output within 1e-5 (fp32 inputs) or 2e-2 (bf16 inputs,
outputs in bf16 rounded once) of max |oracle|; the oracle sees the values
the GPU sees."""
import sys

import numpy as np
import pytest
import torch

from oracle.attn_proj import attn_proj_fwd_bwd, fuse_qkv, split_qkv

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


def _inputs(T, d, hq, hkv, dh, dtype, seed, w_std):
    g = torch.Generator(device=DEV)
    g.manual_seed(seed)
    mk = lambda shape, std: (torch.randn(shape, generator=g, device=DEV) * std).to(dtype)
    nq, nkv = hq * dh, hkv * dh
    return dict(x=mk((T, d), 1.0), wq=mk((d, nq), w_std), wk=mk((d, nkv), w_std), wv=mk((d, nkv), w_std),
                wo=mk((nq, d), w_std), ctx=mk((T, nq), 1.0), gy=mk((T, d), 1.0), dq=mk((T, nq), 1.0),
                dk=mk((T, nkv), 1.0), dv=mk((T, nkv), 1.0))


def run(tpr, c, tp, hq, hkv, dh, layout):
    fuse = lambda a, b, cc: torch.from_numpy(fuse_qkv(f64(a), f64(b), f64(cc), tp, hq, hkv, dh)).to(a.dtype).to(DEV)
    w_qkv = fuse(c["wq"], c["wk"], c["wv"]).contiguous()
    dqkv = fuse(c["dq"], c["dk"], c["dv"]).contiguous()
    w_o = c["wo"]
    if layout == "torch":
        w_qkv, w_o = w_qkv.t().contiguous(), w_o.t().contiguous()
    out = tpr.tp_attn_proj_fwd_bwd(tp, c["x"], w_qkv, w_o, c["ctx"], c["gy"], dqkv, hq, hkv, dh, w_layout=layout)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("layout", ["math", "torch"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("tp,hq,hkv,dh", [(1, 4, 2, 16), (2, 8, 2, 16), (4, 8, 4, 8), (8, 32, 8, 8), (3, 6, 3, 12)])
def test_attn_proj(tpr, dtype, layout, tp, hq, hkv, dh):
    T, d = (272, 320) if dtype == torch.bfloat16 else (40, 64)
    say("attention projections", dtype, layout, "tp", tp, "heads", hq, hkv, dh, (T, d))
    c = _inputs(T, d, hq, hkv, dh, dtype, seed=tp * 100 + hq, w_std=0.05)
    qkv, y, dctx, dx, dwq, dwo = run(tpr, c, tp, hq, hkv, dh, layout)
    want = attn_proj_fwd_bwd(**{k: f64(v) for k, v in c.items()})
    tol = 1e-5 if dtype == torch.float32 else 2e-2
    q, k, v = split_qkv(f64(qkv), tp, hq, hkv, dh)
    dq_, dk_, dv_ = split_qkv(f64(dwq if layout == "math" else dwq.t()), tp, hq, hkv, dh)
    got = dict(q=q, k=k, v=v, y=f64(y), dctx=f64(dctx), dx=f64(dx), dwq=dq_, dwk=dk_, dwv=dv_,
               dwo=f64(dwo if layout == "math" else dwo.t()))
    for name, w in want.items():
        e = rel_err(got[name], w)
        assert e <= tol, (name, e)


def test_attn_proj_llama3_70b_rank_full(tpr):
    # One Llama-3-70B rank at TP = 8: 8 query heads and 1 KV head of 128;
    # every element of every output against the fp64 oracle.
    T, d, hq, hkv, dh = 8192, 8192, 8, 1, 128
    say("attention projections 70B rank, every element", (T, d, hq, hkv, dh))
    c = _inputs(T, d, hq, hkv, dh, torch.bfloat16, seed=7, w_std=0.02)
    qkv, y, dctx, dx, dwq, dwo = run(tpr, c, 1, hq, hkv, dh, "math")
    want = attn_proj_fwd_bwd(**{k: f64(v) for k, v in c.items()})
    q, k, v = split_qkv(f64(qkv), 1, hq, hkv, dh)
    dq_, dk_, dv_ = split_qkv(f64(dwq), 1, hq, hkv, dh)
    got = dict(q=q, k=k, v=v, y=f64(y), dctx=f64(dctx), dx=f64(dx), dwq=dq_, dwk=dk_, dwv=dv_, dwo=f64(dwo))
    for name, w in want.items():
        e = rel_err(got[name], w)
        say(name, "rel err", e)
        assert e <= 2e-2, (name, e)
