"""Pins for the oracle's tensor-parallel attention projections (CPU only)."""
import numpy as np
import pytest
import torch

from oracle.attn_proj import attn_proj_fwd_bwd, check_heads, fuse_qkv, split_qkv, tp_attn_proj_fwd_bwd


def _case(T, d, hq, hkv, dh, seed):
    rng = np.random.default_rng(seed)
    n = lambda *s: rng.standard_normal(s)
    return dict(x=n(T, d), wq=n(d, hq * dh), wk=n(d, hkv * dh), wv=n(d, hkv * dh), wo=n(hq * dh, d),
                ctx=n(T, hq * dh), gy=n(T, d), dq=n(T, hq * dh), dk=n(T, hkv * dh), dv=n(T, hkv * dh))


def test_against_torch_autograd():
    # The projections as torch ops; the core's gradients dQ, dK, dV and the
    # block gradient gy enter as upstream gradients of Q, K, V and y.
    c = _case(7, 12, 4, 2, 3, seed=0)
    t = {k: torch.tensor(v, dtype=torch.float64, requires_grad=True) for k, v in c.items()}
    q, k, v = t["x"] @ t["wq"], t["x"] @ t["wk"], t["x"] @ t["wv"]
    y = t["ctx"] @ t["wo"]
    loss = (q * t["dq"]).sum() + (k * t["dk"]).sum() + (v * t["dv"]).sum() + (y * t["gy"]).sum()
    loss.backward()
    got = attn_proj_fwd_bwd(**c)
    for name, want in (("q", q), ("k", k), ("v", v), ("y", y)):
        np.testing.assert_allclose(got[name], want.detach().numpy(), rtol=1e-13, atol=1e-13)
    for name, key in (("dx", "x"), ("dwq", "wq"), ("dwk", "wk"), ("dwv", "wv"), ("dwo", "wo"), ("dctx", "ctx")):
        np.testing.assert_allclose(got[name], t[key].grad.numpy(), rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("tp,hq,hkv", [(1, 4, 2), (2, 4, 2), (2, 8, 2), (4, 8, 4), (8, 32, 8), (3, 6, 3)])
def test_sharded_equals_unsharded(tp, hq, hkv):
    c = _case(5, 16, hq, hkv, 2, seed=tp * 10 + hq)
    a = attn_proj_fwd_bwd(**c)
    b = tp_attn_proj_fwd_bwd(**c, tp=tp, n_q_heads=hq, n_kv_heads=hkv, head_dim=2)
    for key in a:
        np.testing.assert_allclose(b[key], a[key], rtol=1e-12, atol=1e-12)


def test_dropping_one_rank_breaks_the_sum():
    c = _case(5, 8, 4, 2, 2, seed=3)
    full = tp_attn_proj_fwd_bwd(**c, tp=2, n_q_heads=4, n_kv_heads=2, head_dim=2)
    # rank 1's partial of y alone: ctx[:, 4:8] W_O[4:8]
    part = c["ctx"][:, 4:] @ c["wo"][4:]
    assert np.abs(full["y"] - part).max() > 1e-3


def test_heads_per_rank_of_the_pages_example():
    # Llama-3-8B: 32 query heads, 8 KV heads.  tp = 8 gives 4 and 1 per rank;
    # tp = 16 cannot divide the KV heads.
    assert check_heads(8, 32, 8) == (4, 1)
    assert check_heads(4, 32, 8) == (8, 2)
    with pytest.raises(ValueError, match="partition"):
        check_heads(16, 32, 8)
    with pytest.raises(ValueError, match="partition"):
        check_heads(3, 32, 8)
    with pytest.raises(ValueError, match="shape"):
        check_heads(1, 12, 8)       # query heads not a multiple of KV heads
    with pytest.raises(ValueError, match="partition"):
        check_heads(0, 8, 8)


def test_fused_layout():
    hq, hkv, dh, tp = 8, 2, 3, 2
    wq = np.arange(hq * dh)[None, :] + 0.0
    wk = 100 + np.arange(hkv * dh)[None, :] + 0.0
    wv = 200 + np.arange(hkv * dh)[None, :] + 0.0
    f = fuse_qkv(wq, wk, wv, tp, hq, hkv, dh)
    # rank 0: Q heads 0-3 (cols 0-11), K head 0 (100-102), V head 0 (200-202)
    want0 = list(range(12)) + [100, 101, 102, 200, 201, 202]
    want1 = list(range(12, 24)) + [103, 104, 105, 203, 204, 205]
    assert f[0].tolist() == want0 + want1
    q, k, v = split_qkv(f, tp, hq, hkv, dh)
    np.testing.assert_array_equal(q, wq)
    np.testing.assert_array_equal(k, wk)
    np.testing.assert_array_equal(v, wv)


def test_rank_share_is_tp1_on_rank_shards():
    # One rank's share at tp = 8 equals the tp = 1 computation on its shards.
    hq, hkv, dh, tp = 16, 8, 2, 8
    c = _case(4, 6, hq, hkv, dh, seed=9)
    full = tp_attn_proj_fwd_bwd(**c, tp=tp, n_q_heads=hq, n_kv_heads=hkv, head_dim=dh)
    r, qw, kw = 3, 2 * dh, 1 * dh
    sl = dict(x=c["x"], wq=c["wq"][:, r * qw:(r + 1) * qw], wk=c["wk"][:, r * kw:(r + 1) * kw],
              wv=c["wv"][:, r * kw:(r + 1) * kw], wo=c["wo"][r * qw:(r + 1) * qw], ctx=c["ctx"][:, r * qw:(r + 1) * qw],
              gy=c["gy"], dq=c["dq"][:, r * qw:(r + 1) * qw], dk=c["dk"][:, r * kw:(r + 1) * kw],
              dv=c["dv"][:, r * kw:(r + 1) * kw])
    one = attn_proj_fwd_bwd(**sl)
    np.testing.assert_allclose(one["q"], full["q"][:, r * qw:(r + 1) * qw], rtol=1e-14)
    np.testing.assert_allclose(one["dwo"], full["dwo"][r * qw:(r + 1) * qw], rtol=1e-14)
    np.testing.assert_allclose(one["dctx"], full["dctx"][:, r * qw:(r + 1) * qw], rtol=1e-14)


def test_errors():
    c = _case(3, 4, 2, 1, 2, seed=1)
    bad = dict(c, ctx=c["ctx"][:, :3])
    with pytest.raises(ValueError, match="shape"):
        attn_proj_fwd_bwd(**bad)
    with pytest.raises(ValueError, match="shape"):
        tp_attn_proj_fwd_bwd(**c, tp=1, n_q_heads=2, n_kv_heads=1, head_dim=3)
