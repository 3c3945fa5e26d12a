"""Seeded synthetic inputs for the workloads of this library.

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the method's arithmetic, so both the oracle side and the HIP
side of a test can consume what it produces.  Every draw comes from a
``torch.Generator`` seeded explicitly, on the device the caller names (large
inputs are drawn on the GPU and copied to the host for the oracle).

Distributions (N(mu, s) means mean mu and standard deviation s):

* ``sharded_gemm_tiny``: fp32 A (M x K), B (K x N), G (M x N) ~ U[-1, 1];
  default M=3, K=5, N=4 as in the sharded GEMM page's walk-through.
* ``tp_mlp_tiny``: fp32 x (2, 8, 64), w1 (256, 64), w2 (64, 256) in the torch
  (out, in) layout and G (2, 8, 64), all ~ N(0, 1) -- the TP lesson page's
  self-test shapes.
* ``vocab_ce``: logits (T x V) = bf16(N(0, 2)), labels uniform in [0, V);
  default T=4096, V=128256 (a Llama-3-sized vocabulary).
* ``vocab_ce_opts``: as ``vocab_ce`` over V padded columns with labels
  uniform over the first v_valid, and a fraction (default 1/8) of the
  positions given the ignore label; the measured case is a 128000-entry
  vocabulary padded to 128256 with label smoothing 0.1.
* ``vocab_head``: hidden states h (T x d) ~ N(0, 1) and a vocabulary head
  W (d x V, or its transpose) ~ N(0, w_std), bf16.
* ``rank_mlp``: one tensor-parallel rank's share of a GELU MLP in the math
  layout: x (T x d) ~ N(0, 1), w1 (d x f) and w2 (f x d) ~ N(0, 0.02),
  G (T x d) ~ N(0, 1), rounded to bf16.  Llama-3-8B at TP=8 is T=4096,
  d=4096, f=1792; Llama-3-70B at TP=8 is T=8192, d=8192, f=3584.
* ``inner_gemm``: one rank's inner-axis shard A_r (M x K_r) ~ N(0, 1),
  B_r (K_r x N) ~ N(0, 0.02), G (M x N) ~ N(0, 1), bf16; the 70B rank uses
  M=8192, K_r=1024, N=8192.
"""

import torch


def _gen(device, seed):
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def _normal(shape, std, gen, device, dtype):
    t = torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def sharded_gemm_tiny(M=3, K=5, N=4, seed=0, device="cpu", dtype=torch.float32):
    g = _gen(device, seed)
    a = (torch.rand(M, K, generator=g, device=device) * 2 - 1).to(dtype)
    b = (torch.rand(K, N, generator=g, device=device) * 2 - 1).to(dtype)
    gy = (torch.rand(M, N, generator=g, device=device) * 2 - 1).to(dtype)
    return a, b, gy


def tp_mlp_tiny(seed=0, device="cpu", dtype=torch.float32, batch=(2, 8), d=64, f=256):
    g = _gen(device, seed)
    x = _normal((*batch, d), 1.0, g, device, dtype)
    w1 = _normal((f, d), 1.0, g, device, dtype)
    w2 = _normal((d, f), 1.0, g, device, dtype)
    gy = _normal((*batch, d), 1.0, g, device, dtype)
    return x, w1, w2, gy


def vocab_ce(T=4096, V=128256, seed=0, device="cpu", dtype=torch.bfloat16, std=2.0):
    g = _gen(device, seed)
    logits = _normal((T, V), std, g, device, dtype)
    labels = torch.randint(0, V, (T,), generator=g, device=device, dtype=torch.int64)
    return logits, labels


def vocab_ce_opts(T, V, v_valid, seed=0, device="cpu", dtype=torch.bfloat16, std=2.0, ignore_frac=0.125,
                  ignore_index=-100):
    """Logits like ``vocab_ce`` over a row of V columns of which the first
    v_valid are vocabulary (the padding columns hold the same N(0, std)
    draws), labels uniform over the vocabulary, and about ignore_frac of the
    positions labelled ignore_index."""
    g = _gen(device, seed)
    logits = _normal((T, V), std, g, device, dtype)
    labels = torch.randint(0, v_valid, (T,), generator=g, device=device, dtype=torch.int64)
    drop = torch.rand((T,), generator=g, device=device) < ignore_frac
    labels[drop] = ignore_index
    return logits, labels


def rank_mlp(T, d, f, seed=0, device="cpu", dtype=torch.bfloat16, w_std=0.02):
    g = _gen(device, seed)
    x = _normal((T, d), 1.0, g, device, dtype)
    w1 = _normal((d, f), w_std, g, device, dtype)
    w2 = _normal((f, d), w_std, g, device, dtype)
    gy = _normal((T, d), 1.0, g, device, dtype)
    return x, w1, w2, gy


def inner_gemm(M, K, N, seed=0, device="cpu", dtype=torch.bfloat16, b_std=0.02):
    g = _gen(device, seed)
    a = _normal((M, K), 1.0, g, device, dtype)
    b = _normal((K, N), b_std, g, device, dtype)
    gy = _normal((M, N), 1.0, g, device, dtype)
    return a, b, gy


def vocab_head(T, d, V, seed=0, device="cpu", dtype=torch.bfloat16, w_std=0.02, w_layout="math"):
    """Hidden states h ~ N(0, 1) (T x d), a vocabulary head W ~ N(0, w_std)
    (d x V, or V x d for the torch layout) and uniform labels."""
    g = _gen(device, seed)
    h = _normal((T, d), 1.0, g, device, dtype)
    w = _normal((d, V) if w_layout == "math" else (V, d), w_std, g, device, dtype)
    labels = torch.randint(0, V, (T,), generator=g, device=device, dtype=torch.int64)
    return h, w, labels


# The five workloads, by name and size.  ``kind`` says which entry point
# consumes them.
CONFIGS = {
    "sharded_gemm_m3k5n4": dict(kind="sharded_gemm", M=3, K=5, N=4, parts=(2, 7), dtype="f32"),
    "tp_mlp_tp4_x2x8x64": dict(kind="tp_mlp", tp=4, T=16, d=64, f=256, w_layout="torch", dtype="f32"),
    "vocab_ce_t4096_v128256_p8": dict(kind="vocab_ce", T=4096, V=128256, parts=8, dtype="bf16"),
    "llama3_8b_tp8_rank_mlp": dict(kind="tp_mlp", tp=1, T=4096, d=4096, f=1792, w_layout="math", dtype="bf16"),
    "llama3_70b_tp8_rank_mlp": dict(kind="tp_mlp", tp=1, T=8192, d=8192, f=3584, w_layout="math", dtype="bf16"),
    "llama3_70b_tp8_inner_gemm": dict(kind="sharded_gemm", M=8192, K=1024, N=8192, parts=(1,), axis="inner", dtype="bf16"),
    # next: cross-entropy options (a 128000-entry vocabulary padded to 128256, label smoothing 0.1,
    # one position in eight ignored)
    "vocab_ce_opts_t4096_v128256_p8": dict(kind="vocab_ce_opts", T=4096, V=128256, v_valid=128000, parts=8,
                                           label_smoothing=0.1, ignore_frac=0.125, dtype="bf16"),
    # next: the vocabulary-parallel output head in front of the CE (Llama-3-8B sizes)
    "llama3_8b_vocab_head_ce_p8": dict(kind="vocab_head_ce", T=4096, d=4096, V=128256, parts=8, dtype="bf16"),
}
