"""The C ABI library on the CPU: it loads, exports what the header declares,
its host-side shard planner matches the oracle bit for bit, and it rejects
invalid arguments before touching the GPU (CPU only, no compute calls)."""
import ctypes
import os
import re

import pytest

import oracle
from megatron_mlp_fwd_amd import binding

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "tprank.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(binding.LIB_PATH):
        pytest.skip("libtprank.so is not built")
    return binding.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("sharded_matmul_fwd_bwd", "tp_mlp_fwd_bwd", "vocab_parallel_ce_fwd_bwd", "tprank_shard_range",
              "tprank_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
        ctypes.cast(getattr(lib, name), ctypes.c_void_p)


def test_shard_range_matches_oracle_bit_for_bit(lib):
    for n in list(range(0, 40)) + [128256, 14336, 28672, 8192, 1792, 3584, 2**31 - 1]:
        for parts in list(range(1, 20)) + [64, 1000]:
            want = oracle.shard_ranges(n, parts)
            got = [binding.shard_range(n, parts, r) for r in range(parts)]
            assert got == want, (n, parts)


def test_walkthrough_split(lib):
    assert [binding.shard_range(5, 2, r) for r in range(2)] == [(0, 3), (3, 5)]


@pytest.mark.parametrize("args,code", [
    ((-1, 2, 0), binding.TPR_ERR_SHAPE),
    ((5, 0, 0), binding.TPR_ERR_PARTITION),
    ((5, 2, 2), binding.TPR_ERR_PARTITION),
    ((5, 2, -1), binding.TPR_ERR_PARTITION),
])
def test_shard_range_errors(lib, args, code):
    b, e = ctypes.c_int64(), ctypes.c_int64()
    assert lib.tprank_shard_range(*args, ctypes.byref(b), ctypes.byref(e)) == code
    assert lib.tprank_last_error()


def test_workspace_sizes(lib):
    assert lib.sharded_matmul_workspace_bytes(0, 1, 0, 3, 5, 4) == 0
    assert lib.sharded_matmul_workspace_bytes(0, 2, 0, 3, 5, 4) == 2 * 256     # rows: dB partials 5 x 4 fp32
    assert lib.sharded_matmul_workspace_bytes(2, 8, 1, 8192, 8192, 8192) == 8 * 8192 * 8192 * 4
    assert lib.sharded_matmul_workspace_bytes(3, 2, 0, 3, 5, 4) == 0            # invalid axis
    # bf16: sigma'(P) / dZ and H; 448 fc1 tiles leave 64 compute units free, too few for dH's 448
    assert lib.tp_mlp_workspace_bytes(1, 1, 8192, 8192, 3584) == 2 * 8192 * 3584 * 2
    # 8B rank: 112 fc1 tiles leave room for all 112 dH tiles; fc1's P and dH kept in fp32 (T x f each)
    assert lib.tp_mlp_workspace_bytes(1, 1, 4096, 4096, 1792) == 2 * 4096 * 1792 * 2 + 2 * 4096 * 1792 * 4
    assert lib.tp_mlp_workspace_bytes(4, 0, 16, 64, 256) == 2 * 16 * 256 * 4 + 2 * 4 * 16 * 64 * 4
    assert lib.vocab_parallel_ce_workspace_bytes(8, 4096, 128256) == 4096 * 4


N = None


def test_sharded_matmul_rejects_bad_arguments(lib):
    f = lib.sharded_matmul_fwd_bwd
    assert f(0, 1, 0, -1, 5, 4, N, N, N, N, N, N, N, 0, N) == binding.TPR_ERR_SHAPE
    assert f(0, 0, 0, 3, 5, 4, N, N, N, N, N, N, N, 0, N) == binding.TPR_ERR_PARTITION
    assert f(3, 2, 0, 3, 5, 4, N, N, N, N, N, N, N, 0, N) == binding.TPR_ERR_PARTITION
    assert f(0, 2, 7, 3, 5, 4, N, N, N, N, N, N, N, 0, N) == binding.TPR_ERR_DTYPE
    assert f(0, 2, 0, 3, 5, 4, N, N, N, N, N, N, N, 0, N) == binding.TPR_ERR_NULLPTR
    p = ctypes.c_void_p(16)  # never dereferenced: validation stops first
    assert f(0, 2, 0, 3, 5, 4, p, p, p, p, p, p, N, 0, N) == binding.TPR_ERR_WORKSPACE
    assert b"workspace" in lib.tprank_last_error()


def test_mlp_and_ce_reject_bad_arguments(lib):
    g = lib.tp_mlp_fwd_bwd
    assert g(1, 1, 0, -2, 4, 4, *[N] * 8, N, 0, N) == binding.TPR_ERR_SHAPE
    assert g(0, 1, 0, 2, 4, 4, *[N] * 8, N, 0, N) == binding.TPR_ERR_PARTITION
    assert g(1, 1, 5, 2, 4, 4, *[N] * 8, N, 0, N) == binding.TPR_ERR_DTYPE
    assert g(1, 1, 0, 2, 4, 4, *[N] * 8, N, 0, N) == binding.TPR_ERR_NULLPTR
    h = lib.vocab_parallel_ce_fwd_bwd
    assert h(1, 1, 4, 8, N, N, N, N, N, N, 0, N) == binding.TPR_ERR_NULLPTR
    p = ctypes.c_void_p(16)
    assert h(1, 1, 4, 0, p, p, p, p, N, N, 0, N) == binding.TPR_ERR_SHAPE
    assert h(0, 1, 4, 8, p, p, p, p, N, N, 0, N) == binding.TPR_ERR_PARTITION
    assert h(2, 9, 4, 8, p, p, p, p, N, N, 0, N) == binding.TPR_ERR_DTYPE
    assert h(2, 1, 4, 8, p, p, p, p, N, N, 0, N) == binding.TPR_ERR_WORKSPACE


def test_partial_sum_rejects_bad_arguments(lib):
    f = lib.tprank_partial_sum
    p = ctypes.c_void_p(1 << 20)  # never dereferenced: validation stops first
    assert f(2, -1, p, 8, p, N) == binding.TPR_ERR_SHAPE
    assert f(-1, 8, p, 8, p, N) == binding.TPR_ERR_SHAPE
    assert f(2, 8, p, 7, p, N) == binding.TPR_ERR_SHAPE              # slots overlap each other
    assert f(2, 8, N, 8, p, N) == binding.TPR_ERR_NULLPTR
    assert f(2, 8, p, 8, N, N) == binding.TPR_ERR_NULLPTR
    out = ctypes.c_void_p((1 << 20) + 4 * 12)                       # inside the second slot
    assert f(2, 8, p, 8, out, N) == binding.TPR_ERR_VALUE
    assert b"overlaps" in lib.tprank_last_error()
    assert f(2, 0, N, 0, N, N) == binding.TPR_OK                     # nothing to do, nothing enqueued


def test_ce_noalloc_rejects_bad_arguments(lib):
    f = lib.vocab_parallel_ce_fwd_bwd_noalloc
    p = ctypes.c_void_p(16)  # never dereferenced: validation stops first
    assert f(1, 1, 4, 8, N, N, N, N, N, N) == binding.TPR_ERR_NULLPTR
    assert f(0, 1, 4, 8, p, p, p, p, N, N) == binding.TPR_ERR_PARTITION
    assert f(2, 9, 4, 8, p, p, p, p, N, N) == binding.TPR_ERR_DTYPE
    assert f(1, 1, (1 << 18) + 1, 8, p, p, p, p, N, N) == binding.TPR_ERR_WORKSPACE   # beyond the static array
    assert b"static scratch" in lib.tprank_last_error()


def test_head_ce_workspace_and_bad_arguments(lib):
    ws = lib.vocab_parallel_head_ce_workspace_bytes
    # logits + dlogits (bf16), row losses, and 8 fp32 partials of dh
    assert ws(8, 1, 4096, 4096, 128256) == 2 * 4096 * 128256 * 2 + 4096 * 4 + 8 * 4096 * 4096 * 4
    assert ws(1, 0, 3, 5, 7) == 2 * 256 + 256                                    # fp32, one rank: no partials
    assert ws(0, 1, 3, 5, 7) == 0                                               # invalid parts
    f = lib.vocab_parallel_head_ce_fwd_bwd
    p = ctypes.c_void_p(16)  # never dereferenced: validation stops first
    assert f(2, 1, 0, -1, 4, 8, *[p] * 6, N, 0, N) == binding.TPR_ERR_SHAPE
    assert f(2, 1, 0, 3, 4, 0, *[p] * 6, N, 0, N) == binding.TPR_ERR_SHAPE       # V = 0 with T > 0
    assert f(0, 1, 0, 3, 4, 8, *[p] * 6, N, 0, N) == binding.TPR_ERR_PARTITION
    assert f(2, 7, 0, 3, 4, 8, *[p] * 6, N, 0, N) == binding.TPR_ERR_DTYPE
    assert f(2, 1, 5, 3, 4, 8, *[p] * 6, N, 0, N) == binding.TPR_ERR_DTYPE       # w_layout
    assert f(2, 1, 0, 3, 4, 8, p, p, p, N, p, p, N, 0, N) == binding.TPR_ERR_NULLPTR
    assert f(2, 1, 0, 3, 4, 8, *[p] * 6, N, 0, N) == binding.TPR_ERR_WORKSPACE
    assert b"workspace" in lib.tprank_last_error()


def test_ce_opts_workspace_and_bad_arguments(lib):
    ws = lib.vocab_parallel_ce_opts_workspace_bytes
    assert ws(8, 4096, 128256) == 4096 * 4 + 256   # row losses, then the counted-row total
    assert ws(1, 3, 5) == 256 + 256
    assert ws(0, 3, 5) == 0
    f = lib.vocab_parallel_ce_opts_fwd_bwd
    p = ctypes.c_void_p(16)  # never dereferenced: validation stops first
    ign = binding.NO_IGNORE
    assert f(2, 1, -1, 8, 8, ign, 0.0, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_SHAPE
    assert f(2, 1, 3, 8, 9, ign, 0.0, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_SHAPE      # v_valid > V
    assert f(2, 1, 3, 8, 0, ign, 0.0, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_SHAPE      # v_valid < 1
    assert f(0, 1, 3, 8, 8, ign, 0.0, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_PARTITION
    assert f(2, 9, 3, 8, 8, ign, 0.0, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_DTYPE
    assert f(2, 1, 3, 8, 8, ign, 1.5, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_VALUE
    assert f(2, 1, 3, 8, 8, ign, -0.1, p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_VALUE
    assert f(2, 1, 3, 8, 8, ign, float("nan"), p, p, p, p, N, p, 4096, N) == binding.TPR_ERR_VALUE
    assert b"label_smoothing" in lib.tprank_last_error()
    assert f(2, 1, 3, 8, 8, ign, 0.1, p, N, p, p, N, p, 4096, N) == binding.TPR_ERR_NULLPTR
    assert f(2, 1, 3, 8, 8, ign, 0.1, p, p, p, p, N, p, 16, N) == binding.TPR_ERR_WORKSPACE
    assert f(2, 1, 3, 8, 8, ign, 0.1, p, p, p, p, N, N, 4096, N) == binding.TPR_ERR_WORKSPACE


def test_mlp_act_workspace_and_bad_arguments(lib):
    ws = lib.tp_mlp_act_workspace_bytes
    T, d, f = 8192, 8192, 3584
    assert ws(1, 1, 0, T, d, f) == lib.tp_mlp_workspace_bytes(1, 1, T, d, f)
    # gated: gate, up, H, [dA | dU] (T x f each, bf16), [W1_r | W3_r] (d x 2f), y / dx partials when tp > 1
    assert ws(1, 1, 1, T, d, f) == 5 * T * f * 2 + d * 2 * f * 2
    assert ws(4, 1, 1, T, d, f) == 5 * T * f * 2 + d * 2 * f * 2 + 2 * 4 * T * d * 4
    assert ws(0, 1, 1, T, d, f) == 0
    fn = lib.tp_mlp_act_fwd_bwd
    p = ctypes.c_void_p(16)  # never dereferenced: validation stops first
    args = lambda act, w3, dw3: (1, 1, 0, act, 4, 8, 6, p, p, w3, p, p, p, p, p, dw3, p, p, 1 << 20, N)
    assert fn(*args(3, N, N)) == binding.TPR_ERR_VALUE
    assert b"activation" in lib.tprank_last_error()
    assert fn(*args(-1, N, N)) == binding.TPR_ERR_VALUE
    assert fn(*args(2, p, N)) == binding.TPR_ERR_NULLPTR                      # gated without dw3
    a = list(args(2, p, p))
    a[18] = 16
    assert fn(*a) == binding.TPR_ERR_WORKSPACE


def test_binding_signatures_match_the_header():
    # Every ctypes signature has as many arguments as the header's prototype.
    text = re.sub(r"/\*.*?\*/", "", open(HEADER).read(), flags=re.S)
    protos = {m.group(1): m.group(2) for m in
              re.finditer(r"^\s*(?:const\s+)?\w+\*?\s+\*?(\w+)\s*\(([^)]*)\)\s*;", text, flags=re.M | re.S)}
    for name, (_, args) in binding._SIGS.items():
        params = protos[name].strip()
        n = 0 if params in ("", "void") else params.count(",") + 1
        assert len(args) == n, (name, len(args), n)


def test_attn_proj_workspace_and_bad_arguments(lib):
    ws = lib.tp_attn_proj_workspace_bytes
    assert ws(1, 1, 8192, 8192, 8, 1, 128) == 0
    assert ws(8, 1, 4096, 4096, 32, 8, 128) == 2 * 8 * 4096 * 4096 * 4
    assert ws(8, 1, 4096, 4096, 32, 8, 0) == 0
    f = lib.tp_attn_proj_fwd_bwd
    p = ctypes.c_void_p(16)  # never dereferenced: validation stops first
    call = lambda tp, hq, hkv, dh, dtype=1, layout=0, wsb=1 << 30: f(tp, dtype, layout, 4, 8, hq, hkv, dh,
                                                                      *[p] * 12, p, wsb, N)
    assert call(16, 32, 8, 4) == binding.TPR_ERR_PARTITION      # KV heads not divisible (no replication)
    assert b"KV heads" in lib.tprank_last_error()
    assert call(3, 32, 8, 4) == binding.TPR_ERR_PARTITION
    assert call(0, 32, 8, 4) == binding.TPR_ERR_PARTITION
    assert call(2, 12, 8, 4) == binding.TPR_ERR_SHAPE           # query heads not a multiple of KV heads
    assert call(2, 8, 8, 0) == binding.TPR_ERR_SHAPE
    assert call(2, 8, 8, 4, dtype=5) == binding.TPR_ERR_DTYPE
    assert call(2, 8, 8, 4, layout=2) == binding.TPR_ERR_DTYPE
    assert call(2, 8, 8, 4, wsb=16) == binding.TPR_ERR_WORKSPACE


def _no_gpu():
    try:
        import torch
        return not torch.cuda.is_available()
    except Exception:
        return True


@pytest.mark.skipif(not _no_gpu(), reason="walks the planner with placeholder pointers: only where no GPU is visible")
def test_planner_runs_to_the_first_launch_without_a_device(lib):
    # Valid sizes, 256-byte aligned placeholder pointers that the host never
    # dereferences: each entry point validates, plans its shards, carves its
    # workspace and builds its launches, then the first launch fails because
    # there is no device (TPR_ERR_HIP).  Under the host-sanitized build this
    # puts the whole planner, not only the error paths, under ASan.
    p = ctypes.c_void_p(1 << 32)
    big = 1 << 40
    for axis in (0, 1, 2):
        for dtype in (0, 1):
            for M, K, N, parts in ((3, 5, 4, 2), (3, 5, 4, 7), (300, 136, 520, 3), (8192, 1024, 8192, 8)):
                assert lib.sharded_matmul_fwd_bwd(axis, parts, dtype, M, K, N, p, p, p, p, p, p, p, big, N_) == \
                    binding.TPR_ERR_HIP, (axis, dtype, M, K, N, parts)
    for dtype in (0, 1):
        for tp, T, d, f in ((1, 8192, 8192, 3584), (1, 4096, 4096, 1792), (3, 300, 264, 200), (300, 64, 40, 24)):
            for layout in (0, 1):
                assert lib.tp_mlp_fwd_bwd(tp, dtype, layout, T, d, f, *[p] * 8, p, big, N_) == binding.TPR_ERR_HIP
                for act in (0, 1, 2):
                    for w3 in (N_, p):
                        assert lib.tp_mlp_act_fwd_bwd(tp, dtype, layout, act, T, d, f, p, p, w3, p, p, p, p, p, p, p,
                                                      p, big, N_) == binding.TPR_ERR_HIP
        for tp, hq, hkv, dh in ((1, 8, 1, 128), (2, 8, 2, 16), (8, 32, 8, 8)):
            assert lib.tp_attn_proj_fwd_bwd(tp, dtype, 0, 272, 320, hq, hkv, dh, *[p] * 12, p, big, N_) == \
                binding.TPR_ERR_HIP
        for parts, T, V in ((8, 4096, 128256), (3, 5, 1001), (300, 4, 100), (4, 3, 8 * 11264 + 24)):
            for stats in (N_, p):
                assert lib.vocab_parallel_ce_fwd_bwd(parts, dtype, T, V, p, p, p, p, stats, p, big, N_) == \
                    binding.TPR_ERR_HIP
                assert lib.vocab_parallel_ce_fwd_bwd_noalloc(parts, dtype, T, V, p, p, p, p, stats, N_) == \
                    binding.TPR_ERR_HIP
                assert lib.vocab_parallel_ce_opts_fwd_bwd(parts, dtype, T, V, V - 3, -100, 0.1, p, p, p, p, stats, p,
                                                          big, N_) == binding.TPR_ERR_HIP
            for layout in (0, 1):
                assert lib.vocab_parallel_head_ce_fwd_bwd(parts, dtype, layout, T, 64, V, p, p, p, p, p, p, p, big,
                                                          N_) == binding.TPR_ERR_HIP
    assert lib.tprank_partial_sum(8, 8192 * 8192, p, 8192 * 8192, ctypes.c_void_p(1 << 44), N_) == binding.TPR_ERR_HIP


N_ = None
