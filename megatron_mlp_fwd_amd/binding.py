"""ctypes binding of libtprank (include/tprank.h), same entry-point names.

Argument marshalling only: checks that tensors live on the GPU, are
contiguous and have the shapes and dtypes the C ABI expects (the library
cannot see buffer sizes), allocates outputs and the workspace with torch's
caching allocator on the stream the call launches on (``stream``, else the
current stream), and passes raw device pointers plus that HIP stream.
Every step of the computation runs in the library's HIP kernels; there is no
fallback of any kind -- if the library is missing, loading fails.
"""
import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# The in-tree library; TPRANK_LIB names another build of it (e.g. the
# host-sanitized variant that build.build_host_asan() makes).
LIB_PATH = os.environ.get("TPRANK_LIB") or os.path.join(_PKG, "libtprank.so")

(TPR_OK, TPR_ERR_SHAPE, TPR_ERR_PARTITION, TPR_ERR_DTYPE, TPR_ERR_WORKSPACE, TPR_ERR_NULLPTR, TPR_ERR_HIP,
 TPR_ERR_VALUE) = range(8)
NO_IGNORE = -(2 ** 63)  # an ignore_index no label takes: every row counts
AXES = {"rows": 0, "columns": 1, "inner": 2}
DTYPES = {torch.float32: 0, torch.bfloat16: 1}
W_LAYOUTS = {"math": 0, "torch": 1}
ACTS = {"gelu": 0, "tanh": 1, "silu": 2}

_lib = None

_i64, _i32, _vp, _sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
_SIGS = {
    "tprank_shard_range": (_i32, [_i64, _i32, _i32, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
    "sharded_matmul_workspace_bytes": (_sz, [_i32, _i32, _i32, _i64, _i64, _i64]),
    "sharded_matmul_fwd_bwd": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tp_mlp_workspace_bytes": (_sz, [_i32, _i32, _i64, _i64, _i64]),
    "tp_mlp_fwd_bwd": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "tp_mlp_act_workspace_bytes": (_sz, [_i32, _i32, _i32, _i64, _i64, _i64]),
    "tp_mlp_act_fwd_bwd": (_i32, [_i32, _i32, _i32, _i32, _i64, _i64, _i64] + [_vp] * 11 + [_sz, _vp]),
    "tp_attn_proj_workspace_bytes": (_sz, [_i32, _i32, _i64, _i64, _i32, _i32, _i32]),
    "tp_attn_proj_fwd_bwd": (_i32, [_i32, _i32, _i32, _i64, _i64, _i32, _i32, _i32] + [_vp] * 13 + [_sz, _vp]),
    "vocab_parallel_ce_workspace_bytes": (_sz, [_i32, _i64, _i64]),
    "vocab_parallel_ce_fwd_bwd": (_i32, [_i32, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _sz, _vp]),
    "vocab_parallel_ce_fwd_bwd_noalloc": (_i32, [_i32, _i32, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp]),
    "vocab_parallel_ce_opts_workspace_bytes": (_sz, [_i32, _i64, _i64]),
    "vocab_parallel_ce_opts_fwd_bwd": (_i32, [_i32, _i32, _i64, _i64, _i64, _i64, ctypes.c_float, _vp, _vp, _vp, _vp,
                                              _vp, _vp, _sz, _vp]),
    "vocab_parallel_head_ce_workspace_bytes": (_sz, [_i32, _i32, _i64, _i64, _i64]),
    "vocab_parallel_head_ce_fwd_bwd": (_i32, [_i32, _i32, _i32, _i64, _i64, _i64, _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                              _sz, _vp]),
    "tprank_partial_sum": (_i32, [_i32, _i64, _vp, _i64, _vp, _vp]),
    "tprank_last_error": (ctypes.c_char_p, []),
}


class TprError(RuntimeError):
    """A non-zero status from libtprank; ``code`` is the TPR_ERR_* value."""

    def __init__(self, code, msg):
        super().__init__(f"libtprank error {code}: {msg}")
        self.code = code


def load_library(path=LIB_PATH):
    """Load libtprank.so once (torch is imported first so that both share
    the HIP runtime already in the process)."""
    global _lib
    if _lib is None:
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run `python -m megatron_mlp_fwd_amd.build`")
        lib = ctypes.CDLL(path)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype, fn.argtypes = res, args
        _lib = lib
    return _lib


def _check(status):
    if status != TPR_OK:
        raise TprError(status, load_library().tprank_last_error().decode())


def _ptr(t):
    return None if t is None or t.numel() == 0 else t.data_ptr()


class _On:
    """Device and stream of one call.  Outputs and the workspace that the
    binding allocates are allocated on the stream the kernels are launched
    on: torch's caching allocator hands a freed block only to later
    allocations on the stream it was allocated on, so a workspace dropped
    when the call returns cannot be reused by another stream while the
    call's kernels still run on this one."""

    def __init__(self, device, stream):
        self.device = device
        with torch.cuda.device(device):
            self.stream = stream if stream is not None else torch.cuda.current_stream()
        self._ctx = None

    def __enter__(self):
        self._dev = torch.cuda.device(self.device)
        self._dev.__enter__()
        self._ctx = torch.cuda.stream(self.stream)
        self._ctx.__enter__()
        return self

    def __exit__(self, *exc):
        self._ctx.__exit__(*exc)
        self._dev.__exit__(*exc)
        return False

    @property
    def handle(self):
        return self.stream.cuda_stream


def _need(t, name, shape, dtype, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _workspace(nbytes, device, workspace):
    if nbytes == 0:
        return None, 0
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous() or workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError(f"workspace must be a contiguous tensor of >= {nbytes} bytes on {device}")
        return workspace, workspace.numel() * workspace.element_size()
    return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def shard_range(n, parts, rank):
    """[begin, end) of shard ``rank`` of ``n`` indices over ``parts`` shards."""
    b, e = _i64(), _i64()
    _check(load_library().tprank_shard_range(n, parts, rank, ctypes.byref(b), ctypes.byref(e)))
    return b.value, e.value


def sharded_matmul_workspace_bytes(axis, parts, dtype, M, K, N):
    return load_library().sharded_matmul_workspace_bytes(AXES.get(axis, axis), parts, DTYPES[dtype], M, K, N)


def sharded_matmul_fwd_bwd(axis, parts, A, B, G, out=None, workspace=None, stream=None):
    """Y = A B, dA = G B^T, dB = A^T G computed by ``parts`` simulated ranks
    split along ``axis`` ('rows', 'columns' or 'inner').  Returns fp32
    (Y, dA, dB); ``out`` may supply the three output tensors."""
    lib = load_library()
    ax = AXES[axis] if isinstance(axis, str) else int(axis)
    if A.dim() != 2 or B.dim() != 2:
        raise ValueError("A and B must be 2-D")
    M, K = A.shape
    N = B.shape[1]
    dt = A.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    dev = A.device
    _need(A, "A", (M, K), dt, dev)
    _need(B, "B", (K, N), dt, dev)
    _need(G, "G", (M, N), dt, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty(M, N, device=dev), torch.empty(M, K, device=dev), torch.empty(K, N, device=dev))
        Y, dA, dB = out
        _need(Y, "Y", (M, N), torch.float32, dev)
        _need(dA, "dA", (M, K), torch.float32, dev)
        _need(dB, "dB", (K, N), torch.float32, dev)
        ws, wsb = _workspace(lib.sharded_matmul_workspace_bytes(ax, parts, DTYPES[dt], M, K, N), dev, workspace)
        _check(lib.sharded_matmul_fwd_bwd(ax, parts, DTYPES[dt], M, K, N, _ptr(A), _ptr(B), _ptr(G), _ptr(Y),
                                          _ptr(dA), _ptr(dB), _ptr(ws), wsb, on.handle))
    return Y, dA, dB


def partial_sum(partials, out=None, stream=None):
    """Sum of the fp32 slots ``partials[0] + partials[1] + ...`` (the first
    dimension indexes the simulated ranks), added in slot order.  Returns
    ``out`` (shaped like one slot)."""
    lib = load_library()
    if partials.dim() < 1:
        raise ValueError("partials must have a slot dimension")
    nslots = partials.shape[0]
    shape = tuple(partials.shape[1:])
    dev = partials.device
    _need(partials, "partials", tuple(partials.shape), torch.float32, dev)
    n = 1
    for k in shape:
        n *= k
    with _On(dev, stream) as on:
        if out is None:
            out = torch.empty(shape, device=dev)
        _need(out, "out", shape, torch.float32, dev)
        _check(lib.tprank_partial_sum(nslots, n, _ptr(partials), n, _ptr(out), on.handle))
    return out


def tp_mlp_workspace_bytes(tp, dtype, T, d, f):
    return load_library().tp_mlp_workspace_bytes(tp, DTYPES[dtype], T, d, f)


def tp_mlp_fwd_bwd(tp, x, w1, w2, gy, w_layout="math", out=None, workspace=None, stream=None):
    """Column-then-row GELU MLP over ``tp`` simulated ranks, forward and
    backward for L = sum(y * gy).  ``x``/``gy`` are (..., d) with leading dims
    flattened into tokens.  Returns fp32 (y, dx, dw1, dw2) with y, dx shaped
    like x and dw1, dw2 like w1, w2."""
    lib = load_library()
    layout = W_LAYOUTS[w_layout]
    dt = x.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if w1.dim() != 2 or w2.dim() != 2:
        raise ValueError("w1 and w2 must be 2-D")
    d, f = (w1.shape[0], w1.shape[1]) if layout == 0 else (w1.shape[1], w1.shape[0])
    wshape1, wshape2 = ((d, f), (f, d)) if layout == 0 else ((f, d), (d, f))
    if x.dim() < 1 or x.shape[-1] != d:
        raise ValueError(f"x must be (..., {d})")
    T = 1
    for n in x.shape[:-1]:
        T *= n
    dev = x.device
    xs = tuple(x.shape)
    _need(x, "x", xs, dt, dev)
    _need(gy, "gy", xs, dt, dev)
    _need(w1, "w1", wshape1, dt, dev)
    _need(w2, "w2", wshape2, dt, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty(xs, device=dev), torch.empty(xs, device=dev),
                   torch.empty(wshape1, device=dev), torch.empty(wshape2, device=dev))
        y, dx, dw1, dw2 = out
        _need(y, "y", xs, torch.float32, dev)
        _need(dx, "dx", xs, torch.float32, dev)
        _need(dw1, "dw1", wshape1, torch.float32, dev)
        _need(dw2, "dw2", wshape2, torch.float32, dev)
        ws, wsb = _workspace(lib.tp_mlp_workspace_bytes(tp, DTYPES[dt], T, d, f), dev, workspace)
        _check(lib.tp_mlp_fwd_bwd(tp, DTYPES[dt], layout, T, d, f, _ptr(x), _ptr(w1), _ptr(w2), _ptr(gy), _ptr(y),
                                  _ptr(dx), _ptr(dw1), _ptr(dw2), _ptr(ws), wsb, on.handle))
    return y, dx, dw1, dw2


def tp_mlp_act_workspace_bytes(tp, dtype, gated, T, d, f):
    return load_library().tp_mlp_act_workspace_bytes(tp, DTYPES[dtype], int(bool(gated)), T, d, f)


def tp_mlp_act_fwd_bwd(tp, x, w1, w2, gy, act="gelu", w3=None, w_layout="math", out=None, workspace=None,
                       stream=None):
    """MLP over ``tp`` simulated ranks with activation ``act`` ("gelu",
    "tanh", "silu"), gated by the up projection ``w3`` (same shape and layout
    as ``w1``) when given.  Returns fp32 (y, dx, dw1, dw2, dw3) with dw3 None
    when not gated."""
    lib = load_library()
    layout = W_LAYOUTS[w_layout]
    if act not in ACTS:
        raise ValueError(f"unknown activation {act!r}")
    dt = x.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if w1.dim() != 2 or w2.dim() != 2:
        raise ValueError("w1 and w2 must be 2-D")
    d, f = (w1.shape[0], w1.shape[1]) if layout == 0 else (w1.shape[1], w1.shape[0])
    wshape1, wshape2 = ((d, f), (f, d)) if layout == 0 else ((f, d), (d, f))
    if x.dim() < 1 or x.shape[-1] != d:
        raise ValueError(f"x must be (..., {d})")
    T = 1
    for n in x.shape[:-1]:
        T *= n
    dev = x.device
    xs = tuple(x.shape)
    _need(x, "x", xs, dt, dev)
    _need(gy, "gy", xs, dt, dev)
    _need(w1, "w1", wshape1, dt, dev)
    _need(w2, "w2", wshape2, dt, dev)
    gated = w3 is not None
    if gated:
        _need(w3, "w3", wshape1, dt, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty(xs, device=dev), torch.empty(xs, device=dev), torch.empty(wshape1, device=dev),
                   torch.empty(wshape2, device=dev), torch.empty(wshape1, device=dev) if gated else None)
        y, dx, dw1, dw2, dw3 = out
        _need(y, "y", xs, torch.float32, dev)
        _need(dx, "dx", xs, torch.float32, dev)
        _need(dw1, "dw1", wshape1, torch.float32, dev)
        _need(dw2, "dw2", wshape2, torch.float32, dev)
        if gated:
            _need(dw3, "dw3", wshape1, torch.float32, dev)
        ws, wsb = _workspace(lib.tp_mlp_act_workspace_bytes(tp, DTYPES[dt], int(gated), T, d, f), dev, workspace)
        _check(lib.tp_mlp_act_fwd_bwd(tp, DTYPES[dt], layout, ACTS[act], T, d, f, _ptr(x), _ptr(w1), _ptr(w3),
                                      _ptr(w2), _ptr(gy), _ptr(y), _ptr(dx), _ptr(dw1), _ptr(dw3), _ptr(dw2),
                                      _ptr(ws), wsb, on.handle))
    return y, dx, dw1, dw2, dw3


def tp_attn_proj_workspace_bytes(tp, dtype, T, d, n_q_heads, n_kv_heads, head_dim):
    return load_library().tp_attn_proj_workspace_bytes(tp, DTYPES[dtype], T, d, n_q_heads, n_kv_heads, head_dim)


def tp_attn_proj_fwd_bwd(tp, x, w_qkv, w_o, ctx, gy, dqkv, n_q_heads, n_kv_heads, head_dim, w_layout="math",
                         out=None, workspace=None, stream=None):
    """Attention-block projections over ``tp`` simulated ranks: the fused
    QKV projection (rank-major column blocks of query, K and V heads) and
    the output projection, forward and backward, around an attention core
    whose context ``ctx`` and input gradient ``dqkv`` are given.  Returns
    (qkv, y, dctx, dx, dw_qkv, dw_o): qkv and dctx in the input dtype, the
    rest fp32."""
    lib = load_library()
    layout = W_LAYOUTS[w_layout]
    dt = x.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if x.dim() != 2:
        raise ValueError("x must be 2-D (tokens x d)")
    T, d = x.shape
    nq, nkv = n_q_heads * head_dim, n_kv_heads * head_dim
    nqkv = nq + 2 * nkv
    wqs, wos = ((d, nqkv), (nq, d)) if layout == 0 else ((nqkv, d), (d, nq))
    dev = x.device
    _need(x, "x", (T, d), dt, dev)
    _need(gy, "gy", (T, d), dt, dev)
    _need(w_qkv, "w_qkv", wqs, dt, dev)
    _need(w_o, "w_o", wos, dt, dev)
    _need(ctx, "ctx", (T, nq), dt, dev)
    _need(dqkv, "dqkv", (T, nqkv), dt, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty(T, nqkv, dtype=dt, device=dev), torch.empty(T, d, device=dev),
                   torch.empty(T, nq, dtype=dt, device=dev), torch.empty(T, d, device=dev),
                   torch.empty(wqs, device=dev), torch.empty(wos, device=dev))
        qkv, y, dctx, dx, dwq, dwo = out
        _need(qkv, "qkv", (T, nqkv), dt, dev)
        _need(y, "y", (T, d), torch.float32, dev)
        _need(dctx, "dctx", (T, nq), dt, dev)
        _need(dx, "dx", (T, d), torch.float32, dev)
        _need(dwq, "dw_qkv", wqs, torch.float32, dev)
        _need(dwo, "dw_o", wos, torch.float32, dev)
        ws, wsb = _workspace(lib.tp_attn_proj_workspace_bytes(tp, DTYPES[dt], T, d, n_q_heads, n_kv_heads, head_dim),
                             dev, workspace)
        _check(lib.tp_attn_proj_fwd_bwd(tp, DTYPES[dt], layout, T, d, n_q_heads, n_kv_heads, head_dim, _ptr(x),
                                        _ptr(w_qkv), _ptr(w_o), _ptr(ctx), _ptr(gy), _ptr(dqkv), _ptr(qkv), _ptr(y),
                                        _ptr(dctx), _ptr(dx), _ptr(dwq), _ptr(dwo), _ptr(ws), wsb, on.handle))
    return qkv, y, dctx, dx, dwq, dwo


def vocab_parallel_ce_workspace_bytes(parts, T, V):
    return load_library().vocab_parallel_ce_workspace_bytes(parts, T, V)


def vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=False, out=None, workspace=None, stream=None):
    """Mean cross-entropy over the rows of ``logits`` (T x V) with the
    vocabulary split into ``parts`` shards, and its gradient.  Returns
    (loss: 0-d fp32 tensor, dlogits: like logits, stats: T x parts x 3 fp32
    of (m_r, s_r, t_r) or None)."""
    lib = load_library()
    dt = logits.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D")
    T, V = logits.shape
    dev = logits.device
    _need(logits, "logits", (T, V), dt, dev)
    _need(labels, "labels", (T,), torch.int64, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty((), device=dev), torch.empty(T, V, dtype=dt, device=dev),
                   torch.empty(T, parts, 3, device=dev) if shard_stats else None)
        loss, dlogits, stats = out
        _need(loss, "loss", (), torch.float32, dev)
        _need(dlogits, "dlogits", (T, V), dt, dev)
        if stats is not None:
            _need(stats, "shard_stats", (T, parts, 3), torch.float32, dev)
        ws, wsb = _workspace(lib.vocab_parallel_ce_workspace_bytes(parts, T, V), dev, workspace)
        _check(lib.vocab_parallel_ce_fwd_bwd(parts, DTYPES[dt], T, V, _ptr(logits), _ptr(labels), loss.data_ptr(),
                                             _ptr(dlogits), _ptr(stats), _ptr(ws), wsb, on.handle))
    return loss, dlogits, stats


def vocab_parallel_ce_fwd_bwd_noalloc(parts, logits, labels, out, stream=None):
    """vocab_parallel_ce_fwd_bwd for callers that cannot allocate: ``out`` =
    (loss, dlogits, stats or None) must be supplied, and the library keeps the
    per-row losses in its own static device array (T <= 2^18)."""
    lib = load_library()
    dt = logits.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D")
    T, V = logits.shape
    dev = logits.device
    _need(logits, "logits", (T, V), dt, dev)
    _need(labels, "labels", (T,), torch.int64, dev)
    loss, dlogits, stats = out
    _need(loss, "loss", (), torch.float32, dev)
    _need(dlogits, "dlogits", (T, V), dt, dev)
    if stats is not None:
        _need(stats, "shard_stats", (T, parts, 3), torch.float32, dev)
    with _On(dev, stream) as on:
        _check(lib.vocab_parallel_ce_fwd_bwd_noalloc(parts, DTYPES[dt], T, V, _ptr(logits), _ptr(labels),
                                                     loss.data_ptr(), _ptr(dlogits), _ptr(stats), on.handle))
    return loss, dlogits, stats


def vocab_parallel_ce_opts_workspace_bytes(parts, T, V):
    return load_library().vocab_parallel_ce_opts_workspace_bytes(parts, T, V)


def vocab_parallel_ce_opts_fwd_bwd(parts, logits, labels, v_valid=None, ignore_index=-100, label_smoothing=0.0,
                                   shard_stats=False, out=None, workspace=None, stream=None):
    """Cross-entropy with options over the rows of ``logits`` (T x V, the
    vocabulary split into ``parts`` shards): columns from ``v_valid`` on are
    padding, rows labelled ``ignore_index`` (None: no row is ignored) are left
    out of the mean, and ``label_smoothing`` spreads that share of the target
    over the vocabulary.  Returns (loss, dlogits, stats or None) like
    vocab_parallel_ce_fwd_bwd."""
    lib = load_library()
    dt = logits.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if logits.dim() != 2:
        raise ValueError("logits must be 2-D")
    T, V = logits.shape
    vv = V if v_valid is None else int(v_valid)
    ign = NO_IGNORE if ignore_index is None else int(ignore_index)
    dev = logits.device
    _need(logits, "logits", (T, V), dt, dev)
    _need(labels, "labels", (T,), torch.int64, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty((), device=dev), torch.empty(T, V, dtype=dt, device=dev),
                   torch.empty(T, parts, 3, device=dev) if shard_stats else None)
        loss, dlogits, stats = out
        _need(loss, "loss", (), torch.float32, dev)
        _need(dlogits, "dlogits", (T, V), dt, dev)
        if stats is not None:
            _need(stats, "shard_stats", (T, parts, 3), torch.float32, dev)
        ws, wsb = _workspace(lib.vocab_parallel_ce_opts_workspace_bytes(parts, T, V), dev, workspace)
        _check(lib.vocab_parallel_ce_opts_fwd_bwd(parts, DTYPES[dt], T, V, vv, ign, float(label_smoothing),
                                                  _ptr(logits), _ptr(labels), loss.data_ptr(), _ptr(dlogits),
                                                  _ptr(stats), _ptr(ws), wsb, on.handle))
    return loss, dlogits, stats


def vocab_parallel_head_ce_workspace_bytes(parts, dtype, T, d, V):
    return load_library().vocab_parallel_head_ce_workspace_bytes(parts, DTYPES[dtype], T, d, V)


def vocab_parallel_head_ce_fwd_bwd(parts, h, w, labels, w_layout="math", out=None, workspace=None, stream=None):
    """Vocabulary-parallel output head (``parts`` shards of the vocabulary
    columns of the head ``w``) followed by the mean cross-entropy, forward and
    backward.  ``h`` is T x d; ``w`` is d x V ("math") or V x d ("torch").
    Returns (loss: 0-d fp32 tensor, dh: fp32 like h, dw: fp32 like w)."""
    lib = load_library()
    layout = W_LAYOUTS[w_layout]
    dt = h.dtype
    if dt not in DTYPES:
        raise ValueError(f"unsupported dtype {dt}")
    if h.dim() != 2 or w.dim() != 2:
        raise ValueError("h and w must be 2-D")
    T, d = h.shape
    V = w.shape[1] if layout == 0 else w.shape[0]
    wshape = (d, V) if layout == 0 else (V, d)
    dev = h.device
    _need(h, "h", (T, d), dt, dev)
    _need(w, "w", wshape, dt, dev)
    _need(labels, "labels", (T,), torch.int64, dev)
    with _On(dev, stream) as on:
        if out is None:
            out = (torch.empty((), device=dev), torch.empty(T, d, device=dev), torch.empty(wshape, device=dev))
        loss, dh, dw = out
        _need(loss, "loss", (), torch.float32, dev)
        _need(dh, "dh", (T, d), torch.float32, dev)
        _need(dw, "dw", wshape, torch.float32, dev)
        ws, wsb = _workspace(lib.vocab_parallel_head_ce_workspace_bytes(parts, DTYPES[dt], T, d, V), dev, workspace)
        _check(lib.vocab_parallel_head_ce_fwd_bwd(parts, DTYPES[dt], layout, T, d, V, _ptr(h), _ptr(w), _ptr(labels),
                                                  loss.data_ptr(), _ptr(dh), _ptr(dw), _ptr(ws), wsb,
                                                  on.handle))
    return loss, dh, dw
