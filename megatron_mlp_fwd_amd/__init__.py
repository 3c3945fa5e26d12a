"""One tensor-parallel rank's hot path on AMD Instinct MI355X (gfx950).

Python face of libtprank (include/tprank.h): sharded matrix multiply forward
and backward on the row, column and inner axes; the column-then-row MLP
(GELU, tanh or SiLU, plain or gated by an up projection); the attention
block's QKV (by heads) and output projections;
vocabulary-parallel cross-entropy (plain, or with a padded vocabulary, an
ignore index and label smoothing), alone or behind the vocabulary-parallel
output head.  All compute runs in the library's HIP
kernels; torch provides device memory and streams.
"""
from .binding import (ACTS, AXES, DTYPES, LIB_PATH, W_LAYOUTS, TprError, load_library, partial_sum, shard_range,
                      sharded_matmul_fwd_bwd, sharded_matmul_workspace_bytes, tp_mlp_fwd_bwd,
                      tp_mlp_workspace_bytes, tp_mlp_act_fwd_bwd, tp_mlp_act_workspace_bytes,
                      tp_attn_proj_fwd_bwd, tp_attn_proj_workspace_bytes,
                      vocab_parallel_ce_fwd_bwd, vocab_parallel_ce_workspace_bytes, vocab_parallel_ce_fwd_bwd_noalloc,
                      vocab_parallel_ce_opts_fwd_bwd, vocab_parallel_ce_opts_workspace_bytes,
                      vocab_parallel_head_ce_fwd_bwd, vocab_parallel_head_ce_workspace_bytes)

__all__ = [
    "ACTS", "AXES", "DTYPES", "LIB_PATH", "W_LAYOUTS", "TprError", "load_library", "partial_sum", "shard_range",
    "sharded_matmul_fwd_bwd", "sharded_matmul_workspace_bytes", "tp_mlp_fwd_bwd", "tp_mlp_workspace_bytes",
    "tp_mlp_act_fwd_bwd", "tp_mlp_act_workspace_bytes",
    "tp_attn_proj_fwd_bwd", "tp_attn_proj_workspace_bytes",
    "vocab_parallel_ce_fwd_bwd", "vocab_parallel_ce_workspace_bytes", "vocab_parallel_ce_fwd_bwd_noalloc",
    "vocab_parallel_ce_opts_fwd_bwd", "vocab_parallel_ce_opts_workspace_bytes",
    "vocab_parallel_head_ce_fwd_bwd", "vocab_parallel_head_ce_workspace_bytes",
]
