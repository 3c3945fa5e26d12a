"""Plain fp64 CPU oracle for one tensor-parallel rank's hot path.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute anything in this package: only the tests, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the
HIP library (no headers, helpers, tables or constants) and never imports it.

Every function works in float64 on whatever values it is given (fp32 inputs,
or bf16 inputs widened exactly), rounds no intermediate, and follows the pages
it cites:

* "Sharded GEMM与Backprop：行、列、内维三种切分" (sharded GEMM page) -- the
  bilinear loss, the three single-axis splits and the uneven/empty shard rule;
* "多卡张量：拆开计算，再合回同一结果" (multi-card tensor page) -- the column
  then row MLP, its backward equations and the vocabulary-sharded
  cross-entropy equations;
* "第 6 课：张量并行 TP" (TP lesson page) -- column-parallel and row-parallel
  linears, the block-GEMM identity and the GELU MLP composed from them;
* the multi-card tensor page's vocabulary-split output head (``head.py``):
  logits per vocabulary shard, the sharded cross-entropy, and the hidden
  state's gradient summed across the shards;
* the same page's list of what a real cross-entropy must also handle
  (``ce_options.py``): a padded vocabulary, ignored positions and label
  smoothing, each checked against an unsharded full-vocabulary reference;
* the TP lesson page's other element-wise activations and its gate / up
  column-parallel projections (``mlp_act.py``): tanh and SiLU MLPs and the
  gated MLP, forward and backward, sharded and unsharded;
* the TP lesson page's attention block (``attn_proj.py``): the column-parallel
  QKV projection split by heads (grouped-query heads included) and the
  row-parallel output projection, around an attention core that is not
  part of this.

Where a method reaches a result that has a plain definition (the unsharded
product, the unsharded MLP, the unsharded cross-entropy), the oracle used for
parity is that definition; the literal per-rank simulations are kept beside it
so that tests can show the two agree.

Every public function is pinned by ``tests/test_oracle_*.py`` against facts
that do not come from this package (the pages' worked shapes, library
routines, brute force, finite differences, closed forms and invariants).
"""

from .sharding import shard_range, shard_ranges
from .matmul import AXES, check_matmul_args, matmul_grads, sharded_matmul, sharded_matmul_partials
from .mlp import gelu, gelu_prime, to_math_layout, mlp_fwd_bwd, tp_mlp_fwd_bwd, mlp_sampled
from .ce import cross_entropy, vocab_parallel_ce
from .head import head_ce, vocab_parallel_head_ce
from .ce_options import cross_entropy_opts, vocab_parallel_ce_opts
from .attn_proj import attn_proj_fwd_bwd, check_heads, fuse_qkv, split_qkv, tp_attn_proj_fwd_bwd
from .mlp_act import ACTS, act, act_prime, mlp_act_fwd_bwd, mlp_act_sampled, tp_mlp_act_fwd_bwd

__all__ = [
    "shard_range", "shard_ranges",
    "AXES", "check_matmul_args", "matmul_grads", "sharded_matmul", "sharded_matmul_partials",
    "gelu", "gelu_prime", "to_math_layout", "mlp_fwd_bwd", "tp_mlp_fwd_bwd", "mlp_sampled",
    "cross_entropy", "vocab_parallel_ce",
    "head_ce", "vocab_parallel_head_ce",
    "cross_entropy_opts", "vocab_parallel_ce_opts",
    "attn_proj_fwd_bwd", "check_heads", "fuse_qkv", "split_qkv", "tp_attn_proj_fwd_bwd",
    "ACTS", "act", "act_prime", "mlp_act_fwd_bwd", "mlp_act_sampled", "tp_mlp_act_fwd_bwd",
]
