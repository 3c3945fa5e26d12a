"""vocab_parallel_ce_fwd_bwd_noalloc: the cross-entropy entry point that
allocates nothing (its per-row losses sit in the library's static device
array) against the workspace entry point on the same inputs, through the C
ABI: two calls in a row, the second with a smaller input, each bit for bit
equal to vocab_parallel_ce_fwd_bwd (the same kernels run) and element by
element within the gradient bound of ce_checks.py against the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads
from ce_checks import assert_grad_elementwise, target_rows

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def tpr():
    import megatron_mlp_fwd_amd as m
    m.load_library()
    torch.cuda.set_device(0)
    return m


def _outs(T, V, parts, dtype, stats):
    return (torch.full((), float("nan"), device=DEV), torch.full((T, V), float("nan"), dtype=dtype, device=DEV),
            torch.full((T, parts, 3), float("nan"), device=DEV) if stats else None)


def test_noalloc_equals_workspace_entry_point(tpr):
    cases = [(512, 128256, 8, torch.bfloat16, False), (64, 32000, 3, torch.bfloat16, True),
             (5, 1001, 2, torch.float32, False)]
    for T, V, parts, dtype, stats in cases:   # each call smaller than the one before
        say("no-alloc CE", T, V, parts, dtype, "stats" if stats else "no stats")
        logits, labels = workloads.vocab_ce(T=T, V=V, seed=T + V, device=DEV, dtype=dtype)
        got = tpr.vocab_parallel_ce_fwd_bwd_noalloc(parts, logits, labels, out=_outs(T, V, parts, dtype, stats))
        ref = tpr.vocab_parallel_ce_fwd_bwd(parts, logits, labels, shard_stats=stats)
        torch.cuda.synchronize()
        assert torch.equal(got[0], ref[0]) and torch.equal(got[1], ref[1])
        if stats:
            assert torch.equal(got[2], ref[2])
        z, y = logits.double().cpu().numpy(), labels.cpu().numpy()
        wl, _, wg = oracle.cross_entropy(z, y)
        assert abs(got[0].item() - wl) <= 1e-5 * abs(wl)
        kind = "f32" if dtype == torch.float32 else "bf16"
        assert_grad_elementwise(got[1].double().cpu().numpy(), wg, target_rows(y, V), T, kind, "no-alloc dlogits")


def test_noalloc_rejects_more_rows_than_its_array(tpr):
    import ctypes
    lib = tpr.load_library()
    p = ctypes.c_void_p(16)  # never dereferenced: the call fails before any launch
    T = (1 << 18) + 1
    assert lib.vocab_parallel_ce_fwd_bwd_noalloc(1, 1, T, 8, p, p, p, p, None, None) == tpr.binding.TPR_ERR_WORKSPACE
    assert b"static scratch" in lib.tprank_last_error()
