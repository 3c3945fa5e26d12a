"""The C ABI used from C itself, without Python: a C99 program that includes
include/tprank.h (compiled with -std=c99 -pedantic -Werror, so the header is
plain C) and links libtprank.so, then drives the host-side part of the
boundary: shard planning, workspace sizes and the argument checks that every
entry point runs before it enqueues anything.  No call reaches a device."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB_DIR = os.path.join(ROOT, "megatron_mlp_fwd_amd")

PROGRAM = r"""
#include <stdio.h>
#include <string.h>
#include "tprank.h"

static int fails = 0;
#define EXPECT(cond) do { if (!(cond)) { printf("FAILED line %d: %s\n", __LINE__, #cond); ++fails; } } while (0)

int main(void) {
  int64_t b = -1, e = -1, total = 0;
  int r;
  /* [GEMM] 手动走一遍: K = 5 over 2 parts is 3 then 2 */
  EXPECT(tprank_shard_range(5, 2, 0, &b, &e) == TPR_OK && b == 0 && e == 3);
  EXPECT(tprank_shard_range(5, 2, 1, &b, &e) == TPR_OK && b == 3 && e == 5);
  /* more parts than indices: the trailing shards are empty, the ranges tile [0, n) */
  for (r = 0; r < 7; ++r) {
    EXPECT(tprank_shard_range(3, 7, r, &b, &e) == TPR_OK && e >= b);
    total += e - b;
  }
  EXPECT(total == 3);
  EXPECT(tprank_shard_range(5, 0, 0, &b, &e) == TPR_ERR_PARTITION);
  EXPECT(strlen(tprank_last_error()) > 0);
  EXPECT(tprank_shard_range(-1, 2, 0, &b, &e) == TPR_ERR_SHAPE);
  EXPECT(tprank_shard_range(5, 2, 2, &b, &e) == TPR_ERR_PARTITION);
  EXPECT(tprank_shard_range(5, 2, 0, NULL, &e) == TPR_ERR_NULLPTR);

  /* workspace sizes: a rows split of a 3 x 5 x 4 fp32 problem sums dB (5 x 4) over 2 partials */
  EXPECT(sharded_matmul_workspace_bytes(TPR_ROWS, 1, TPR_F32, 3, 5, 4) == 0);
  EXPECT(sharded_matmul_workspace_bytes(TPR_ROWS, 2, TPR_F32, 3, 5, 4) == 2 * 256);
  EXPECT(vocab_parallel_ce_workspace_bytes(8, 4096, 128256) == 4096 * 4);
  EXPECT(tp_mlp_workspace_bytes(0, TPR_BF16, 16, 64, 256) == 0);

  /* argument checks run before any launch: each call below fails on the host */
  EXPECT(sharded_matmul_fwd_bwd(7, 1, TPR_F32, 3, 5, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)
         == TPR_ERR_PARTITION);
  EXPECT(sharded_matmul_fwd_bwd(TPR_ROWS, 1, 9, 3, 5, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)
         == TPR_ERR_DTYPE);
  EXPECT(sharded_matmul_fwd_bwd(TPR_ROWS, 1, TPR_F32, 3, 5, 4, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)
         == TPR_ERR_NULLPTR);
  EXPECT(tp_mlp_fwd_bwd(0, TPR_BF16, TPR_W_MATH, 16, 64, 256, NULL, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                        NULL, 0, NULL) == TPR_ERR_PARTITION);
  EXPECT(tp_mlp_act_fwd_bwd(1, TPR_BF16, TPR_W_MATH, 9, 16, 64, 256, NULL, NULL, NULL, NULL, NULL, NULL, NULL,
                            NULL, NULL, NULL, NULL, 0, NULL) != TPR_OK);
  EXPECT(vocab_parallel_ce_fwd_bwd(0, TPR_BF16, 4, 16, NULL, NULL, NULL, NULL, NULL, NULL, 0, NULL)
         == TPR_ERR_PARTITION);
  EXPECT(vocab_parallel_ce_fwd_bwd_noalloc(1, TPR_BF16, 4, 16, NULL, NULL, NULL, NULL, NULL, NULL)
         == TPR_ERR_NULLPTR);
  EXPECT(tprank_partial_sum(2, 16, NULL, 16, NULL, NULL) == TPR_ERR_NULLPTR);
  EXPECT(tprank_partial_sum(-1, 16, NULL, 16, NULL, NULL) != TPR_OK);
  EXPECT(strlen(tprank_last_error()) > 0);

  if (fails == 0) printf("ok\n");
  return fails == 0 ? 0 : 1;
}
"""


def _gpu_visible():
    import torch
    return torch.cuda.device_count() > 0  # counts without initialising the runtime


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.skipif(_gpu_visible(), reason="a host-only check: runs where no GPU is visible")
def test_c_program_uses_the_abi(tmp_path):
    lib = os.path.join(LIB_DIR, "libtprank.so")
    if not os.path.exists(lib):
        pytest.skip("libtprank.so is not built")
    src = tmp_path / "abi.c"
    exe = tmp_path / "abi"
    src.write_text(PROGRAM)
    cc = subprocess.run(["gcc", "-std=c99", "-pedantic", "-Wall", "-Wextra", "-Werror",
                         "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe),
                         "-L", LIB_DIR, "-ltprank", "-Wl,-rpath," + LIB_DIR],
                        capture_output=True, text=True)
    assert cc.returncode == 0, cc.stderr
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.strip().endswith("ok"), run.stdout + run.stderr
