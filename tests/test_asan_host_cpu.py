"""The host side of the C ABI under AddressSanitizer, on the CPU.

capi.cpp (argument validation, shard planning, workspace carving, the
partial-sum and no-allocation entry points' checks) is rebuilt with ASan on
its host pass and linked with the regular device objects; the CPU ABI tests
then run against that library in a child process with the sanitizer runtime
preloaded.  Any heap, stack or global buffer overflow, use after free or
double free in the host code aborts the child and fails this test.
"""
import os
import subprocess
import sys

import pytest

from megatron_mlp_fwd_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_abi_cpu_tests_under_host_asan():
    if not os.path.exists(build.HIPCC) or not os.path.exists(build.ASAN_RUNTIME):
        pytest.skip("hipcc or the clang ASan runtime is not installed")
    lib = build.build_host_asan()
    env = dict(os.environ, TPRANK_LIB=lib, LD_PRELOAD=build.ASAN_RUNTIME,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    assert " passed" in r.stdout, out[-2000:]
    # the child really ran the sanitized library with the runtime loaded
    probe = ("from megatron_mlp_fwd_amd import binding; binding.load_library(); "
             "maps = open('/proc/self/maps').read(); "
             "print(binding.LIB_PATH in maps, 'libclang_rt.asan' in maps)")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.stdout.split() == ["True", "True"], r.stdout + r.stderr[-2000:]
