"""Build libtprank.so in place with hipcc for gfx950.

Usage: ``python -m megatron_mlp_fwd_amd.build`` (or ``build()`` from Python).
Every call recompiles every source; objects go to ``_build/`` (git-ignored),
the library to ``megatron_mlp_fwd_amd/libtprank.so``.

``build_host_asan()`` makes a variant for checking the host side: the C ABI's
argument validation, shard planning and workspace carving (capi.cpp) built
with AddressSanitizer on the host pass only, linked with the regular device
objects, into ``_build/asan/libtprank.so``.  Load it with the sanitizer
runtime preloaded (``ASAN_RUNTIME``) and ``TPRANK_LIB`` pointing at it.
"""
import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT = os.path.join(PKG, "libtprank.so")
BUILD = os.path.join(ROOT, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 instructions are disabled: hipcc would otherwise form
# v_pk_{add,mul,fma}_f32 from ordinary float code.
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}", f"-I{CSRC}",
]
SOURCES = ["gemm_bf16.hip", "gemm_bf16_dma.hip", "gemm_f32.hip", "reduce.hip", "vocab_ce.hip", "glu.hip", "capi.cpp"]


def _compile(src):
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in (r.stderr or "").splitlines() if noise not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{err}")
    return obj, err


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        results = list(ex.map(_compile, SOURCES))
    for (_, err), src in zip(results, SOURCES):
        if err.strip() and verbose:
            print(f"[{src}]\n{err}", file=sys.stderr)
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for o, _ in results]]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    shutil.move(tmp, OUT)
    return OUT


ASAN_RUNTIME = "/opt/rocm/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"


def build_host_asan():
    """Host-sanitized variant of the library (see the module docstring);
    returns its path.  Builds the regular objects first when they are missing."""
    if not all(os.path.exists(os.path.join(BUILD, os.path.splitext(s)[0] + ".o")) for s in SOURCES):
        build()
    out_dir = os.path.join(BUILD, "asan")
    os.makedirs(out_dir, exist_ok=True)
    obj = os.path.join(out_dir, "capi.o")
    host_asan = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
    cmd = [HIPCC, *FLAGS, *host_asan, "-x", "hip", "-c", os.path.join(CSRC, "capi.cpp"), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for capi.cpp (host ASan):\n{r.stderr}")
    objs = [obj] + [os.path.join(BUILD, os.path.splitext(s)[0] + ".o") for s in SOURCES if s != "capi.cpp"]
    lib = os.path.join(out_dir, "libtprank.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Xarch_host", "-fsanitize=address",
           "-shared-libasan", "-o", lib, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed (host ASan):\n{r.stderr}")
    return lib


if __name__ == "__main__":
    print(build(verbose=True))
