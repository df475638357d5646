"""Build libattn97.so in-tree with hipcc for gfx950.

Every translation unit is compiled as HIP for gfx950 only, with packed
fp32 instructions disabled (-packed-fp32-ops), then linked into one shared
library next to this file.  Object files go to ``_build/`` (git-ignored).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libattn97.so")
UBENCH_SRC = os.path.join(HERE, "microbench", "ubench.hip")
UBENCH = os.path.join(HERE, "microbench", "ubench")

SOURCES = ["attn_api.cpp", "attn_fwd.hip", "attn_bwd.hip", "attn_bwd_dq.hip", "attn_fp8.hip"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the attention library needs the ROCm toolchain to build")


def _flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        "-I", INCLUDE,
        "-I", CSRC,
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # keep private arrays in registers (LLVM would otherwise move some into LDS)
        "-mllvm", "-disable-promote-alloca-to-lds",
        # MFMA results in arch VGPRs: with accumulators in AGPRs the compiler
        # copies them back and forth every loop iteration in the one-wave kernels
        "-mllvm", "-amdgpu-mfma-vgpr-form",
    ]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), "-x", "hip", *_flags(), "-c", os.path.join(CSRC, src), "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature name; that warning is harmless
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines()
            if "packed-fp32-ops' is not a recognized feature" not in ln]
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs), file=sys.stderr)
    return obj


def build_microbench() -> str:
    """Compile the pipe-ceiling microbenchmark (a standalone program)."""
    cmd = [_hipcc(), "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-I", INCLUDE, "-I", CSRC,
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", UBENCH_SRC, "-o", UBENCH + ".tmp"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed for microbench/ubench.hip:\n" + res.stdout + res.stderr)
    os.replace(UBENCH + ".tmp", UBENCH)
    return UBENCH


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libattn97.so (and build the
    microbenchmark program); returns the library's path."""
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES) + 1) as ex:
        ub = ex.submit(build_microbench)
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
        ub.result()
    tmp = LIB + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n" + res.stdout + res.stderr)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
