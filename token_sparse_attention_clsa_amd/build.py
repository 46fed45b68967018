"""Builds libclsa.so (the HIP kernels + C ABI) in-tree for gfx950.

Every source is compiled with hipcc for ``--offload-arch=gfx950`` only; the
shared library lands next to this file, where the binding loads it.
Packed fp32 instructions are disabled for all device code.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libclsa.so")
SOURCES = ["api.cpp", "index_score.hip", "topk.hip", "sparse_attn.hip", "block_union.hip",
           "block_attn.hip", "cache_append.hip", "static_step.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the CLSA library needs ROCm's hipcc to build")


def compile_flags():
    return [
        f"--offload-arch={ARCH}",
        "-mcode-object-version=5",  # loadable by the HIP runtime bundled with torch
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-command-line-argument",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    ]


def build(verbose: bool = False) -> str:
    """Compile every source and link libclsa.so. Always rebuilds."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    flags = compile_flags()

    def one(src):
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        cmd = [cc] + flags + ["-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(one, SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [cc, f"--offload-arch={ARCH}", "-mcode-object-version=5", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
