"""Build ``libfll.so`` (the C-ABI library) in-tree with hipcc for gfx950.

Usage: ``python lm_head_projection_token_amd/build.py`` or ``build()``.
Compiles every source under ``csrc/`` and links them into
``lm_head_projection_token_amd/libfll.so``. No GPU is needed: hipcc
cross-compiles the gfx950 code objects.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libfll.so")
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

ARCH = "gfx950"
SOURCES = ["fll_api.cpp", "gemm_bf16.hip", "gemm_fp32.hip", "row_kernels.hip"]

# Packed fp32 VALU instructions are switched off for all device code.
COMMON = [
    "-x", "hip", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wno-unused-function", "-I", INCLUDE,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfll.so)")


def _run(cmd):
    res = subprocess.run(cmd, capture_output=True, text=True)
    # The host pass warns that it does not know the packed-fp32 feature.
    err = "\n".join(l for l in res.stderr.splitlines()
                    if "packed-fp32-ops" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed: {' '.join(cmd)}\n{err}")
    return err


def build(verbose: bool = False, extra_flags=()) -> str:
    """Compile all sources and link ``libfll.so``; returns its path."""
    hipcc = _hipcc()
    os.makedirs(BUILD, exist_ok=True)

    def compile_one(src):
        obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *COMMON, *extra_flags, "-c", os.path.join(CSRC, src), "-o", obj]
        msg = _run(cmd)
        if verbose and msg.strip():
            print(msg, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=min(len(SOURCES), 8)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB, file=sys.stderr)
    return LIB


ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
CLIENT_DIR = os.path.join(os.path.dirname(PKG), "tests", "c_client")
CLIENT = os.path.join(CLIENT_DIR, "fll_client")


def build_c_client() -> str:
    """Compile the plain C client of the library (``tests/c_client``) with
    gcc against include/fll.h, the in-tree libfll.so and the HIP runtime; it
    finds libfll.so next to the repository at run time (rpath $ORIGIN)."""
    src = os.path.join(CLIENT_DIR, "fll_client.c")
    tmp = CLIENT + ".tmp"
    _run(["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-Werror",
          "-D__HIP_PLATFORM_AMD__", "-I", INCLUDE, "-I", os.path.join(ROCM, "include"),
          src, "-o", tmp, "-L", PKG, "-lfll", "-L", os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath,$ORIGIN/../../lm_head_projection_token_amd",
          "-Wl,-rpath," + os.path.join(ROCM, "lib")])
    os.replace(tmp, CLIENT)
    return CLIENT


if __name__ == "__main__":
    build(verbose=True)
    build_c_client()
