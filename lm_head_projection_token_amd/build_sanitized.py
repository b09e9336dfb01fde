"""Host-sanitized build of the C-ABI library, for the CPU tests.

``build_host_sanitized(out_dir)`` compiles ``csrc/fll_api.cpp`` (the planner,
the argument checks and the dispatch: all of the library's host code) with
AddressSanitizer and UndefinedBehaviorSanitizer on its host side only (the
device side of a HIP file is never sanitized here), links it with the
in-tree kernel objects into ``libfll_san.so``, and returns the path. Load it
with ``FLL_LIBRARY=<path>`` and the sanitizer runtime preloaded
(``asan_runtime()``); ``tests/test_sanitized_host.py`` runs the ABI tests
that way.
"""

from __future__ import annotations

import glob
import os
import subprocess

import importlib.util

_here = os.path.dirname(os.path.abspath(__file__))
_spec = importlib.util.spec_from_file_location("_fll_build", os.path.join(_here, "build.py"))
_b = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_b)

# host-only sanitizer flags: each one behind -Xarch_host
HOST_SANITIZE = [
    "-Xarch_host", "-fsanitize=address",
    "-Xarch_host", "-fsanitize=undefined",
    "-Xarch_host", "-fno-sanitize-recover=undefined",
    "-Xarch_host", "-fno-omit-frame-pointer",
]
LLVM_BIN = "/opt/rocm/llvm/bin"


def asan_runtime() -> str:
    """Path of clang's shared AddressSanitizer runtime (with UBSan)."""
    hits = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("clang's AddressSanitizer runtime not found")
    return hits[-1]


def build_host_sanitized(out_dir: str) -> str:
    hipcc = _b._hipcc()
    os.makedirs(out_dir, exist_ok=True)
    kernels = [os.path.join(_b.BUILD, os.path.splitext(s)[0] + ".o")
               for s in _b.SOURCES if s != "fll_api.cpp"]
    if not all(os.path.exists(o) for o in kernels):
        _b.build()
    obj = os.path.join(out_dir, "fll_api_san.o")
    flags = [f for f in _b.COMMON if f != "-O3"]
    _b._run([hipcc, *flags, "-O1", "-g", *HOST_SANITIZE, "-c",
             os.path.join(_b.CSRC, "fll_api.cpp"), "-o", obj])
    lib = os.path.join(out_dir, "libfll_san.so")
    link = [os.path.join(LLVM_BIN, "clang++"), "-shared", "-shared-libsan",
            "-fsanitize=address,undefined", obj, *kernels, "-L/opt/rocm/lib",
            "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", lib]
    subprocess.run(link, check=True, capture_output=True, text=True)
    return lib
