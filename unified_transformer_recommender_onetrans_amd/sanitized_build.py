"""The library with its C ABI layer built under host sanitizers (for the host-only ABI tests).

onetrans_api.cpp (validation, layouts, launch sequences) is compiled with host
AddressSanitizer and UndefinedBehaviorSanitizer; the kernels are the ordinary objects of
build.py (device code is never sanitized). Nothing on a GPU run loads this library.
"""
from __future__ import annotations

import os
import subprocess

from .build import ARCH, BUILD_DIR, CSRC, FLAGS, HIPCC, SOURCES, VGPR_FORM, build

ASAN_RUNTIME = "/opt/rocm/lib/llvm/lib/clang/22/lib/linux/libclang_rt.asan-x86_64.so"
SANITIZED_LIB = os.path.join(BUILD_DIR, "asan", "libonetrans_asan.so")


def build_sanitized(verbose: bool = False) -> str:
    """The same library with the C ABI layer (onetrans_api.cpp: validation, layouts, launch
    sequences) built with host AddressSanitizer and UndefinedBehaviorSanitizer; the kernels
    are the ordinary objects (device code is never sanitized). Load it with the ASan runtime
    preloaded (ASAN_RUNTIME) and ONETRANS_LIB pointing at it; it serves the host-only ABI tests."""
    os.makedirs(os.path.dirname(SANITIZED_LIB), exist_ok=True)
    objs = [os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o") for src in SOURCES if src.endswith(".hip")]
    if not all(os.path.exists(o) for o in objs):
        build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined"]
    api = os.path.join(os.path.dirname(SANITIZED_LIB), "onetrans_api.o")
    cmd = ([HIPCC] + [f for f in FLAGS if f != "-O3"] + VGPR_FORM + ["-O1", "-g"] + san +
           ["-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all",
            "-c", os.path.join(CSRC, "onetrans_api.cpp"), "-o", api])
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized compile failed:\n{r.stderr}")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC"] + san + ["-shared-libasan", "-o", SANITIZED_LIB, api] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized link failed:\n{r.stderr}")
    if verbose:
        print(f"built {SANITIZED_LIB}")
    return SANITIZED_LIB
