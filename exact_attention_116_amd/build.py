"""Compile the HIP sources of the attention library into ``libfa.so`` (gfx950).

Each source is compiled to an object under ``_build/`` in parallel, then
linked in place next to this file, so the library travels with the source
tree.  Usage: ``python -m exact_attention_116_amd.build`` (or ``build()``).
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libfa.so")
SOURCES = ["fa_fwd_bf16.hip", "fa_fwd_fp8.hip", "fa_decode.hip", "fa_decode_gqa.hip", "fa_bwd.hip", "fa_fp8_quant.hip",
           "fa_api.cpp"]
ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
# Packed fp32 VALU forms are kept out of the generated code.
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-result"]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build step failed:\n" + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"]
        cmds.append([HIPCC, *lang, *COMMON, "-c", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    with ThreadPoolExecutor(jobs or min(8, len(cmds))) as ex:
        for r in ex.map(_run, cmds):
            if verbose and (r.stdout or r.stderr):
                sys.stdout.write(r.stdout + r.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


ASAN_LIB = os.path.join(BUILD_DIR, "libfa_host_asan.so")


def build_host_asan() -> str:
    """CPU-only build of the C-ABI layer (fa_api.cpp) under AddressSanitizer,
    linked with host stand-ins for the HIP runtime calls and the kernel
    launchers (csrc/host_stubs.cpp); no device code.  For the CPU tests of
    argument validation and workspace handling.  Loading it into Python
    needs the sanitizer runtime preloaded (``asan_runtime()``)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    tmp = ASAN_LIB + ".tmp"
    _run(["g++", "-std=c++17", "-O1", "-g", "-fPIC", "-shared", "-fsanitize=address",
          "-fno-omit-frame-pointer", "-D__HIP_PLATFORM_AMD__", "-I", "/opt/rocm/include",
          "-I", os.path.join(ROOT, "include"), os.path.join(CSRC, "fa_api.cpp"),
          os.path.join(CSRC, "host_stubs.cpp"), "-o", tmp])
    os.replace(tmp, ASAN_LIB)
    return ASAN_LIB


def asan_runtime() -> str:
    """Path of the compiler's AddressSanitizer runtime (to LD_PRELOAD)."""
    return _run(["g++", "-print-file-name=libasan.so"]).stdout.strip()


if __name__ == "__main__":
    print(build(verbose=True))
