"""Build the HIP library ``libsparse_topk.so`` in-tree for gfx950.

Usage: ``python -m sparse_attention_indexer_amd.build`` (or ``build()``).
hipcc cross-compiles without a GPU present. The sources compile to
objects in ``_build/`` side by side, then link into the shared library.

``build_api_sanitizer_driver()`` builds ``_build/api_asan_driver``: the C ABI
host code (``topk_api.hip``) with the host address and undefined-behaviour
sanitizers, linked with the same kernel object and a driver that calls every
entry point with host-checkable bad arguments (tests/sanitize/api_driver.cpp).
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libsparse_topk.so")
SOURCES = ["topk_kernels.hip", "topk_api.hip", "prologue.hip", "logits.hip", "hisparse.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ROCM_LIB = "/opt/rocm/lib"
CLANGXX = "/opt/rocm/llvm/bin/clang++"   # host compiler of hipcc: one sanitizer runtime for all objects

# Packed FP32 instructions are kept out of generated code; plain float code
# runs on the scalar-lane FP32 units instead.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]
# The score producer runs without IEEE mode: there a ReLU of a matrix-core
# result is one v_max_f32, while IEEE mode first quiets a possible signalling
# NaN with a second one, which doubles the epilogue's ALU work per score.
SOURCE_FLAGS = {"logits.hip": ["-mno-amdgpu-ieee", "-fno-honor-nans"]}
# Host-only sanitizers for the C ABI object (device code is built as usual).
HOST_SANITIZE = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=all"]


def _obj(src: str, suffix: str = "") -> str:
    return os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")


def _compile(src: str, out: str, extra: list[str], verbose: bool) -> subprocess.Popen:
    cmd = [HIPCC, *FLAGS, *SOURCE_FLAGS.get(src, []), *extra, "-I", INCLUDE, "-I", CSRC, "-c",
           os.path.join(CSRC, src), "-o", out]
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.Popen(cmd)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    procs = [(_compile(s, _obj(s), extra or [], verbose), s) for s in SOURCES]
    for p, s in procs:
        if p.wait() != 0:
            raise subprocess.CalledProcessError(p.returncode, f"hipcc {s}")
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *[_obj(s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def build_api_sanitizer_driver(verbose: bool = False) -> str:
    """The sanitized C ABI host code plus its test driver (needs the kernel
    object from build())."""
    kern = _obj("topk_kernels.hip")
    if not os.path.exists(kern):
        build(verbose)
    api = _obj("topk_api.hip", "_asan")
    p = _compile("topk_api.hip", api, ["-O1", "-g", *HOST_SANITIZE], verbose)
    if p.wait() != 0:
        raise subprocess.CalledProcessError(p.returncode, "hipcc topk_api.hip (sanitized host)")
    drv_src = os.path.join(ROOT, "tests", "sanitize", "api_driver.cpp")
    drv_obj = os.path.join(BUILD, "api_driver.o")
    out = os.path.join(BUILD, "api_asan_driver")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    subprocess.check_call([CLANGXX, "-O1", "-g", "-std=c++17", *san, "-I", INCLUDE, "-c", drv_src, "-o", drv_obj])
    subprocess.check_call([CLANGXX, *san, drv_obj, api, kern, "-L", ROCM_LIB, "-lamdhip64",
                           f"-Wl,-rpath,{ROCM_LIB}", "-o", out])
    return out


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
