"""Build the HIP library ``libsparse_topk.so`` in-tree for gfx950.

Usage: ``python -m sparse_attention_indexer_amd.build`` (or ``build()``).
hipcc cross-compiles without a GPU present.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libsparse_topk.so")
SOURCES = ["topk_kernels.hip", "topk_api.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed FP32 instructions are kept out of generated code; plain float code
# runs on the scalar-lane FP32 units instead.
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    tmp = LIB + f".tmp{os.getpid()}"
    cmd = [HIPCC, *FLAGS, *(extra or []), "-I", INCLUDE, "-I", CSRC,
           *[os.path.join(CSRC, s) for s in SOURCES], "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
