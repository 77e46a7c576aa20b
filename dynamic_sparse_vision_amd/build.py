"""Build libdcnv4.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m dynamic_sparse_vision_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdcnv4.so")
SOURCES = [os.path.join(CSRC, n) for n in ("dcnv4_kernels.hip", "dcnv4_tiled.hip", "dcnv4_api.cpp",
                                            "fdattn_kernels.hip", "fdattn_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # coordinates and weights use explicit fmaf only: nothing else is contracted
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    cmd = [HIPCC, *FLAGS, *SOURCES, "-o", LIB + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
