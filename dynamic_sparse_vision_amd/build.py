"""Build libdcnv4.so (HIP, gfx950) in-tree with hipcc.

Every source is compiled to an object in parallel, with the compiler's
kernel resource report on; the build fails when any kernel uses scratch
memory (register spills or a private array demoted to memory), so that no
kernel of the library runs with per-lane scratch.  The objects are then
linked into one shared library.

Usage: python -m dynamic_sparse_vision_amd.build [-v]
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdcnv4.so")
SOURCE_NAMES = ("dcnv4_kernels.hip", "dcnv4_tiled_fwd.hip", "dcnv4_tiled_bwd_offsets.hip",
                "dcnv4_tiled_bwd_values.hip", "dcnv4_tiled_launch.hip", "dcnv4_api.cpp",
                "fdattn_kernels.hip", "fdattn_noalloc.hip", "fdattn_api.cpp")
SOURCES = [os.path.join(CSRC, n) for n in SOURCE_NAMES]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "-x", "hip", "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    # coordinates and weights use explicit fmaf only: nothing else is contracted
    "-ffp-contract=off",
    # no packed fp32 instructions (v_pk_*_f32) in the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fvisibility=hidden", "-Wall", "-Wno-unused-command-line-argument",
    "-I", INCLUDE, "-I", CSRC,
]
# per-kernel register / scratch / occupancy report on stderr
RESOURCE_FLAGS = ["-Rpass-analysis=kernel-resource-usage"]


class ScratchError(RuntimeError):
    """A kernel of the library uses scratch memory."""


def parse_resource_report(text: str):
    """[(mangled kernel name, {field: int})] from the compiler's
    kernel-resource-usage remarks."""
    kernels = []
    cur = None
    for line in text.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = (m.group(1), {})
            kernels.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z ]+?)(?: \[[^\]]*\])?: (\d+)\s", line + " ")
        if m and cur is not None:
            cur[1][m.group(1).strip()] = int(m.group(2))
    return kernels


def demangle(names):
    try:
        out = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True,
                             check=True).stdout.splitlines()
        return out if len(out) == len(names) else list(names)
    except (OSError, subprocess.CalledProcessError):
        return list(names)


def compile_one(src: str, obj: str, verbose: bool):
    cmd = [HIPCC, *FLAGS, *RESOURCE_FLAGS, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    warnings = [ln for ln in r.stderr.splitlines() if "warning:" in ln and "packed-fp32-ops" not in ln]
    if r.returncode != 0:
        sys.stderr.write(r.stderr)
        raise subprocess.CalledProcessError(r.returncode, cmd)
    return parse_resource_report(r.stderr), warnings


def build(verbose: bool = False) -> str:
    tmp = tempfile.mkdtemp(prefix="dcnv4_build_")
    try:
        objs = [os.path.join(tmp, os.path.basename(s) + ".o") for s in SOURCES]
        workers = min(len(SOURCES), max(1, min(16, os.cpu_count() or 1)))
        with cf.ThreadPoolExecutor(workers) as ex:
            results = list(ex.map(lambda so: compile_one(so[0], so[1], verbose), zip(SOURCES, objs)))
        scratch = []
        nkernels = 0
        for src, (kernels, warnings) in zip(SOURCES, results):
            for w in warnings:
                print(w, file=sys.stderr)
            nkernels += len(kernels)
            if src.endswith(".hip") and "__global__" in open(src).read() and not kernels:
                raise ScratchError(f"no kernel resource report for {os.path.basename(src)}: "
                                   "cannot check its kernels for scratch memory")
            for name, fields in kernels:
                if fields.get("ScratchSize", 0) > 0:
                    scratch.append((os.path.basename(src), name, fields))
        if scratch:
            pretty = demangle([n for _, n, _ in scratch])
            lines = [f"  {s}: {d}: ScratchSize {f.get('ScratchSize')} B/lane, VGPRs {f.get('VGPRs')}"
                     for (s, _, f), d in zip(scratch, pretty)]
            raise ScratchError("kernels using scratch memory:\n" + "\n".join(lines))
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", LIB + ".tmp"]
        if verbose:
            print(" ".join(cmd), flush=True)
        subprocess.run(cmd, check=True)
        os.replace(LIB + ".tmp", LIB)
        if verbose:
            print(f"{nkernels} kernels, none uses scratch memory", flush=True)
        return LIB
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
