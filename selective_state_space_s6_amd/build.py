"""Build libselscan.so (the HIP kernels and the C ABI) in-tree with hipcc for gfx950.

    python -m selective_state_space_s6_amd.build

Packed-FP32 instruction selection is disabled for every HIP translation unit."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libselscan.so")
SOURCES = [os.path.join(CSRC, "scan_kernels.hip"), os.path.join(CSRC, "bwd_kernels.hip"),
           os.path.join(CSRC, "ssd_kernels.hip"), os.path.join(CSRC, "selscan_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=" + ARCH,
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-result",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile every source and link libselscan.so; always recompiles."""
    objs = []
    builddir = os.path.join(PKG, "_build")
    os.makedirs(builddir, exist_ok=True)
    procs = []
    for src in SOURCES:                                       # the sources compile concurrently
        obj = os.path.join(builddir, os.path.basename(src) + ".o")
        lang = ["-x", "hip"]
        cmd = [HIPCC] + COMMON_FLAGS + lang + ["-c", src, "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((subprocess.Popen(cmd), cmd))
        objs.append(obj)
    for proc, cmd in procs:
        if proc.wait() != 0:
            raise subprocess.CalledProcessError(proc.returncode, cmd)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def asm(out_path: str) -> None:
    """Write the gfx950 assembly of the kernels (for inspection)."""
    cmd = [HIPCC] + COMMON_FLAGS + ["-x", "hip", "--cuda-device-only", "-S", SOURCES[0], "-o", out_path]
    subprocess.check_call(cmd)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
