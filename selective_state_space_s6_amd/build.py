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
# issue-rate and bandwidth probes (bench.py --microbench), same flags, a library of their own
MICROBENCH_SRC = os.path.join(CSRC, "microbench.hip")
MICROBENCH_LIB = os.path.join(PKG, "libselscan_microbench.so")
# the forward scan's kernels are instantiated per element type and pass in units of their
# own (scan_inst_*.hip), which compile in parallel
SCAN_UNITS = [os.path.join(CSRC, "scan_inst_%s_%s.hip" % (io, ps))
              for io in ("f32", "bf16") for ps in ("single", "state", "apply")]
SOURCES = SCAN_UNITS + [os.path.join(CSRC, "bwd_kernels.hip"), os.path.join(CSRC, "bwd_ti_kernels.hip"), os.path.join(CSRC, "scan_kernels.hip"),
                        os.path.join(CSRC, "conv_kernels.hip"), os.path.join(CSRC, "ssd_kernels.hip"),
                        os.path.join(CSRC, "selscan_api.cpp")]
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
    jobs = max(1, min(len(SOURCES), os.cpu_count() or 1, 16))
    pending = []
    for src in SOURCES + [MICROBENCH_SRC]:
        obj = os.path.join(builddir, os.path.basename(src) + ".o")
        pending.append(([HIPCC] + COMMON_FLAGS + ["-x", "hip", "-c", src, "-o", obj]))
        objs.append(obj)
    mb_obj = objs.pop()
    running = []
    while pending or running:                                 # at most `jobs` compiles at once
        while pending and len(running) < jobs:
            cmd = pending.pop(0)
            if verbose:
                print(" ".join(cmd), flush=True)
            running.append((subprocess.Popen(cmd), cmd))
        proc, cmd = running.pop(0)
        if proc.wait() != 0:
            for other, _ in running:
                other.wait()
            raise subprocess.CalledProcessError(proc.returncode, cmd)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    tmp = MICROBENCH_LIB + ".tmp%d" % os.getpid()
    subprocess.check_call([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, mb_obj])
    os.replace(tmp, MICROBENCH_LIB)
    return LIB


def asm(out_path: str, source: str = "") -> None:
    """Write the gfx950 assembly of one unit's kernels (for inspection; default: the first
    scan unit)."""
    cmd = [HIPCC] + COMMON_FLAGS + ["-x", "hip", "--cuda-device-only", "-S", source or SOURCES[0], "-o", out_path]
    subprocess.check_call(cmd)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
