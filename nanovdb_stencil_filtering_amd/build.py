"""Compile the HIP library libvbm.so for gfx950, in-tree.

hipcc compiles the kernels and the C-ABI launchers (vbm_kernels.hip); g++
compiles the host grid builder (vbm_build.cpp); hipcc links both into
nanovdb_stencil_filtering_amd/_lib/libvbm.so.  Kernel resource usage (VGPRs,
SGPRs, scratch, LDS, occupancy) is written to _lib/resource_usage.txt.
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBDIR = os.path.join(PKG, "_lib")
LIB = os.path.join(LIBDIR, "libvbm.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-ffp-contract=off", "-fno-fast-math", "-fno-gpu-flush-denormals-to-zero",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    # packed-FP32 forms are kept out of generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Rpass-analysis=kernel-resource-usage",
    "-I" + INCLUDE, "-I" + CSRC,
]
CXX_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE]


def _run(cmd, log=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if log is not None:
        with open(log, "w") as f:
            f.write(r.stdout)
    if r.returncode != 0:
        sys.stderr.write(r.stdout[-20000:])
        raise RuntimeError("command failed: " + " ".join(cmd))
    return r.stdout


def build() -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    k_obj = os.path.join(LIBDIR, "vbm_kernels.o")
    b_obj = os.path.join(LIBDIR, "vbm_build.o")
    _run([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "vbm_kernels.hip"), "-o", k_obj],
         log=os.path.join(LIBDIR, "resource_usage.txt"))
    _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "vbm_build.cpp"), "-o", b_obj])
    tmp = LIB + ".tmp%d" % os.getpid()
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", k_obj, b_obj, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build())
