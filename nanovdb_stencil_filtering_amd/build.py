"""Compile the HIP library libvbm.so for gfx950, in-tree.

hipcc compiles the kernels and the C-ABI launchers (vbm_kernels.hip) and the
device-side grid build (vbm_build_device.hip) in parallel; g++ compiles the
host grid builder (vbm_build.cpp); hipcc links them into
nanovdb_stencil_filtering_amd/_lib/libvbm.so.  Kernel resource usage (VGPRs,
SGPRs, scratch, LDS, occupancy) is written to _lib/resource_usage.txt.  Three
libraries for the tests are built beside it: libvbm_poison.so (the same
library with every brick cell poisoned before each brick pass),
libvbm_divcheck.so (the GPU check of the WENO kernels' shortcut divisions) and
libvbm_example.so (a consumer written on the device header alone).
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
# checking build for the tests: every brick cell poisoned before each brick pass
POISON_LIB = os.path.join(LIBDIR, "libvbm_poison.so")
# GPU check of the WENO kernels' shortcut divisions (tests/division_check.hip)
DIVCHECK_LIB = os.path.join(LIBDIR, "libvbm_divcheck.so")
DIVCHECK_SRC = os.path.join(ROOT, "tests", "division_check.hip")
# a consumer written on the device header alone (tests/custom_consumer.hip)
EXAMPLE_LIB = os.path.join(LIBDIR, "libvbm_example.so")
EXAMPLE_SRC = os.path.join(ROOT, "tests", "custom_consumer.hip")
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
CXX_FLAGS = ["-std=c++17", "-O2", "-fPIC", "-Wall", "-Wextra", "-I" + INCLUDE, "-I" + CSRC]


def _run(cmd, log=None):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if log is not None:
        with open(log, "w") as f:
            f.write(r.stdout)
    if r.returncode != 0:
        sys.stderr.write(r.stdout[-20000:])
        raise RuntimeError("command failed: " + " ".join(cmd))
    return r.stdout


def _start(cmd, log):
    f = open(log, "w")
    return subprocess.Popen(cmd, stdout=f, stderr=subprocess.STDOUT, text=True), f, cmd, log


def _finish(job):
    proc, f, cmd, log = job
    rc = proc.wait()
    f.close()
    if rc != 0:
        with open(log) as fh:
            sys.stderr.write(fh.read()[-20000:])
        raise RuntimeError("command failed: " + " ".join(cmd))


def build() -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    k_obj = os.path.join(LIBDIR, "vbm_kernels.o")
    p_obj = os.path.join(LIBDIR, "vbm_kernels_poison.o")
    d_obj = os.path.join(LIBDIR, "vbm_build_device.o")
    b_obj = os.path.join(LIBDIR, "vbm_build.o")
    # the HIP sources compile in parallel
    kernels = os.path.join(CSRC, "vbm_kernels.hip")
    jobs = [_start([HIPCC, *HIP_FLAGS, "-c", kernels, "-o", k_obj], os.path.join(LIBDIR, "resource_usage.txt")),
            _start([HIPCC, *HIP_FLAGS, "-DVBM_POISON_LDS=1", "-c", kernels, "-o", p_obj],
                   os.path.join(LIBDIR, "resource_usage_poison.txt")),
            _start([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, "vbm_build_device.hip"), "-o", d_obj],
                   os.path.join(LIBDIR, "resource_usage_build_device.txt")),
            _start([HIPCC, *HIP_FLAGS, "-shared", DIVCHECK_SRC, "-o", DIVCHECK_LIB + ".tmp%d" % os.getpid()],
                   os.path.join(LIBDIR, "divcheck_build.txt")),
            _start([HIPCC, *HIP_FLAGS, "-shared", EXAMPLE_SRC, "-o", EXAMPLE_LIB + ".tmp%d" % os.getpid()],
                   os.path.join(LIBDIR, "example_build.txt"))]
    _run(["g++", *CXX_FLAGS, "-c", os.path.join(CSRC, "vbm_build.cpp"), "-o", b_obj])
    for j in jobs:
        _finish(j)
    os.replace(DIVCHECK_LIB + ".tmp%d" % os.getpid(), DIVCHECK_LIB)
    os.replace(EXAMPLE_LIB + ".tmp%d" % os.getpid(), EXAMPLE_LIB)
    for lib, objs in ((LIB, [k_obj, d_obj, b_obj]), (POISON_LIB, [p_obj, d_obj, b_obj])):
        tmp = lib + ".tmp%d" % os.getpid()
        _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", *objs, "-o", tmp])
        os.replace(tmp, lib)
    return LIB


if __name__ == "__main__":
    print(build())
