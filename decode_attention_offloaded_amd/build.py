"""Build the HIP library ``libkvd.so`` in-tree (gfx950).

Every HIP source is compiled with packed-FP32 instructions disabled (the
hardware's packed fp32 forms are not used anywhere in this library).
"""
from __future__ import annotations

import concurrent.futures
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build", "kvd")
LIB_PATH = os.path.join(PKG, "libkvd.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CODE_OBJECT = ["-mcode-object-version=5"]  # loadable by the ROCm 7.0 runtime torch ships
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I" + INCLUDE, "-I" + CSRC]
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
# The kernels' leading scalar arguments go into SGPRs at wave launch (up to the
# 14 user SGPRs left for them); the code object keeps a prologue that loads
# them from memory where the firmware does not preload.
KERNARG_PRELOAD = ["-mllvm", "-amdgpu-kernarg-preload-count=16"]
# MFMA accumulators in ordinary VGPRs (the register file is unified): with the
# accumulator registers, the softmax rescale of the output accumulators made
# the compiler copy all of them out and back on every loop iteration.
MFMA_VGPR = ["-mllvm", "-amdgpu-mfma-vgpr-form"]
HIP_SOURCES = ["kvd_attend.hip", "kvd_hbm_probe.hip"]
HOST_SOURCES = ["kvd_plan.cpp", "kvd_errors.cpp", "kvd_ring_core.cpp", "kvd_ring_hip.cpp", "kvd_residency.cpp",
                "kvd_probe.cpp"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += ["--offload-arch=" + ARCH] + CODE_OBJECT + NO_PACKED_FP32 + KERNARG_PRELOAD + MFMA_VGPR
    cmd += ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libkvd.so next to this file.  Returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = HIP_SOURCES + HOST_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH] + CODE_OBJECT + objs + ["-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
