"""Build the plain C client of libkvd.so (tests only): tests/cclient/kvd_client.c
compiled with gcc against include/kvd.h, the HIP runtime and the in-tree
library (found at run time through an $ORIGIN-relative rpath)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
PKG = os.path.join(ROOT, "decode_attention_offloaded_amd")
SRC = os.path.join(HERE, "cclient", "kvd_client.c")
EXE = os.path.join(HERE, "cclient", "kvd_client")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(force: bool = False) -> str:
    if force or not os.path.exists(EXE):
        tmp = EXE + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-D__HIP_PLATFORM_AMD__",
               "-I" + os.path.join(ROOT, "include"), "-I" + os.path.join(ROCM, "include"), SRC,
               "-L" + PKG, "-lkvd", "-Wl,-rpath,$ORIGIN/../../decode_attention_offloaded_amd",
               "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lm",
               "-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, EXE)
    return EXE


if __name__ == "__main__":
    print(build(force=True))
