"""Build the CPU ring simulator (tests only): the product's ring core compiled
with g++ against a simulated transport (tests/ringsim/ringsim.cpp)."""
from __future__ import annotations

import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "decode_attention_offloaded_amd", "csrc")
LIB = os.path.join(HERE, "ringsim", "libringsim.so")
SOURCES = [os.path.join(HERE, "ringsim", "ringsim.cpp"), os.path.join(CSRC, "kvd_ring_core.cpp"),
           os.path.join(CSRC, "kvd_errors.cpp")]


def build(force: bool = False, sanitize: bool = False) -> str:
    if force or not os.path.exists(LIB):
        tmp = LIB + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + SOURCES + ["-o", tmp]
        if sanitize:
            cmd[1:1] = ["-fsanitize=address,undefined", "-fno-omit-frame-pointer"]
        subprocess.check_call(cmd)
        os.replace(tmp, LIB)
    return LIB


FUZZ = os.path.join(HERE, "ringsim", "ringsim_fuzz")
FUZZ_SOURCES = [os.path.join(HERE, "ringsim", "fuzz_main.cpp"), os.path.join(HERE, "ringsim", "ringsim.cpp"),
                os.path.join(CSRC, "kvd_ring_core.cpp"), os.path.join(CSRC, "kvd_errors.cpp"),
                os.path.join(CSRC, "kvd_plan.cpp"), os.path.join(CSRC, "kvd_residency.cpp")]


def build_fuzz(force: bool = False) -> str:
    """The randomised host-code checks (tests/ringsim/fuzz_main.cpp) as an
    executable built with g++, AddressSanitizer and UBSan (host code only)."""
    if force or not os.path.exists(FUZZ):
        tmp = FUZZ + ".tmp%d" % os.getpid()
        cmd = ["g++", "-O1", "-g", "-std=c++17", "-Wall", "-Wextra", "-fsanitize=address,undefined",
               "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer",
               "-I" + os.path.join(ROOT, "include"), "-I" + CSRC] + FUZZ_SOURCES + ["-o", tmp]
        subprocess.check_call(cmd)
        os.replace(tmp, FUZZ)
    return FUZZ
