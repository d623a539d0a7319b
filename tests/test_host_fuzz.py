"""Randomised argument checks of the host code under AddressSanitizer and
UBSan (tests/ringsim/fuzz_main.cpp, built with g++ by tests/ringsim_build.py):
split plans (every accepted plan's invariants, visible ranges against brute
force), tile sizes, residency plans and ring calls on the simulated runtime.
Runs on the CPU."""
import subprocess

import pytest

from tests import ringsim_build


@pytest.mark.parametrize("seed", [1, 2])
def test_host_code_under_sanitizers(seed):
    exe = ringsim_build.build_fuzz()
    r = subprocess.run([exe, str(seed), "5000"], capture_output=True, text=True, timeout=300)
    print(r.stdout, r.stderr[-4000:])
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failed checks" in r.stdout
    accepted = int(r.stdout.split("iterations: ")[1].split(" plans accepted")[0])
    assert accepted > 1000   # the valid half of the distribution is exercised
