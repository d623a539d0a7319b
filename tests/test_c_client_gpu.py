"""The C ABI from plain C: tests/cclient/kvd_client.c (built by
tests/cclient_build.py with gcc against include/kvd.h, the HIP runtime and
libkvd.so; no Python in the process) attends one layer from device memory and
a 3-layer host-resident stack through depth-0 and depth-1 rings over two decode
steps.  Its outputs are checked here against the oracle, and the two ring
depths against each other bit for bit."""
import os
import subprocess

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs
from tests import cclient_build

pytestmark = pytest.mark.gpu


def test_c_client(oracle, tmp_path):
    exe = cclient_build.EXE
    if not os.path.exists(exe):
        pytest.fail("the C client is not built (run __graft_entry__.build())")
    n_layers, n_rows, hq, hkv, d = 3, 3000, 40, 8, 128
    c = inputs.Config(93, "c_client", n_layers, 1, n_rows, hq, hkv, d)
    ks, vs, qs = [], [], []
    for l in range(n_layers):
        r = c.layer_rng(l)
        ks.append(inputs.random_kv_rows(r, n_rows, hkv, d))
        vs.append(inputs.random_kv_rows(r, n_rows, hkv, d))
        qs.append(inputs.random_q(r, 1, hq, d))
    np.concatenate(ks).tofile(tmp_path / "k.bin")
    np.concatenate(vs).tofile(tmp_path / "v.bin")
    np.concatenate(qs).astype(np.float32).tofile(tmp_path / "q.bin")
    print("running", exe, flush=True)
    r = subprocess.run([exe, str(tmp_path), str(n_layers), str(n_rows), str(hq), str(hkv), str(d)],
                       capture_output=True, text=True, timeout=120)
    print(r.stdout, r.stderr)
    assert r.returncode == 0, r.stderr
    assert "depth 1: engaged 1" in r.stdout and "invalid head_dim -> -1" in r.stdout
    dev = np.fromfile(tmp_path / "out_device.bin", dtype=np.float32).reshape(1, hq, d)
    d0 = np.fromfile(tmp_path / "out_ring_d0.bin", dtype=np.float32).reshape(n_layers, hq, d)
    d1 = np.fromfile(tmp_path / "out_ring_d1.bin", dtype=np.float32).reshape(n_layers, hq, d)
    assert np.array_equal(d0, d1)              # pipelined = ordered, bitwise
    assert np.array_equal(dev[0], d0[0])       # slot view = device tensor, same plan
    for l in range(n_layers):
        ref = oracle.attend(qs[l], [[(ks[l], vs[l], 0)]], hkv, d, threads=8)
        err = np.max(np.abs(d1[l].astype(np.float64) - ref[0]))
        assert err <= 1e-3, (l, err)
