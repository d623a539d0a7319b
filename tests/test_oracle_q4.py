"""Pins of the oracle's q4_0 V path (asymmetric cache: q8_0 K, q4_0 V).

- hand-decoded q4_0 blocks (tests/golden/q4_0_blocks.txt);
- the q4_0 path against the independently pinned q8_0 path: a q4_0 block and a
  q8_0 block with the same scale bits and codes (nibble - 8) hold the same
  values, so the two attention results must be equal in fp64;
- closed forms: one-row context returns that row's V; a zero query returns the
  mean of V;
- the ring size with narrower V rows."""
import os

import numpy as np
import pytest

from decode_attention_offloaded_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    cases = []
    with open(os.path.join(GOLDEN, "q4_0_blocks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            assert parts[0] == "case" and len(parts) == 3 + 32
            cases.append((int(parts[1], 16), bytes.fromhex(parts[2]), [float(x) for x in parts[3:]]))
    return cases


@pytest.mark.parametrize("case", _golden())
def test_q4_0_golden_blocks(oracle, case):
    bits, qs, expect = case
    blk = np.frombuffer(bytes([bits & 0xFF, bits >> 8]) + qs, dtype=np.uint8)
    assert blk.size == 18
    vals = oracle.dequant_q4_0(blk)
    assert vals.tolist() == expect


def test_pack_q4_0_matches_the_golden_layout(oracle):
    # byte j = j | (15 - j) << 4 in the first golden case: codes j and 16 + j
    nib = np.array([list(range(16)) + list(range(15, -1, -1))], dtype=np.uint8)
    blk = inputs.pack_q4_0(nib, np.array([0x3C00], dtype=np.uint16))
    assert blk.tobytes() == bytes([0x00, 0x3C]) + bytes.fromhex("F0E1D2C3B4A5968778695A4B3C2D1E0F")


def _q4_and_q8(rng, n_rows, hkv, d):
    """The same V values as q4_0 rows and as q8_0 rows."""
    nb = hkv * d // 32
    nib = rng.integers(0, 16, size=(n_rows, nb, 32), dtype=np.uint8)
    sb = rng.uniform(0.08, 0.32, size=(n_rows, nb)).astype(np.float16).view(np.uint16)
    v4 = inputs.pack_q4_0(nib, sb)
    v8 = inputs.pack_q8_0(nib.astype(np.int16) - 8, sb)
    return v4, v8


@pytest.mark.parametrize("hq,hkv,d,n", [(8, 2, 64, 37), (40, 8, 128, 200), (6, 3, 32, 9)])
def test_q4_0_path_equals_q8_0_path_on_equal_values(oracle, hq, hkv, d, n):
    rng = np.random.default_rng(hq * 1000 + n)
    k = inputs.random_kv_rows(rng, n, hkv, d)
    v4, v8 = _q4_and_q8(rng, n, hkv, d)
    q = inputs.random_q(rng, 2, hq, d)
    a4 = oracle.attend(q, [[(k, v4, 0)]] * 2, hkv, d, v_type=oracle.V_Q4_0, window=n // 2 + 1)
    a8 = oracle.attend(q, [[(k, v8, 0)]] * 2, hkv, d, window=n // 2 + 1)
    assert np.array_equal(a4, a8)
    # and through two segments with padded strides
    pad4 = np.concatenate([v4, rng.integers(0, 256, (n, 6), dtype=np.uint8)], axis=1)
    s1 = n // 3
    b4 = oracle.attend(q, [[(k[:s1], pad4[:s1], 0), (k[s1:], pad4[s1:], s1)]] * 2, hkv, d,
                       v_type=oracle.V_Q4_0, window=n // 2 + 1)
    assert np.allclose(b4, a8, rtol=0, atol=1e-12)


def test_q4_0_closed_forms(oracle):
    rng = np.random.default_rng(9)
    hkv, d, hq = 2, 64, 8
    k = inputs.random_kv_rows(rng, 5, hkv, d)
    v4 = inputs.random_kv_rows_q4_0(rng, 5, hkv, d)
    q = inputs.random_q(rng, 1, hq, d)
    # one-row context: the output is that row's V (head g of query head h = h // 4)
    one = oracle.attend(q, [[(k[:1], v4[:1], 0)]], hkv, d, v_type=oracle.V_Q4_0)
    vals = oracle.dequant_q4_0(v4[0]).reshape(hkv, d)
    for h in range(hq):
        assert np.array_equal(one[0, h], vals[h // 4])
    # zero query: equal weights, the mean of V over the rows
    z = oracle.attend(np.zeros_like(q), [[(k, v4, 0)]], hkv, d, v_type=oracle.V_Q4_0)
    allv = np.stack([oracle.dequant_q4_0(v4[t]).reshape(hkv, d) for t in range(5)])
    for h in range(hq):
        assert np.allclose(z[0, h], allv[:, h // 4].mean(axis=0), rtol=0, atol=1e-15)


def test_ring_bytes_with_narrow_v_rows(oracle):
    rb8, rb4 = inputs.row_bytes(8, 128), inputs.row_bytes_q4_0(8, 128)
    assert (rb8, rb4) == (1088, 576)
    assert oracle.ring_bytes_kv(1, 16384, rb8, rb8) == oracle.ring_bytes(1, 16384, rb8)
    assert oracle.ring_bytes_kv(1, 16384, rb8, rb4) == 3 * 16384 * (1088 + 576)
    assert oracle.ring_bytes_kv(0, 16384, rb8, rb4) == 0
    # V bytes per row fall from 1088 to 576: the staged K+V per row falls by 23.5%
    assert abs(1 - (rb8 + rb4) / (2 * rb8) - 0.2353) < 1e-4


def test_oracle_rejects_unknown_v_type(oracle):
    rng = np.random.default_rng(1)
    k = inputs.random_kv_rows(rng, 3, 1, 32)
    with pytest.raises(ValueError):
        oracle.attend(inputs.random_q(rng, 1, 1, 32), [[(k, k, 0)]], 1, 32, v_type=7)
