"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it draws random codes, scales
and queries and lays the codes out in the q8_0 byte format (a little-endian
binary16 scale followed by 32 signed int8 codes per 34-byte block; rows are
token-major, each row holding every KV head).  Decoding, attention and
anything else the method computes happen elsewhere (the HIP library, and
independently the oracle).

Recipe (the workloads the pages describe, made synthetic):
  * codes: integers uniform in [-127, 127] (never -128);
  * scales: uniform in [0.005, 0.02] drawn in fp64, rounded to binary16
    (round to nearest even); the stored bits are the truth;
  * queries: fp32 N(0, 1);
  * seed = 20260 + config index; a per-layer stream is default_rng([seed, layer]);
  * batched variable-length contexts: lognormal(mu = ln 4096, sigma = 1.0),
    rounded, clipped to [1024, 32768].
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

QK = 32
BLOCK_BYTES = 34


def row_bytes(n_head_kv: int, head_dim: int) -> int:
    """Bytes of one token row of K (or of V): every KV head, head_dim/32 blocks each."""
    return n_head_kv * (head_dim // QK) * BLOCK_BYTES


def pack_q8_0(codes: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Lay out codes int8 [..., n_blocks, 32] and binary16 bit patterns uint16
    [..., n_blocks] as 34-byte blocks -> uint8 [..., n_blocks * 34]."""
    codes = np.asarray(codes, dtype=np.int8)
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    lead = codes.shape[:-2]
    nb = codes.shape[-2]
    out = np.empty(lead + (nb, BLOCK_BYTES), dtype=np.uint8)
    out[..., 0] = (scale_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (scale_bits >> 8).astype(np.uint8)
    out[..., 2:] = codes.view(np.uint8)
    return out.reshape(lead + (nb * BLOCK_BYTES,))


def random_kv_rows(rng: np.random.Generator, n_rows: int, n_head_kv: int, head_dim: int,
                   scale_lo: float = 0.005, scale_hi: float = 0.02):
    """One tensor (K or V) of n_rows token rows -> uint8 [n_rows, row_bytes]."""
    nb = n_head_kv * head_dim // QK
    codes = rng.integers(-127, 128, size=(n_rows, nb, QK), dtype=np.int16).astype(np.int8)
    scales = rng.uniform(scale_lo, scale_hi, size=(n_rows, nb)).astype(np.float16)
    return pack_q8_0(codes, scales.view(np.uint16))


Q4_BLOCK_BYTES = 18


def row_bytes_q4_0(n_head_kv: int, head_dim: int) -> int:
    """Bytes of one token row of a q4_0 tensor: every KV head, head_dim/32 blocks of 18 B."""
    return n_head_kv * (head_dim // QK) * Q4_BLOCK_BYTES


def pack_q4_0(nibbles: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """Lay out 4-bit codes uint8 [..., n_blocks, 32] (0..15, code j of the block)
    and binary16 bit patterns [..., n_blocks] as 18-byte q4_0 blocks: byte 2 + j
    holds code j in its low nibble and code 16 + j in its high nibble."""
    nib = np.asarray(nibbles, dtype=np.uint8)
    if (nib > 15).any():
        raise ValueError("4-bit codes must be 0..15")
    scale_bits = np.asarray(scale_bits, dtype=np.uint16)
    lead = nib.shape[:-2]
    nb = nib.shape[-2]
    out = np.empty(lead + (nb, Q4_BLOCK_BYTES), dtype=np.uint8)
    out[..., 0] = (scale_bits & 0xFF).astype(np.uint8)
    out[..., 1] = (scale_bits >> 8).astype(np.uint8)
    out[..., 2:] = nib[..., :16] | (nib[..., 16:] << 4)
    return out.reshape(lead + (nb * Q4_BLOCK_BYTES,))


def random_kv_rows_q4_0(rng: np.random.Generator, n_rows: int, n_head_kv: int, head_dim: int,
                        scale_lo: float = 0.08, scale_hi: float = 0.32):
    """One q4_0 tensor (V) of n_rows token rows -> uint8 [n_rows, row_bytes_q4_0].
    Codes uniform over 0..15; the default scales (16x the q8_0 ones) give values
    d * (code - 8) over the same range as the q8_0 rows."""
    nb = n_head_kv * head_dim // QK
    nib = rng.integers(0, 16, size=(n_rows, nb, QK), dtype=np.uint8)
    scales = rng.uniform(scale_lo, scale_hi, size=(n_rows, nb)).astype(np.float16)
    return pack_q4_0(nib, scales.view(np.uint16))


def random_q(rng: np.random.Generator, n_seq: int, n_head_q: int, head_dim: int) -> np.ndarray:
    return rng.standard_normal(size=(n_seq, n_head_q, head_dim)).astype(np.float32)


def lognormal_lengths(rng: np.random.Generator, n: int, median: int = 4096, sigma: float = 1.0,
                      lo: int = 1024, hi: int = 32768) -> np.ndarray:
    x = rng.lognormal(mean=np.log(median), sigma=sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


@dataclass(frozen=True)
class Config:
    index: int
    name: str
    n_layers: int
    n_seq: int
    n_ctx: int
    n_head_q: int
    n_head_kv: int
    head_dim: int
    notes: str = ""
    extra: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return 20260 + self.index

    @property
    def row_bytes(self) -> int:
        return row_bytes(self.n_head_kv, self.head_dim)

    def layer_rng(self, layer: int) -> np.random.Generator:
        return np.random.default_rng([self.seed, layer])


CONFIGS = {
    0: Config(0, "tiny", 1, 1, 256, 8, 2, 64, "device-resident, oracle-sized"),
    1: Config(1, "single_layer_4k", 1, 1, 4096, 40, 8, 128, "device-resident, HBM GB/s"),
    2: Config(2, "host_resident_16k", 64, 1, 16384, 40, 8, 128, "pinned host KV, depth 0 vs 1, 128 MiB",
              {"gemv": (5120, 27648), "depths": (0, 1), "budgets_mib": (128,)}),
    3: Config(3, "host_resident_128k", 64, 1, 131072, 40, 8, 128, "pinned host KV, depth 0/1/2",
              {"gemv": (5120, 27648), "depths": (0, 1, 2), "budgets_mib": (128, 1024)}),
    4: Config(4, "batched_varlen_swa", 64, 16, 4096, 40, 8, 128, "lognormal lengths, SWA odd layers",
              {"window": 4096, "depth": 1, "budget_mib": 1024}),
}


def config(i: int) -> Config:
    return CONFIGS[i]
