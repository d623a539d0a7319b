"""fp64 CPU oracle for decode attention over a q8_0 KV cache.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The product library
(``decode_attention_offloaded_amd``) never imports, links or calls it, and this
package imports nothing from the product.

The arithmetic lives in ``kvd_oracle.c`` (plain C, fp64); this module builds it
with gcc when no built copy exists and marshals numpy arrays into it.  See the
header of ``kvd_oracle.c`` for what is computed and which passages of the pages
each step follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kvd_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libkvd_oracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP for the multi-core baseline)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-fopenmp", "-Wall", "-shared", "-fPIC",
                               _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class Seg(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_rows", ctypes.c_int64),
                ("pos0", ctypes.c_int64), ("row_stride", ctypes.c_int64)]


class SegKV(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_rows", ctypes.c_int64),
                ("pos0", ctypes.c_int64), ("k_stride", ctypes.c_int64), ("v_stride", ctypes.c_int64)]


V_Q8_0, V_Q4_0 = 0, 1


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        L.kvd_oracle_f16_to_f64.restype = ctypes.c_double
        L.kvd_oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
        L.kvd_oracle_dequant_q8_0.restype = None
        L.kvd_oracle_dequant_q8_0.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.kvd_oracle_attend_f64.restype = ctypes.c_int
        L.kvd_oracle_attend_f64.argtypes = [ctypes.c_int32] * 6 + [
            ctypes.c_double, ctypes.c_void_p, ctypes.POINTER(Seg), ctypes.c_void_p, ctypes.c_void_p,
            ctypes.c_int32]
        L.kvd_oracle_dequant_q4_0.restype = None
        L.kvd_oracle_dequant_q4_0.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
        L.kvd_oracle_attend_kv_f64.restype = ctypes.c_int
        L.kvd_oracle_attend_kv_f64.argtypes = [ctypes.c_int32] * 6 + [
            ctypes.c_double, ctypes.c_int32, ctypes.c_void_p, ctypes.POINTER(SegKV), ctypes.c_void_p,
            ctypes.c_void_p, ctypes.c_int32]
        L.kvd_oracle_ring_bytes_kv.restype = ctypes.c_int64
        L.kvd_oracle_ring_bytes_kv.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        L.kvd_oracle_ring_bytes.restype = ctypes.c_int64
        L.kvd_oracle_ring_bytes.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64]
        L.kvd_oracle_ring_fits.restype = ctypes.c_int
        L.kvd_oracle_ring_fits.argtypes = [ctypes.c_int32, ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        _lib = L
    return _lib


def f16_to_f64(bits) -> np.ndarray:
    """Decode binary16 bit patterns one by one through the C decoder."""
    L = lib()
    bits = np.asarray(bits, dtype=np.uint16).ravel()
    return np.array([L.kvd_oracle_f16_to_f64(int(b)) for b in bits], dtype=np.float64)


def dequant_q8_0(blocks: np.ndarray) -> np.ndarray:
    """Dequantise a byte buffer of whole q8_0 blocks (34 bytes each) to fp64."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).ravel()
    if b.size % 34:
        raise ValueError("not a whole number of 34-byte blocks")
    n = b.size // 34
    out = np.empty(n * 32, dtype=np.float64)
    lib().kvd_oracle_dequant_q8_0(b.ctypes.data, n, out.ctypes.data)
    return out


def attend(q: np.ndarray, segs, n_head_kv: int, head_dim: int, window: int = 0, scale=None,
           q_pos=None, threads: int = 1, v_type: int = V_Q8_0) -> np.ndarray:
    """Decode attention in fp64.

    q      : float32 [n_seq, n_head_q, head_dim]
    segs   : per sequence, a list of segments ``(k_rows, v_rows, pos0)``; k_rows and
             v_rows are uint8 arrays [n_rows, row_bytes] (row_bytes >= the packed row;
             V rows may be narrower than K rows when V is q4_0).
    q_pos  : None (query at the newest row) or a sequence of ints.
    v_type : V_Q8_0 (34-byte blocks) or V_Q4_0 (18-byte blocks); K is always q8_0.
    Returns float64 [n_seq, n_head_q, head_dim].
    """
    q = np.ascontiguousarray(q, dtype=np.float32)
    n_seq, n_head_q, hd = q.shape
    assert hd == head_dim
    n_seg = len(segs[0])
    if any(len(s) != n_seg for s in segs):
        raise ValueError("every sequence needs the same number of segments")
    keep = []
    arr = (SegKV * (n_seq * n_seg))()
    for s, seq in enumerate(segs):
        for j, (k_rows, v_rows, pos0) in enumerate(seq):
            k_rows = np.ascontiguousarray(k_rows, dtype=np.uint8)
            v_rows = np.ascontiguousarray(v_rows, dtype=np.uint8)
            if k_rows.ndim != 2 or v_rows.ndim != 2 or k_rows.shape[0] != v_rows.shape[0]:
                raise ValueError("segment rows must be 2-D with as many V rows as K rows")
            if v_type == V_Q8_0 and k_rows.shape != v_rows.shape:
                raise ValueError("q8_0 V rows must match the K rows")
            keep += [k_rows, v_rows]
            arr[s * n_seg + j] = SegKV(k_rows.ctypes.data, v_rows.ctypes.data, k_rows.shape[0], int(pos0),
                                       k_rows.shape[1], v_rows.shape[1])
    qp = None
    if q_pos is not None:
        qp = np.ascontiguousarray(q_pos, dtype=np.int64)
        keep.append(qp)
    if scale is None:
        scale = 1.0 / np.sqrt(head_dim)
    out = np.empty((n_seq, n_head_q, head_dim), dtype=np.float64)
    rc = lib().kvd_oracle_attend_kv_f64(n_seq, n_head_q, n_head_kv, head_dim, n_seg, int(window), float(scale),
                                        int(v_type), q.ctypes.data, arr, None if qp is None else qp.ctypes.data,
                                        out.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the input (rc=%d)" % rc)
    return out


def attend_symmetric(q: np.ndarray, segs, n_head_kv: int, head_dim: int, window: int = 0, scale=None,
                     q_pos=None, threads: int = 1) -> np.ndarray:
    """The q8_0/q8_0 entry point with one row stride per segment (kvd_oracle_attend_f64)."""
    q = np.ascontiguousarray(q, dtype=np.float32)
    n_seq, n_head_q, _ = q.shape
    n_seg = len(segs[0])
    keep = []
    arr = (Seg * (n_seq * n_seg))()
    for s, seq in enumerate(segs):
        for j, (k_rows, v_rows, pos0) in enumerate(seq):
            k_rows = np.ascontiguousarray(k_rows, dtype=np.uint8)
            v_rows = np.ascontiguousarray(v_rows, dtype=np.uint8)
            keep += [k_rows, v_rows]
            arr[s * n_seg + j] = Seg(k_rows.ctypes.data, v_rows.ctypes.data, k_rows.shape[0], int(pos0),
                                     k_rows.shape[1])
    qp = None if q_pos is None else np.ascontiguousarray(q_pos, dtype=np.int64)
    scale = 1.0 / np.sqrt(head_dim) if scale is None else scale
    out = np.empty((n_seq, n_head_q, head_dim), dtype=np.float64)
    rc = lib().kvd_oracle_attend_f64(n_seq, n_head_q, n_head_kv, head_dim, n_seg, int(window), float(scale),
                                     q.ctypes.data, arr, None if qp is None else qp.ctypes.data,
                                     out.ctypes.data, int(threads))
    if rc != 0:
        raise ValueError("oracle rejected the input (rc=%d)" % rc)
    return out


def dequant_q4_0(blocks: np.ndarray) -> np.ndarray:
    """Dequantise a byte buffer of whole q4_0 blocks (18 bytes each) to fp64."""
    b = np.ascontiguousarray(blocks, dtype=np.uint8).ravel()
    if b.size % 18:
        raise ValueError("not a whole number of 18-byte blocks")
    n = b.size // 18
    out = np.empty(n * 32, dtype=np.float64)
    lib().kvd_oracle_dequant_q4_0(b.ctypes.data, n, out.ctypes.data)
    return out


def ring_bytes_kv(depth: int, cap_rows: int, k_row_bytes: int, v_row_bytes: int) -> int:
    return int(lib().kvd_oracle_ring_bytes_kv(depth, cap_rows, k_row_bytes, v_row_bytes))


def ring_bytes(depth: int, cap_rows: int, row_bytes: int) -> int:
    return int(lib().kvd_oracle_ring_bytes(depth, cap_rows, row_bytes))


def ring_fits(depth: int, cap_rows: int, row_bytes: int, budget_bytes: int) -> bool:
    return bool(lib().kvd_oracle_ring_fits(depth, cap_rows, row_bytes, budget_bytes))
