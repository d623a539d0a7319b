"""Thin ctypes binding over ``libkvd.so`` (the C ABI in ``include/kvd.h``).

Argument marshalling only: every step of the path runs in the library's HIP
kernels and HIP runtime calls.  Torch provides device memory, pinned host
memory and streams.  If the library is not built this module raises; it has no
fallback of any kind.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libkvd.so")

KVD_OK = 0
KVD_DECLINED = 1
KVD_EINVAL = -1
KVD_ENOMEM = -2
KVD_EHIP = -3
KVD_ESTATE = -4
STAGE_PREFETCH = 1
STAGE_ACQUIRE = 2
TYPE_Q8_0 = 0
TYPE_Q4_0 = 1


class KvSeg(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_rows", ctypes.c_int64),
                ("pos0", ctypes.c_int64), ("row_stride", ctypes.c_int64), ("v_row_stride", ctypes.c_int64)]


class AttnArgs(ctypes.Structure):
    _fields_ = [("n_seq", ctypes.c_int32), ("n_head_q", ctypes.c_int32), ("n_head_kv", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("n_seg", ctypes.c_int32), ("window", ctypes.c_int32),
                ("split_rows", ctypes.c_int32), ("scale", ctypes.c_float), ("q", ctypes.c_void_p),
                ("out", ctypes.c_void_p), ("segs", ctypes.POINTER(KvSeg)), ("q_pos", ctypes.POINTER(ctypes.c_int64)),
                ("workspace", ctypes.c_void_p), ("workspace_bytes", ctypes.c_size_t), ("v_type", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class StageArgs(ctypes.Structure):
    _fields_ = [("layer", ctypes.c_int32), ("flags", ctypes.c_int32), ("host_k", ctypes.c_void_p),
                ("host_v", ctypes.c_void_p), ("row_bytes", ctypes.c_int64), ("n_rows", ctypes.c_int64),
                ("stable_rows", ctypes.c_int64), ("cap_rows", ctypes.c_int64), ("ordered_k", ctypes.c_void_p),
                ("ordered_v", ctypes.c_void_p), ("v_row_bytes", ctypes.c_int64)]


class SlotView(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("n_rows", ctypes.c_int64),
                ("row_stride", ctypes.c_int64), ("pipelined", ctypes.c_int32), ("slot", ctypes.c_int32),
                ("v_row_stride", ctypes.c_int64)]


class ResidencyPlan(ctypes.Structure):
    _fields_ = [("n_resident", ctypes.c_int32), ("use_ring", ctypes.c_int32), ("resident_bytes", ctypes.c_int64),
                ("ring_bytes", ctypes.c_int64), ("staged_bytes_per_step", ctypes.c_int64),
                ("est_ms_per_step", ctypes.c_double)]


class RingStats(ctypes.Structure):
    _fields_ = [("depth", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("engaged", ctypes.c_int32),
                ("declined", ctypes.c_int32), ("device", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("budget_bytes", ctypes.c_int64), ("need_bytes", ctypes.c_int64), ("ring_bytes", ctypes.c_int64),
                ("slot_rows", ctypes.c_int64), ("n_prefetch", ctypes.c_int64),
                ("n_acquire_pipelined", ctypes.c_int64), ("n_acquire_primed", ctypes.c_int64),
                ("n_acquire_ordered", ctypes.c_int64), ("bytes_early", ctypes.c_int64),
                ("bytes_late", ctypes.c_int64), ("bytes_ordered", ctypes.c_int64)]


class KvdError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__("kvd error %d: %s" % (code, msg))
        self.code = code


_lib = None


def _declare(L):
    c_int, c_void_p, c_size_t = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    L.kvd_last_error.restype = ctypes.c_char_p
    L.kvd_last_error.argtypes = []
    L.kvd_version.restype = ctypes.c_char_p
    L.kvd_version.argtypes = []
    L.kvd_link_probe.restype = c_int
    L.kvd_link_probe.argtypes = [c_size_t, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    L.kvd_hbm_read_probe.restype = c_int
    L.kvd_hbm_read_probe.argtypes = [c_size_t, ctypes.c_int32, ctypes.POINTER(ctypes.c_double)]
    L.kvd_attend_workspace_bytes.restype = c_int
    L.kvd_attend_workspace_bytes.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(c_size_t)]
    L.kvd_attend_plan.restype = c_int
    L.kvd_attend_plan.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(ctypes.c_int32),
                                  ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_int64)]
    L.kvd_attend_load_mode.restype = c_int
    L.kvd_attend_load_mode.argtypes = [ctypes.POINTER(AttnArgs), ctypes.POINTER(ctypes.c_int32)]
    L.kvd_attend_decode.restype = c_int
    L.kvd_attend_decode.argtypes = [ctypes.POINTER(AttnArgs), c_void_p]
    L.kvd_attend_decode_noalloc.restype = c_int
    L.kvd_attend_decode_noalloc.argtypes = [ctypes.POINTER(AttnArgs), c_void_p]
    L.kvd_attend_decode_partial.restype = c_int
    L.kvd_attend_decode_partial.argtypes = [ctypes.POINTER(AttnArgs), c_void_p, c_void_p]
    L.kvd_attend_merge.restype = c_int
    L.kvd_attend_merge.argtypes = [c_void_p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                   c_void_p, c_void_p]
    L.kvd_ring_tile_rows.restype = c_int
    L.kvd_ring_tile_rows.argtypes = [ctypes.c_int32, c_size_t, ctypes.c_int64, ctypes.c_double,
                                     ctypes.POINTER(ctypes.c_int64)]
    L.kvd_plan_residency.restype = c_int
    L.kvd_plan_residency.argtypes = [ctypes.c_int32, ctypes.c_int64, c_size_t, ctypes.c_int32, ctypes.c_double,
                                     ctypes.c_double, ctypes.POINTER(ResidencyPlan)]
    L.kvd_ring_create.restype = c_void_p
    L.kvd_ring_create.argtypes = [ctypes.c_int32, c_size_t]
    L.kvd_ring_stage_layer.restype = c_int
    L.kvd_ring_stage_layer.argtypes = [c_void_p, ctypes.POINTER(StageArgs), c_void_p, ctypes.POINTER(SlotView)]
    L.kvd_ring_release.restype = c_int
    L.kvd_ring_release.argtypes = [c_void_p, ctypes.c_int32, c_void_p]
    L.kvd_ring_stats_get.restype = c_int
    L.kvd_ring_stats_get.argtypes = [c_void_p, ctypes.POINTER(RingStats), c_size_t]
    L.kvd_ring_set_transfer_delay.restype = c_int
    L.kvd_ring_set_transfer_delay.argtypes = [c_void_p, ctypes.c_uint32, ctypes.c_uint64]
    L.kvd_ring_destroy.restype = None
    L.kvd_ring_destroy.argtypes = [c_void_p]


def lib():
    """The loaded library; raises if it has not been built (no fallback)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libkvd.so is not built (run __graft_entry__.build() or "
                               "python -m decode_attention_offloaded_amd.build)")
        # Load torch's HIP runtime first so that libkvd.so binds to the same
        # libamdhip64 (same soname): one runtime, shared streams and memory.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        L = ctypes.CDLL(LIB_PATH)
        _declare(L)
        _lib = L
    return _lib


def last_error() -> str:
    return lib().kvd_last_error().decode()


def version() -> str:
    return lib().kvd_version().decode()


def link_probe(nbytes: int, n_streams: int = 2, reps: int = 10) -> float:
    """kvd_link_probe: pinned host-to-device GB/s over n_streams streams (median of reps)."""
    g = ctypes.c_double(0.0)
    _check(lib().kvd_link_probe(int(nbytes), int(n_streams), int(reps), ctypes.byref(g)))
    return float(g.value)


def hbm_read_probe(nbytes: int, reps: int = 7) -> float:
    """kvd_hbm_read_probe: streaming-read GB/s of device memory (median of reps)."""
    g = ctypes.c_double(0.0)
    _check(lib().kvd_hbm_read_probe(int(nbytes), int(reps), ctypes.byref(g)))
    return float(g.value)


def _check(rc: int, allow=(KVD_OK,)) -> int:
    if rc not in allow:
        raise KvdError(rc, last_error())
    return rc


def _stream_handle(stream) -> int:
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return int(stream.cuda_stream) if hasattr(stream, "cuda_stream") else int(stream)


# ------------------------------------------------------------------ attention

def make_args(q, out, segs: Sequence[Sequence], n_head_kv: int, window: int = 0, scale: Optional[float] = None,
              q_pos=None, split_rows: int = 0, v_type: int = TYPE_Q8_0):
    """Build kvd_attn_args from torch tensors.

    q, out : float32 CUDA tensors [n_seq, n_head_q, head_dim], contiguous.
    segs   : per sequence, a list of segments ``(k, v, pos0)``; k and v are uint8
             CUDA tensors [n_rows, >= row bytes] (row strides k.stride(0) and
             v.stride(0); v narrower than k when v_type is TYPE_Q4_0); or
             ``(k_ptr, v_ptr, n_rows, pos0, row_stride[, v_row_stride])`` with raw
             device addresses.
    Returns (AttnArgs, keepalive).
    """
    n_seq, n_head_q, head_dim = q.shape
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must have q's shape")
    n_seg = len(segs[0])
    arr = (KvSeg * (n_seq * n_seg))()
    for s, seq in enumerate(segs):
        if len(seq) != n_seg:
            raise ValueError("every sequence needs the same number of segments")
        for j, seg in enumerate(seq):
            if len(seg) == 3:
                k, v, pos0 = seg
                if k.dtype.itemsize != 1 or v.dtype.itemsize != 1 or k.dim() != 2 or v.dim() != 2:
                    raise ValueError("segment k/v must be 2-D byte tensors")
                if k.shape[0] != v.shape[0]:
                    raise ValueError("segment k and v must have as many rows")
                if v_type == TYPE_Q8_0 and (tuple(k.shape) != tuple(v.shape) or k.stride() != v.stride()):
                    raise ValueError("q8_0 segment k/v must share one geometry")
                if k.stride(1) != 1 or v.stride(1) != 1:
                    raise ValueError("segment rows must be contiguous")
                arr[s * n_seg + j] = KvSeg(k.data_ptr(), v.data_ptr(), k.shape[0], int(pos0), k.stride(0),
                                           v.stride(0))
            else:
                kp, vp, n_rows, pos0, stride = seg[:5]
                vstride = seg[5] if len(seg) > 5 else 0
                arr[s * n_seg + j] = KvSeg(int(kp), int(vp), int(n_rows), int(pos0), int(stride), int(vstride))
    qp = None
    if q_pos is not None:
        qp = (ctypes.c_int64 * n_seq)(*[int(x) for x in q_pos])
    if scale is None:
        scale = head_dim ** -0.5
    a = AttnArgs(n_seq, n_head_q, n_head_kv, head_dim, n_seg, int(window), int(split_rows), float(scale),
                 q.data_ptr(), out.data_ptr(), arr, qp, None, 0, int(v_type), 0)
    return a, (arr, qp)


def workspace_bytes(args: AttnArgs) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().kvd_attend_workspace_bytes(ctypes.byref(args), ctypes.byref(n)))
    return int(n.value)


def attend_plan(args: AttnArgs):
    """(rows per split, waves per decode workgroup, total splits) of a call."""
    sr, w, ns = ctypes.c_int32(0), ctypes.c_int32(0), ctypes.c_int64(0)
    _check(lib().kvd_attend_plan(ctypes.byref(args), ctypes.byref(sr), ctypes.byref(w), ctypes.byref(ns)))
    return int(sr.value), int(w.value), int(ns.value)


def attend_load_mode(args: AttnArgs) -> int:
    """The decode kernel's load mode for the call's first launch (0 dword, 1
    16-byte via registers, 2 16-byte straight into LDS)."""
    m = ctypes.c_int32(-1)
    _check(lib().kvd_attend_load_mode(ctypes.byref(args), ctypes.byref(m)))
    return int(m.value)


class Workspace:
    """Per-device scratch for split partials, grown on demand and reused.

    Calls that share a workspace must be ordered (one stream, or streams
    ordered by events): they write the same partials.  Growing it waits for
    the device first, so no launch still in flight uses the buffer it drops.
    A buffer that a captured graph may use (handed out during capture) is
    never dropped: when the workspace grows past it, during capture or later,
    it is kept for the life of the workspace, since the graph can replay into
    it at any time.
    """

    def __init__(self):
        self._buf = {}
        self._captured = set()  # device indices whose current buffer a captured graph uses
        self._kept = []

    def get(self, nbytes: int, device):
        import torch
        if nbytes == 0:
            return None
        key = torch.device(device).index
        capturing = torch.cuda.is_current_stream_capturing()
        buf = self._buf.get(key)
        if buf is None or buf.numel() < nbytes:
            if buf is not None:
                if capturing or key in self._captured:
                    self._kept.append(buf)
                else:
                    torch.cuda.synchronize(device)
                nbytes = max(nbytes, 2 * buf.numel())
            buf = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=device)
            self._buf[key] = buf
            self._captured.discard(key)
        if capturing:
            self._captured.add(key)
        return buf


_default_ws = Workspace()


def attend_decode(q, out, segs, n_head_kv: int, window: int = 0, scale: Optional[float] = None, q_pos=None,
                  split_rows: int = 0, stream=None, workspace: Optional[Workspace] = None, v_type: int = TYPE_Q8_0):
    """Enqueue decode attention on ``stream`` (default: torch's current stream).

    ``workspace`` holds the split partials (default: one shared by every call
    that passes none); calls that share one must be ordered on the device."""
    import torch
    if not (q.is_cuda and out.is_cuda) or q.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("q and out must be float32 CUDA tensors")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous")
    a, keep = make_args(q, out, segs, n_head_kv, window, scale, q_pos, split_rows, v_type)
    nbytes = workspace_bytes(a)
    ws = (workspace or _default_ws).get(nbytes, q.device)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
    _check(lib().kvd_attend_decode(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out


def attend_decode_noalloc(q, out, segs, n_head_kv: int, window: int = 0, scale: Optional[float] = None,
                          q_pos=None, split_rows: int = 0, stream=None, v_type: int = TYPE_Q8_0):
    """kvd_attend_decode_noalloc: as attend_decode, with the split partials in
    the library's built-in device array (no workspace, no allocation).  Calls
    on one GPU share that array and must be ordered."""
    import torch
    if not (q.is_cuda and out.is_cuda) or q.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("q and out must be float32 CUDA tensors")
    if not (q.is_contiguous() and out.is_contiguous()):
        raise ValueError("q and out must be contiguous")
    a, keep = make_args(q, out, segs, n_head_kv, window, scale, q_pos, split_rows, v_type)
    _check(lib().kvd_attend_decode_noalloc(ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream))))
    return out


def partial_floats(n_seq: int, n_head_q: int, head_dim: int) -> int:
    """Floats of one partial result: o [S][H][D], then m [S][H], then l [S][H]."""
    return (head_dim + 2) * n_seq * n_head_q


def attend_decode_partial(q, partial, segs, n_head_kv: int, window: int = 0, scale: Optional[float] = None,
                          q_pos=None, split_rows: int = 0, stream=None, workspace: Optional[Workspace] = None,
                          v_type: int = TYPE_Q8_0):
    """Enqueue decode attention over these rows only, leaving the unnormalised
    result (o, m, l) in ``partial`` (a float32 CUDA tensor of at least
    partial_floats(...) elements, e.g. one row of a [n_part, ...] tensor)."""
    import torch
    if not (q.is_cuda and partial.is_cuda) or q.dtype != torch.float32 or partial.dtype != torch.float32:
        raise ValueError("q and partial must be float32 CUDA tensors")
    if not (q.is_contiguous() and partial.is_contiguous()):
        raise ValueError("q and partial must be contiguous")
    n_seq, n_head_q, head_dim = q.shape
    if partial.numel() < partial_floats(n_seq, n_head_q, head_dim):
        raise ValueError("partial is too small")
    a, keep = make_args(q, q, segs, n_head_kv, window, scale, q_pos, split_rows, v_type)
    a.out = None
    nbytes = workspace_bytes(a)
    ws = (workspace or _default_ws).get(nbytes, q.device)
    if ws is not None:
        a.workspace = ws.data_ptr()
        a.workspace_bytes = ws.numel()
    _check(lib().kvd_attend_decode_partial(ctypes.byref(a), ctypes.c_void_p(partial.data_ptr()),
                                           ctypes.c_void_p(_stream_handle(stream))))
    return partial


def attend_merge(partials, n_part: int, out, stream=None):
    """out[S, H, D] = merge of partials[0:n_part] (a contiguous float32 CUDA
    tensor holding n_part partial results back to back), in part order."""
    import torch
    if not (partials.is_cuda and out.is_cuda) or partials.dtype != torch.float32 or out.dtype != torch.float32:
        raise ValueError("partials and out must be float32 CUDA tensors")
    if not (partials.is_contiguous() and out.is_contiguous()):
        raise ValueError("partials and out must be contiguous")
    n_seq, n_head_q, head_dim = out.shape
    if partials.numel() < n_part * partial_floats(n_seq, n_head_q, head_dim):
        raise ValueError("partials holds fewer than n_part results")
    _check(lib().kvd_attend_merge(ctypes.c_void_p(partials.data_ptr()), int(n_part), int(n_seq), int(n_head_q),
                                  int(head_dim), ctypes.c_void_p(out.data_ptr()),
                                  ctypes.c_void_p(_stream_handle(stream))))
    return out


def tile_rows(depth: int, budget_bytes: int, row_bytes: int, max_tile_bytes: float = 0.0):
    """(rc, rows) from kvd_ring_tile_rows: rc is KVD_OK or KVD_DECLINED."""
    r = ctypes.c_int64(0)
    rc = lib().kvd_ring_tile_rows(int(depth), int(budget_bytes), int(row_bytes), float(max_tile_bytes),
                                  ctypes.byref(r))
    if rc < 0:
        raise KvdError(rc, last_error())
    return rc, int(r.value)


def plan_residency(n_layers: int, layer_bytes: int, budget_bytes: int, depth: int, link_gbps: float = 0.0,
                   compute_ms: float = 0.0) -> dict:
    """kvd_plan_residency as a dict."""
    p = ResidencyPlan()
    _check(lib().kvd_plan_residency(int(n_layers), int(layer_bytes), int(budget_bytes), int(depth),
                                    float(link_gbps), float(compute_ms), ctypes.byref(p)))
    return {name: getattr(p, name) for name, _ in ResidencyPlan._fields_}


# ------------------------------------------------------------------ staging ring

class Ring:
    """A staging ring (``kvd_ring_*``).  One host thread, one device."""

    def __init__(self, depth: int, budget_bytes: int):
        h = lib().kvd_ring_create(int(depth), int(budget_bytes))
        if not h:
            raise KvdError(KVD_EINVAL, last_error())
        self._h = ctypes.c_void_p(h)
        self.depth = depth

    def stage(self, layer: int, flags: int, host_k: int, host_v: int, row_bytes: int, n_rows: int,
              stable_rows: int, cap_rows: int, ordered_k: int = 0, ordered_v: int = 0, stream=None,
              v_row_bytes: int = 0):
        """Returns (rc, SlotView); rc is KVD_OK or KVD_DECLINED, errors raise."""
        a = StageArgs(int(layer), int(flags), int(host_k), int(host_v), int(row_bytes), int(n_rows),
                      int(stable_rows), int(cap_rows), int(ordered_k) or None, int(ordered_v) or None,
                      int(v_row_bytes))
        view = SlotView()
        rc = lib().kvd_ring_stage_layer(self._h, ctypes.byref(a), ctypes.c_void_p(_stream_handle(stream)),
                                        ctypes.byref(view))
        _check(rc, (KVD_OK, KVD_DECLINED))
        return rc, view

    def release(self, layer: int, stream=None):
        _check(lib().kvd_ring_release(self._h, int(layer), ctypes.c_void_p(_stream_handle(stream))))

    def set_transfer_delay(self, max_us: int, seed: int = 1):
        """Test support: random 0..max_us microsecond holds before every
        transfer-stream copy (0 = off)."""
        _check(lib().kvd_ring_set_transfer_delay(self._h, int(max_us), int(seed)))

    def stats(self) -> dict:
        st = RingStats()
        _check(lib().kvd_ring_stats_get(self._h, ctypes.byref(st), ctypes.sizeof(st)))
        return {name: getattr(st, name) for name, _ in RingStats._fields_}

    def close(self):
        if self._h:
            lib().kvd_ring_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
