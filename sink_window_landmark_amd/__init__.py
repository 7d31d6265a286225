"""Python binding of libswl (sink + window + landmark attention on MI355X).

Argument marshalling only: every step of the layer runs in the HIP kernels
of ``libswl.so``; this module checks tensor shapes, dtypes and devices,
turns torch tensors into device pointers and the current HIP stream into a
``hipStream_t``, and raises on a non-zero status.  The functions carry the
names of the C entry points declared in ``include/swl.h``.

There is no CPU path: if ``libswl.so`` has not been built, importing the
binding's functions raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import math
import os
from typing import Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswl.so")

SWL_OK, SWL_EINVAL, SWL_EHIP, SWL_ESIZE = 0, 1, 2, 3
SUB = 64
NOALLOC_SCRATCH_BYTES = 4 << 20   # SWL_NOALLOC_SCRATCH_BYTES

# Entry points declared by include/swl.h.
EXPORTS = ("swl_scratch_bytes", "swl_init_state", "swl_attend_chunk", "swl_commit",
           "swl_prefill", "swl_prefill_traced", "swl_commit_rows", "swl_seal", "swl_rewind",
           "swl_attend_token", "swl_status_str", "swl_prefill_fused", "swl_attend_chunk_fused",
           "swl_commit_fused", "swl_commit_rows_fused", "swl_attend_token_fused",
           "swl_attend_token_noalloc")

# Stage ids of swl_stage_fn (enum swl_stage).
STAGES = ("far_score", "far_scan", "dtheta", "theta_scan", "attend", "ring", "meta", "kv_split",
          "value_scale")
STAGE_FN = ctypes.CFUNCTYPE(None, ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p)


class SwlError(RuntimeError):
    pass


class _Geom(ctypes.Structure):
    _fields_ = [("G", ctypes.c_int32), ("H", ctypes.c_int32), ("m", ctypes.c_int32),
                ("W", ctypes.c_int32), ("ns", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("scale", ctypes.c_float), ("rect", ctypes.c_int32)]


_P = ctypes.c_void_p


class _State(ctypes.Structure):
    _fields_ = [("meta", _P), ("ring_k", _P), ("ring_v", _P), ("sink_k", _P), ("sink_v", _P),
                ("k_tilde", _P), ("q_tilde", _P), ("mu", _P), ("mz", _P), ("theta", _P)]


class _Fuse(ctypes.Structure):
    _fields_ = [("rope", _P), ("gate", _P), ("gate_scale", _P)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libswl.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise SwlError(f"libswl.so is not built ({path}); run __graft_entry__.build() or "
                       "python sink_window_landmark_amd/build.py")
    lib = ctypes.CDLL(path)
    G, S = ctypes.POINTER(_Geom), ctypes.POINTER(_State)
    lib.swl_scratch_bytes.restype = ctypes.c_size_t
    lib.swl_scratch_bytes.argtypes = [G, ctypes.c_int64]
    lib.swl_init_state.restype = ctypes.c_int
    lib.swl_init_state.argtypes = [G, S, _P, _P]
    lib.swl_attend_chunk.restype = ctypes.c_int
    lib.swl_attend_chunk.argtypes = [G, S, _P, _P, _P, ctypes.c_int32, _P, _P, ctypes.c_size_t, _P]
    lib.swl_commit.restype = ctypes.c_int
    lib.swl_commit.argtypes = [G, S, _P, _P, ctypes.c_int32, _P, ctypes.c_size_t, _P]
    lib.swl_prefill.restype = ctypes.c_int
    lib.swl_prefill.argtypes = [G, S, _P, _P, _P, ctypes.c_int64, _P, _P, ctypes.c_size_t, _P]
    lib.swl_prefill_traced.restype = ctypes.c_int
    lib.swl_prefill_traced.argtypes = [G, S, _P, _P, _P, ctypes.c_int64, _P, _P, ctypes.c_size_t,
                                       _P, STAGE_FN, _P]
    lib.swl_commit_rows.restype = ctypes.c_int
    lib.swl_commit_rows.argtypes = [G, S, _P, _P, ctypes.c_int64, _P, ctypes.c_size_t, _P]
    lib.swl_seal.restype = ctypes.c_int
    lib.swl_seal.argtypes = [G, S, _P, _P, _P, ctypes.c_int64, _P, ctypes.c_size_t, _P]
    lib.swl_rewind.restype = ctypes.c_int
    lib.swl_rewind.argtypes = [G, S, _P]
    lib.swl_attend_token.restype = ctypes.c_int
    lib.swl_attend_token.argtypes = [G, S, _P, _P, _P, _P, _P, ctypes.c_size_t, _P]
    F = ctypes.POINTER(_Fuse)
    lib.swl_prefill_fused.restype = ctypes.c_int
    lib.swl_prefill_fused.argtypes = [G, S, _P, _P, _P, ctypes.c_int64, F, _P, _P, ctypes.c_size_t,
                                      _P]
    lib.swl_attend_chunk_fused.restype = ctypes.c_int
    lib.swl_attend_chunk_fused.argtypes = [G, S, _P, _P, _P, ctypes.c_int32, F, _P, _P,
                                           ctypes.c_size_t, _P]
    lib.swl_commit_fused.restype = ctypes.c_int
    lib.swl_commit_fused.argtypes = [G, S, _P, _P, ctypes.c_int32, F, _P, ctypes.c_size_t, _P]
    lib.swl_commit_rows_fused.restype = ctypes.c_int
    lib.swl_commit_rows_fused.argtypes = [G, S, _P, _P, ctypes.c_int64, F, _P, ctypes.c_size_t, _P]
    lib.swl_attend_token_fused.restype = ctypes.c_int
    lib.swl_attend_token_fused.argtypes = [G, S, _P, _P, _P, F, _P, _P, ctypes.c_size_t, _P]
    lib.swl_attend_token_noalloc.restype = ctypes.c_int
    lib.swl_attend_token_noalloc.argtypes = [G, S, _P, _P, _P, F, _P, _P]
    lib.swl_status_str.restype = ctypes.c_char_p
    lib.swl_status_str.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


@dataclasses.dataclass(frozen=True)
class Geom:
    """Layer geometry (swl_geom): G KV groups x H query heads, m landmarks,
    ring stride W, ns sinks, key/value widths d/dv."""
    G: int
    H: int
    m: int
    W: int
    ns: int
    d: int
    dv: int
    scale: Optional[float] = None
    rect: bool = False

    @property
    def nh(self) -> int:
        return self.G * self.H

    def c(self) -> _Geom:
        """The swl_geom struct (built once per Geom)."""
        cached = self.__dict__.get("_c")
        if cached is None:
            sc = self.scale if self.scale is not None else 1.0 / math.sqrt(self.d)
            cached = _Geom(self.G, self.H, self.m, self.W, self.ns, self.d, self.dv, sc,
                           int(self.rect))
            object.__setattr__(self, "_c", cached)
        return cached


class LayerState:
    """A layer's device state as torch tensors in the swl.h layouts."""

    FIELDS = ("meta", "ring_k", "ring_v", "sink_k", "sink_v", "k_tilde", "q_tilde", "mu",
              "mz", "theta")

    def __init__(self, geom: Geom, **tensors):
        self.geom = geom
        for f in self.FIELDS:
            setattr(self, f, tensors[f])
        self._check()

    def shapes(self):
        g = self.geom
        return dict(meta=(g.G, 4), ring_k=(g.G, g.W, g.d), ring_v=(g.G, g.W, g.dv),
                    sink_k=(g.G, g.ns, g.d), sink_v=(g.G, g.ns, g.dv), k_tilde=(g.G, g.m, g.d),
                    q_tilde=(g.nh, g.m, g.d), mu=(g.nh, g.m, g.m), mz=(g.nh, 2, g.m),
                    theta=(g.nh, g.m, g.dv))

    def _check(self):
        import torch
        for f, shp in self.shapes().items():
            t = getattr(self, f)
            want = torch.int32 if f == "meta" else torch.float32
            if tuple(t.shape) != shp or t.dtype != want or not t.is_contiguous() or not t.is_cuda:
                raise ValueError(f"state.{f}: want contiguous {want} {shp} on the GPU, got "
                                 f"{t.dtype} {tuple(t.shape)} on {t.device}")

    @classmethod
    def from_host(cls, geom: Geom, host, device="cuda"):
        """Copy a host state (numpy arrays with the same field names; meta as
        u32) to the device.  ``meta`` is held as int32 bits."""
        import numpy as np
        import torch
        t = {}
        for f in cls.FIELDS:
            a = np.ascontiguousarray(getattr(host, f))
            if f == "meta":
                a = a.astype(np.uint32).view(np.int32)
            else:
                a = a.astype(np.float32)
            t[f] = torch.from_numpy(a.copy()).to(device)
        return cls(geom, **t)

    def clone(self) -> "LayerState":
        return LayerState(self.geom, **{f: getattr(self, f).clone() for f in self.FIELDS})

    def __setattr__(self, name, value):
        if name in self.FIELDS:
            self.__dict__.pop("_c", None)   # a replaced field needs a new struct
        object.__setattr__(self, name, value)

    def c(self) -> _State:
        """The swl_state struct of device pointers (built once, and again after
        a field is replaced)."""
        cached = self.__dict__.get("_c")
        if cached is None:
            cached = _State(*(getattr(self, f).data_ptr() for f in self.FIELDS))
            self.__dict__["_c"] = cached
        return cached


def _stream(stream) -> Optional[int]:
    """A hipStream_t handle: torch's current stream by default, a torch
    Stream, or an integer handle as is."""
    if isinstance(stream, int):
        return stream
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _check(name, t, shape, dtype=None):
    import torch
    dtype = dtype or torch.float32
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or not t.is_cuda:
        raise ValueError(f"{name}: want contiguous {dtype} {tuple(shape)} on the GPU, got "
                         f"{t.dtype} {tuple(t.shape)} on {t.device}")


def _raise(rc: int, what: str):
    if rc != SWL_OK:
        msg = load_library().swl_status_str(rc).decode()
        raise SwlError(f"{what}: {msg} (status {rc})")


def swl_scratch_bytes(geom: Geom, rows: int) -> int:
    return int(load_library().swl_scratch_bytes(ctypes.byref(geom.c()), int(rows)))


def alloc_scratch(geom: Geom, rows: int, device="cuda"):
    import torch
    n = swl_scratch_bytes(geom, rows)
    if n == 0:
        raise SwlError("invalid geometry")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _windows_arg(state, windows):
    """The u32 array of per-group window overrides, or None."""
    if windows is None:
        return None
    g = state.geom
    if len(windows) != g.G:
        raise ValueError("one window override per group")
    return (ctypes.c_uint32 * g.G)(*[int(w) for w in windows])


def swl_init_state(state: LayerState, windows: Optional[Sequence[int]] = None, stream=None):
    arr = _windows_arg(state, windows)
    rc = load_library().swl_init_state(ctypes.byref(state.geom.c()), ctypes.byref(state.c()),
                                       ctypes.cast(arr, _P) if arr is not None else None,
                                       _stream(stream))
    _raise(rc, "swl_init_state")


def _rows_args(state, q, k, v, out, rows):
    g = state.geom
    if q is not None:
        _check("q", q, (rows, g.nh, g.d))
    _check("k", k, (rows, g.G, g.d))
    _check("v", v, (rows, g.G, g.dv))
    if out is not None:
        _check("out", out, (rows, g.nh, g.dv))


def swl_attend_chunk(state: LayerState, q, k, v, out, scratch, stream=None):
    rows = q.shape[0]
    _rows_args(state, q, k, v, out, rows)
    rc = load_library().swl_attend_chunk(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), rows, out.data_ptr(), scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_attend_chunk")


def swl_commit(state: LayerState, k, v, scratch, stream=None):
    rows = k.shape[0]
    _rows_args(state, None, k, v, None, rows)
    rc = load_library().swl_commit(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), k.data_ptr(), v.data_ptr(), rows,
        scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_commit")


def swl_commit_rows(state: LayerState, k, v, scratch, stream=None):
    """The state after the rows of k, v without their attention (the accepted
    rows of a verify)."""
    rows = k.shape[0]
    _rows_args(state, None, k, v, None, rows)
    rc = load_library().swl_commit_rows(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), k.data_ptr(), v.data_ptr(), rows,
        scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_commit_rows")


def swl_seal(state: LayerState, k, v, scratch, windows: Optional[Sequence[int]] = None,
             stream=None):
    """The state sealed from the exact rows k, v (the landmarks, mu and sinks
    already in ``state``)."""
    rows = k.shape[0]
    _rows_args(state, None, k, v, None, rows)
    win = _windows_arg(state, windows)
    rc = load_library().swl_seal(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()),
        ctypes.cast(win, ctypes.c_void_p) if win is not None else None,
        k.data_ptr(), v.data_ptr(), rows, scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_seal")


def swl_rewind(state: LayerState, stream=None):
    """Undo the bookkeeping of the last push in every group."""
    rc = load_library().swl_rewind(ctypes.byref(state.geom.c()), ctypes.byref(state.c()),
                                   _stream(stream))
    _raise(rc, "swl_rewind")


def swl_prefill(state: LayerState, q, k, v, out, scratch, stream=None):
    rows = q.shape[0]
    _rows_args(state, q, k, v, out, rows)
    rc = load_library().swl_prefill(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), rows, out.data_ptr(), scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_prefill")


def swl_prefill_traced(state: LayerState, q, k, v, out, scratch, on_stage, stream=None):
    """swl_prefill with ``on_stage(stage_name, begin)`` called on the host around
    every launch (see swl_stage_fn)."""
    rows = q.shape[0]
    _rows_args(state, q, k, v, out, rows)
    cb = STAGE_FN(lambda sid, begin, _u: on_stage(STAGES[sid], bool(begin)))
    rc = load_library().swl_prefill_traced(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), rows, out.data_ptr(), scratch.data_ptr(), scratch.numel(), _stream(stream),
        cb, None)
    _raise(rc, "swl_prefill_traced")


def swl_attend_token(state: LayerState, q, k, v, out, scratch, stream=None):
    _rows_args(state, q, k, v, out, 1)
    rc = load_library().swl_attend_token(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), out.data_ptr(), scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_attend_token")


def _fuse_arg(state, rows, rope=None, gate=None, gate_scale=None):
    """The swl_fuse struct of optional RoPE table [rows][d], gate
    pre-activations [rows][nh][dv] and gate scale [nh][dv] (device tensors)."""
    g = state.geom
    if rope is not None:
        _check("rope", rope, (rows, g.d))
    if gate is not None:
        _check("gate", gate, (rows, g.nh, g.dv))
        if gate_scale is None:
            raise ValueError("gate needs gate_scale")
    if gate_scale is not None:
        _check("gate_scale", gate_scale, (g.nh, g.dv))
    ptr = lambda t: t.data_ptr() if t is not None else None
    return _Fuse(ptr(rope), ptr(gate), ptr(gate_scale))


def swl_prefill_fused(state: LayerState, q, k, v, out, scratch, rope=None, gate=None,
                      gate_scale=None, stream=None):
    """swl_prefill with q, k before RoPE (``rope`` table rows) and/or the
    sigmoid output gate (``gate``, ``gate_scale``)."""
    rows = q.shape[0]
    _rows_args(state, q, k, v, out, rows)
    f = _fuse_arg(state, rows, rope, gate, gate_scale)
    rc = load_library().swl_prefill_fused(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), rows, ctypes.byref(f), out.data_ptr(), scratch.data_ptr(), scratch.numel(),
        _stream(stream))
    _raise(rc, "swl_prefill_fused")


def swl_attend_chunk_fused(state: LayerState, q, k, v, out, scratch, rope=None, gate=None,
                           gate_scale=None, stream=None):
    rows = q.shape[0]
    _rows_args(state, q, k, v, out, rows)
    f = _fuse_arg(state, rows, rope, gate, gate_scale)
    rc = load_library().swl_attend_chunk_fused(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), rows, ctypes.byref(f), out.data_ptr(), scratch.data_ptr(), scratch.numel(),
        _stream(stream))
    _raise(rc, "swl_attend_chunk_fused")


def swl_commit_fused(state: LayerState, k, v, scratch, rope=None, stream=None):
    rows = k.shape[0]
    _rows_args(state, None, k, v, None, rows)
    f = _fuse_arg(state, rows, rope)
    rc = load_library().swl_commit_fused(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), k.data_ptr(), v.data_ptr(), rows,
        ctypes.byref(f), scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_commit_fused")


def swl_commit_rows_fused(state: LayerState, k, v, scratch, rope=None, stream=None):
    rows = k.shape[0]
    _rows_args(state, None, k, v, None, rows)
    f = _fuse_arg(state, rows, rope)
    rc = load_library().swl_commit_rows_fused(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), k.data_ptr(), v.data_ptr(), rows,
        ctypes.byref(f), scratch.data_ptr(), scratch.numel(), _stream(stream))
    _raise(rc, "swl_commit_rows_fused")


def swl_attend_token_fused(state: LayerState, q, k, v, out, scratch, rope=None, gate=None,
                           gate_scale=None, stream=None):
    _rows_args(state, q, k, v, out, 1)
    f = _fuse_arg(state, 1, rope, gate, gate_scale)
    rc = load_library().swl_attend_token_fused(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), ctypes.byref(f), out.data_ptr(), scratch.data_ptr(), scratch.numel(),
        _stream(stream))
    _raise(rc, "swl_attend_token_fused")


def swl_attend_token_noalloc(state: LayerState, q, k, v, out, rope=None, gate=None,
                             gate_scale=None, stream=None):
    """swl_attend_token(_fused) without a scratch argument: the library's
    static per-GPU scratch holds the partials (for callers that cannot
    allocate).  Calls that overlap on one GPU race."""
    _rows_args(state, q, k, v, out, 1)
    fz = rope is not None or gate is not None or gate_scale is not None
    f = _fuse_arg(state, 1, rope, gate, gate_scale) if fz else None
    rc = load_library().swl_attend_token_noalloc(
        ctypes.byref(state.geom.c()), ctypes.byref(state.c()), q.data_ptr(), k.data_ptr(),
        v.data_ptr(), ctypes.byref(f) if f is not None else None, out.data_ptr(),
        _stream(stream))
    _raise(rc, "swl_attend_token_noalloc")


# Short aliases.
scratch_bytes = swl_scratch_bytes
init_state = swl_init_state
attend_chunk = swl_attend_chunk
commit = swl_commit
prefill = swl_prefill
attend_token = swl_attend_token
