"""CPU oracle of the sealed O(1) attention layer.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg may import this package; the GPU library and
its Python binding never do, and nothing here imports them.

* ``SerialOracle``: a float64 serial stepper (``swl_oracle.c``), one row at
  a time, restated from the chunk kernels of cortiq-engine 0.8.51
  ``src/gpu_wgpu/o1_batch.rs`` run with a chunk of one row (see the C file's
  header for the step).  Groups are independent; within a group the heads
  are split over threads that each replay the group's ring pushes.
* ``chunked``: a float64 numpy restatement of the 64-row sub-chunk
  algorithm of the same page (far max jumps to its post-chunk value, prefix
  far mass, in-chunk causal coefficients), used to pin the serial oracle
  ("chunked equals serial up to rounding", o1_batch.rs module doc).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "swl_oracle.c")
_LIB = os.path.join(_HERE, "libswl_oracle.so")
_lock = threading.Lock()
_lib = None


def build() -> str:
    """Compile the C oracle (gcc, -O2, no fast-math)."""
    cmd = ["gcc", "-O2", "-fno-fast-math", "-shared", "-fPIC", "-std=c11",
           _SRC, "-o", _LIB + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB + ".tmp", _LIB)
    return _LIB


class _Geom(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("m", ctypes.c_int32), ("W", ctypes.c_int32),
                ("wg", ctypes.c_int32), ("ns", ctypes.c_int32), ("d", ctypes.c_int32),
                ("dv", ctypes.c_int32), ("rect", ctypes.c_int32), ("scale", ctypes.c_double),
                ("h_lo", ctypes.c_int32), ("h_hi", ctypes.c_int32)]


_P = ctypes.c_void_p


class _State(ctypes.Structure):
    _fields_ = [("meta", _P), ("ring_k", _P), ("ring_v", _P), ("sink_k", _P),
                ("sink_v", _P), ("k_tilde", _P), ("q_tilde", _P), ("mu", _P),
                ("M", _P), ("Z", _P), ("theta", _P)]


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
            lib.swlo_step_rows.restype = ctypes.c_int
            lib.swlo_step_rows.argtypes = [
                ctypes.POINTER(_Geom), ctypes.POINTER(_State), ctypes.c_int64,
                _P, ctypes.c_int64, _P, ctypes.c_int64, _P, ctypes.c_int64,
                _P, ctypes.c_int64, _P]
            _lib = lib
    return _lib


def _ptr(a: np.ndarray, offset_elems: int = 0) -> int:
    return a.ctypes.data + offset_elems * a.itemsize


class SerialOracle:
    """float64 serial stepper over a whole layer (all groups).

    ``state`` is a :class:`synth.State` (fp32 arrays, u32 meta) — the same
    layouts the GPU library takes.  ``geom`` fields: G, H, m, W, ns, d, dv,
    scale, rect.
    """

    def __init__(self, G, H, m, W, ns, d, dv, scale, rect, state, threads: Optional[int] = None):
        self.G, self.H, self.m, self.W, self.ns, self.d, self.dv = G, H, m, W, ns, d, dv
        self.scale, self.rect = float(scale), int(bool(rect))
        nh = G * H
        meta = np.asarray(state.meta, dtype=np.int64).reshape(G, 4)
        self.windows = [int(meta[g, 3]) if meta[g, 3] else W for g in range(G)]
        self.sink_k = np.ascontiguousarray(state.sink_k, np.float64).reshape(G, ns, d)
        self.sink_v = np.ascontiguousarray(state.sink_v, np.float64).reshape(G, ns, dv)
        self.k_tilde = np.ascontiguousarray(state.k_tilde, np.float64).reshape(G, m, d)
        self.q_tilde = np.ascontiguousarray(state.q_tilde, np.float64).reshape(nh, m, d)
        self.mu = np.ascontiguousarray(state.mu, np.float64).reshape(nh, m, m)
        mz = np.asarray(state.mz, np.float64).reshape(nh, 2, m)
        self.M = np.ascontiguousarray(mz[:, 0, :])
        self.Z = np.ascontiguousarray(mz[:, 1, :])
        self.theta = np.ascontiguousarray(state.theta, np.float64).reshape(nh, m, dv)
        threads = threads or min(nh, os.cpu_count() or 1)
        per_group = max(1, min(H, threads // G if threads >= G else 1))
        bounds = np.linspace(0, H, per_group + 1).astype(int)
        self.parts = []  # (g, h_lo, h_hi, meta(int64[3]), ring_k, ring_v)
        for g in range(G):
            for i in range(per_group):
                h_lo, h_hi = int(bounds[i]), int(bounds[i + 1])
                if h_hi <= h_lo:
                    continue
                self.parts.append(dict(
                    g=g, h_lo=h_lo, h_hi=h_hi,
                    meta=np.array(meta[g, :3], dtype=np.int64, copy=True),
                    ring_k=np.array(state.ring_k[g], np.float64, copy=True).reshape(W, d),
                    ring_v=np.array(state.ring_v[g], np.float64, copy=True).reshape(W, dv)))
        self.threads = min(len(self.parts), threads)

    # -- stepping -------------------------------------------------------------
    def _run_part(self, p, q, k, v, out, slots):
        lib = _load()
        g = p["g"]
        H, m, d, dv, G = self.H, self.m, self.d, self.dv, self.G
        geom = _Geom(H=H, m=m, W=self.W, wg=self.windows[g], ns=self.ns, d=d, dv=dv,
                     rect=self.rect, scale=self.scale, h_lo=p["h_lo"], h_hi=p["h_hi"])
        st = _State(meta=_ptr(p["meta"]), ring_k=_ptr(p["ring_k"]), ring_v=_ptr(p["ring_v"]),
                    sink_k=_ptr(self.sink_k, g * self.ns * d),
                    sink_v=_ptr(self.sink_v, g * self.ns * dv),
                    k_tilde=_ptr(self.k_tilde, g * m * d),
                    q_tilde=_ptr(self.q_tilde, g * H * m * d),
                    mu=_ptr(self.mu, g * H * m * m),
                    M=_ptr(self.M, g * H * m), Z=_ptr(self.Z, g * H * m),
                    theta=_ptr(self.theta, g * H * m * dv))
        rows = q.shape[0]
        rc = lib.swlo_step_rows(
            ctypes.byref(geom), ctypes.byref(st), rows,
            _ptr(q, g * H * d), G * H * d, _ptr(k, g * d), G * d, _ptr(v, g * dv), G * dv,
            _ptr(out, g * H * dv) if out is not None else None, G * H * dv,
            _ptr(slots) if slots is not None else None)
        if rc != 0:
            raise RuntimeError("oracle rejected its arguments")

    def step(self, q, k, v, want: Optional[np.ndarray] = None) -> np.ndarray:
        """Step the rows of q [rows][nh][d], k [rows][G][d], v [rows][G][dv].

        Returns the attention output of every row as float64 [rows][nh][dv],
        or, when ``want`` (bool [rows]) is given, of the wanted rows only, in
        row order.  The state advances over every row either way.
        """
        q = np.ascontiguousarray(q, np.float32)
        k = np.ascontiguousarray(k, np.float32)
        v = np.ascontiguousarray(v, np.float32)
        rows = q.shape[0]
        assert q.shape == (rows, self.G * self.H, self.d)
        assert k.shape == (rows, self.G, self.d) and v.shape == (rows, self.G, self.dv)
        if want is None:
            slots = None
            n_out = rows
        else:
            want = np.asarray(want, bool)
            slots = np.full(rows, -1, np.int64)
            idx = np.nonzero(want)[0]
            slots[idx] = np.arange(idx.size)
            n_out = idx.size
        out = np.zeros((n_out, self.G * self.H, self.dv), np.float64)
        if len(self.parts) == 1 or self.threads <= 1:
            for p in self.parts:
                self._run_part(p, q, k, v, out, slots)
        else:
            with ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(lambda p: self._run_part(p, q, k, v, out, slots), self.parts))
        return out

    # -- state in the GPU library's layouts ---------------------------------
    def rewind(self) -> None:
        """Undo the bookkeeping of the last push of every group, as the
        pages' ``dory_o1_back`` (cortiq-engine 0.8.77 src/gpu_wgpu/dory.rs)
        does: after a push that evicted, the head steps back one slot and
        the far count drops by one; after any other push the window loses
        its newest row.  Ring rows and M, Z, Theta stay as they are.

        Readings where the page is silent: the page takes a full window to
        mean that the last push evicted, which is not so for the push that
        filled the window (it evicted nothing, and the far count is still
        0); a full window with a far count of 0 is therefore undone as a
        plain push.  An empty window (the page does not guard it) is left
        alone."""
        for p in self.parts:
            wg = self.windows[p["g"]]
            ln, hd, nf = (int(x) for x in p["meta"])
            if ln == wg and nf > 0:
                p["meta"][1] = (hd + wg - 1) % wg
                p["meta"][2] = nf - 1
            elif ln > 0:
                p["meta"][0] = ln - 1

    def meta(self) -> np.ndarray:
        out = np.zeros((self.G, 4), np.uint32)
        for p in self.parts:
            if p["h_lo"] == 0:
                out[p["g"], :3] = p["meta"]
        for g in range(self.G):
            out[g, 3] = 0 if self.windows[g] == self.W else self.windows[g]
        return out

    def ring(self):
        rk = np.zeros((self.G, self.W, self.d))
        rv = np.zeros((self.G, self.W, self.dv))
        for p in self.parts:
            if p["h_lo"] == 0:
                rk[p["g"]] = p["ring_k"]
                rv[p["g"]] = p["ring_v"]
        return rk, rv

    def mz(self) -> np.ndarray:
        return np.stack([self.M, self.Z], axis=1)


def from_config(cfg, state, threads: Optional[int] = None) -> SerialOracle:
    """A :class:`SerialOracle` for a :class:`synth.Config` and its state."""
    return SerialOracle(cfg.G, cfg.H, cfg.m, cfg.W, cfg.ns, cfg.d, cfg.dv, cfg.scale,
                        cfg.rect, state, threads=threads)
