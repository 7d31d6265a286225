"""Seeded synthetic inputs for the sink + window + landmark attention layer.

This module only *draws* inputs: states, prompt rows and decode rows, in the
layouts the layer uses at its boundary. It holds none of the method's
arithmetic (no scores, no softmax, no far-field update), so that the CPU
oracle and the GPU path can both be fed from it without sharing any code
that computes a result.

Layouts (row-major, fp32 unless noted):

* q            [rows][G*H][d]    rotated queries, head gh = g*H + h
* k, v         [rows][G][d|dv]   rotated keys and values
* sink_k/v     [G][ns][d|dv]
* ring_k/v     [G][W][d|dv]      W is the ring stride (widest window)
* k_tilde      [G][m][d]         landmark keys
* q_tilde      [G*H][m][d]       landmark queries
* mu           [G*H][m][m]       landmark weights
* meta         u32 [G][4]        (len, head, nfar, window override)

Random draws follow ``numpy.random.default_rng([seed, stream, block])``:
stream 0 is the state, stream 1 the prompt rows, drawn per 64-row block so
any block can be regenerated without the rows before it. Values are drawn
in float64 and cast to float32 once, after any rotation.

RoPE (rotate-half pairs (x_j, x_{j+d/2}), angle pos * 10000**(-2j/d),
computed in float64) is an input-preparation step: the layer receives the
rotated rows, as the pages' chunk kernels do.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np

BLOCK = 64  # rows per generator block (also the layer's sub-chunk height)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    G: int
    H: int
    d: int
    dv: int
    ns: int
    W: int
    m: int
    rows: int
    windows: Optional[Sequence[int]] = None  # per-group window override (None: W)
    len0: int = 0          # initial ring length per group
    head0: int = 0         # initial ring head per group
    rope: bool = False
    landmark_scale: float = 1.0   # K~ and Q~ are N(0,1) * landmark_scale
    spike97: bool = False  # key of prompt row r scaled x4 when (r+1) % 97 == 0
    decode_steps: int = 0
    rect: bool = False
    seed: int = 0

    @property
    def nh(self) -> int:
        return self.G * self.H

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def window(self, g: int) -> int:
        if self.windows is None:
            return self.W
        return int(self.windows[g])

    def meta_windows(self) -> List[int]:
        """Meta slot 3 values (0 = the layer's W)."""
        if self.windows is None:
            return [0] * self.G
        return [int(w) for w in self.windows]

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


# The five workloads the layer is measured and checked on.
TINY = Config("tiny", G=1, H=2, d=32, dv=32, ns=4, W=16, m=8, rows=64,
              len0=10, head0=0, rope=False, landmark_scale=1.0)
SMALL = Config("small", G=2, H=4, d=128, dv=128, ns=4, W=1024, m=32, rows=4096,
               rope=True, landmark_scale=1.0 / math.sqrt(128))
MAXWIN = Config("maxwin", G=4, H=4, d=128, dv=128, ns=4, W=2048, m=64, rows=32768,
                rope=True, landmark_scale=1.0 / math.sqrt(128))
DECODE = MAXWIN.replace(name="decode", decode_steps=4096)
MIXED = Config("mixed", G=4, H=4, d=128, dv=128, ns=4, W=2048, m=64, rows=131072,
               windows=(512, 1024, 2048, 2048), rope=True,
               landmark_scale=1.0 / math.sqrt(128), spike97=True)

CONFIGS = {c.name: c for c in (TINY, SMALL, MAXWIN, DECODE, MIXED)}


def _rng(cfg: Config, stream: int, block: int) -> np.random.Generator:
    return np.random.default_rng([cfg.seed, stream, block])


def rope_rotate(x: np.ndarray, pos: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE of ``x[..., rows-axis, ..., d]`` in float64.

    ``x`` has shape [rows, heads, d]; ``pos`` has shape [rows].
    """
    d = x.shape[-1]
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    inv = 10000.0 ** (-2.0 * j / d)
    ang = pos.astype(np.float64)[:, None] * inv[None, :]          # [rows][half]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def rope_table(pos: np.ndarray, d: int) -> np.ndarray:
    """RoPE table rows [rows][d] as float32: cos of the d/2 pair angles
    pos * 10000^(-2j/d), then their sin, computed in float64."""
    half = d // 2
    j = np.arange(half, dtype=np.float64)
    ang = np.asarray(pos, np.float64)[:, None] * (10000.0 ** (-2.0 * j / d))[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1).astype(np.float32)


def gate_inputs(cfg: Config, start: int, count: int):
    """Gate pre-activations z [count][nh][dv] (N(0, 1)) and the per-(head,
    column) scale [nh][dv] (uniform in [0.5, 2]) as float32."""
    r = _rng(cfg, 7, start)
    z = r.standard_normal((count, cfg.nh, cfg.dv)).astype(np.float32)
    s = np.random.default_rng([cfg.seed, 8]).uniform(0.5, 2.0, (cfg.nh, cfg.dv)).astype(np.float32)
    return z, s


@dataclasses.dataclass
class State:
    """Host copy of a layer state (fp32 arrays, u32 meta)."""
    meta: np.ndarray
    ring_k: np.ndarray
    ring_v: np.ndarray
    sink_k: np.ndarray
    sink_v: np.ndarray
    k_tilde: np.ndarray
    q_tilde: np.ndarray
    mu: np.ndarray
    mz: np.ndarray
    theta: np.ndarray

    def copy(self) -> "State":
        return State(**{f.name: getattr(self, f.name).copy()
                        for f in dataclasses.fields(self)})


def make_state(cfg: Config, mu: Optional[np.ndarray] = None) -> State:
    """The initial state: sinks, landmarks, mu, an optional pre-filled ring
    (``cfg.len0`` rows at slots (head0 + x) mod w_g) and an empty far field
    (M = -inf, Z = 0, Theta = 0, nfar = 0)."""
    G, H, d, dv, ns, W, m = cfg.G, cfg.H, cfg.d, cfg.dv, cfg.ns, cfg.W, cfg.m
    nh = G * H
    r = _rng(cfg, 0, 0)
    sink_k = r.standard_normal((G, ns, d))
    sink_v = r.standard_normal((G, ns, dv))
    k_tilde = r.standard_normal((G, m, d)) * cfg.landmark_scale
    q_tilde = r.standard_normal((nh, m, d)) * cfg.landmark_scale
    mu_d = np.abs(r.standard_normal((nh, m, m))) / m
    ring_rows_k = r.standard_normal((G, max(cfg.len0, 0), d))
    ring_rows_v = r.standard_normal((G, max(cfg.len0, 0), dv))
    if cfg.rope:
        pos = np.arange(ns)
        sink_k = np.stack([rope_rotate(sink_k[g][:, None, :], pos)[:, 0, :]
                           for g in range(G)])
        if cfg.len0:
            rp = ns + np.arange(cfg.len0)
            ring_rows_k = np.stack([rope_rotate(ring_rows_k[g][:, None, :], rp)[:, 0, :]
                                    for g in range(G)])
    ring_k = np.zeros((G, W, d), np.float32)
    ring_v = np.zeros((G, W, dv), np.float32)
    meta = np.zeros((G, 4), np.uint32)
    for g in range(G):
        wg = cfg.window(g)
        if cfg.len0 > wg:
            raise ValueError("initial ring longer than its window")
        for x in range(cfg.len0):
            slot = (cfg.head0 + x) % wg
            ring_k[g, slot] = ring_rows_k[g, x]
            ring_v[g, slot] = ring_rows_v[g, x]
        meta[g] = (cfg.len0, cfg.head0 % wg, 0, cfg.meta_windows()[g])
    mz = np.zeros((nh, 2, m), np.float32)
    mz[:, 0, :] = -np.inf
    theta = np.zeros((nh, m, dv), np.float32)
    return State(meta=meta,
                 ring_k=ring_k, ring_v=ring_v,
                 sink_k=sink_k.astype(np.float32), sink_v=sink_v.astype(np.float32),
                 k_tilde=k_tilde.astype(np.float32), q_tilde=q_tilde.astype(np.float32),
                 mu=(mu_d if mu is None else mu).astype(np.float32),
                 mz=mz, theta=theta)


def _block(cfg: Config, b: int):
    G, nh, d, dv = cfg.G, cfg.nh, cfg.d, cfg.dv
    r = _rng(cfg, 1, b)
    q = r.standard_normal((BLOCK, nh, d))
    k = r.standard_normal((BLOCK, G, d))
    v = r.standard_normal((BLOCK, G, dv))
    rows = b * BLOCK + np.arange(BLOCK)
    if cfg.rope:
        pos = cfg.ns + cfg.len0 + rows
        q = rope_rotate(q, pos)
        k = rope_rotate(k, pos)
    q = q.astype(np.float32)
    k = k.astype(np.float32)
    v = v.astype(np.float32)
    if cfg.spike97:
        sel = (rows + 1) % 97 == 0
        k[sel] *= np.float32(4.0)
    return q, k, v


def rows(cfg: Config, r0: int, r1: int):
    """Prompt (or decode) rows [r0, r1) as (q, k, v), fp32, contiguous.

    Decode rows continue the prompt stream: decode step t is row
    ``cfg.rows + t``.
    """
    if r1 <= r0:
        z = np.zeros
        return (z((0, cfg.nh, cfg.d), np.float32), z((0, cfg.G, cfg.d), np.float32),
                z((0, cfg.G, cfg.dv), np.float32))
    b0, b1 = r0 // BLOCK, (r1 - 1) // BLOCK
    parts = [_block(cfg, b) for b in range(b0, b1 + 1)]
    q = np.concatenate([p[0] for p in parts])
    k = np.concatenate([p[1] for p in parts])
    v = np.concatenate([p[2] for p in parts])
    lo = r0 - b0 * BLOCK
    hi = lo + (r1 - r0)
    return (np.ascontiguousarray(q[lo:hi]), np.ascontiguousarray(k[lo:hi]),
            np.ascontiguousarray(v[lo:hi]))


def jit(a: np.ndarray, b: int) -> np.ndarray:
    """The pages' deterministic test values: ((37a + 13b + 3) mod 83)/83 - 0.5
    (o1_batch.rs, test ``o1_batch_matches_serial_steps``)."""
    a = np.asarray(a, dtype=np.int64)
    return (((a * 37 + b * 13 + 3) % 83) / 83.0 - 0.5).astype(np.float32)


def jit_rows(G: int, H: int, d: int, base: int, n: int):
    """q, k, v for ``n`` rows starting at stream row ``base`` in the pages'
    jit layout ([rows][nh][d], [rows][G][d]), offsets 5, 6, 7."""
    nh = G * H
    q = jit(np.arange(n * nh * d) + base * nh * d, 5).reshape(n, nh, d)
    k = jit(np.arange(n * G * d) + base * G * d, 6).reshape(n, G, d)
    v = jit(np.arange(n * G * d) + base * G * d, 7).reshape(n, G, d)
    return q, k, v
