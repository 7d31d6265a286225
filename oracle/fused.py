"""float64 restatement of the ingest and output steps around the chunk path
(TEST INFRASTRUCTURE ONLY: only the tests, the smoke check and the
benchmark's CPU-baseline leg use it; it shares nothing with the GPU library).

Written from the per-row kernels of cortiq-engine 0.8.77
``src/gpu_wgpu/dory.rs``: the preparation kernel (``dory_prep``) turns each
query and key head by the rotate-half RoPE of the row's table before the
key enters the ring, and the output kernels (``dory_gate1``,
``dory_ogate``) multiply the normalised attention output by a sigmoid gate.

* RoPE: the table row of a chunk row holds cos of the d/2 pair angles, then
  their sin (the page's harness fills it in float64 and stores float32).
  Pair (j, j + d/2) of a head vector x becomes
  (x_j c_j - x_{j+d/2} s_j, x_{j+d/2} c_j + x_j s_j).  Values are not
  rotated.  (The page's kernel also normalises each head to unit length and
  scales the queries; that is the model's choice and stays outside.)
* Gate: out[r, h, t] times 1 / (1 + exp(-z[r, h, t] s[h, t])), z the row's
  gate pre-activation and s a per-(head, column) scale.

``step_fused`` composes them with the serial oracle: rotate q and k, step,
gate the output.
"""
from __future__ import annotations

from typing import Optional

import numpy as np


def rope_rows(x: np.ndarray, table: np.ndarray) -> np.ndarray:
    """Rotate-half RoPE of x [rows][heads][d] by table [rows][d], in float64."""
    x = np.asarray(x, np.float64)
    t = np.asarray(table, np.float64)
    rows, heads, d = x.shape
    assert t.shape == (rows, d) and d % 2 == 0
    h = d // 2
    out = np.empty_like(x)
    for r in range(rows):
        c, s = t[r, :h], t[r, h:]
        for a in range(heads):
            lo, hi = x[r, a, :h], x[r, a, h:]
            out[r, a, :h] = lo * c - hi * s
            out[r, a, h:] = hi * c + lo * s
    return out


def sigmoid(x: np.ndarray) -> np.ndarray:
    """1 / (1 + exp(-x)) in float64, written so that neither branch overflows."""
    x = np.asarray(x, np.float64)
    e = np.exp(-np.abs(x))
    return np.where(x >= 0, 1.0 / (1.0 + e), e / (1.0 + e))


def gate_rows(out: np.ndarray, z: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """out [rows][nh][dv] times sigmoid(z [rows][nh][dv] * scale [nh][dv])."""
    out = np.asarray(out, np.float64)
    z = np.asarray(z, np.float64)
    scale = np.asarray(scale, np.float64)
    assert z.shape == out.shape and scale.shape == out.shape[1:]
    return out * sigmoid(z * scale[None])


def step_fused(orc, q, k, v, rope: Optional[np.ndarray] = None, gate: Optional[np.ndarray] = None,
               gate_scale: Optional[np.ndarray] = None) -> np.ndarray:
    """One call of the fused path on the serial oracle ``orc``: q and k of
    the rows rotated by ``rope`` (when given, else taken as they are), the
    oracle stepped over the rows, the output gated (when ``gate`` is given).
    The rotated q and k enter the oracle as float32, the type the layer's
    ring stores."""
    if rope is not None:
        q = rope_rows(q, rope).astype(np.float32)
        k = rope_rows(k, rope).astype(np.float32)
    out = orc.step(q, k, v)
    if gate is not None:
        out = gate_rows(out, gate, gate_scale)
    return out
