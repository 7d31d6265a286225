"""Helpers of the GPU parity tests: device copies, state readback and the
tolerance check.  The GPU path is always reached through the C ABI
(sink_window_landmark_amd); expected values always come from the CPU oracle.

Tolerance (float32 path against the float64 oracle): |got - want| <=
ATOL + RTOL * |want| elementwise for outputs, M and Z; for Theta the
relative part is taken against the landmark's accumulator scale
(max_t |Theta_b[t]|), since Theta_b is a sum of thousands of signed terms
whose float32 rounding is set by that scale, not by each element.  Ring
contents and meta are compared bit for bit.
"""
from __future__ import annotations

import os
import sys

import numpy as np

ATOL = 1e-5
RTOL = 1e-4


def torch():
    import torch as t
    return t


def dev(a):
    t = torch()
    return t.from_numpy(np.ascontiguousarray(a)).to("cuda")


def geom_of(cfg):
    import sink_window_landmark_amd as swl
    return swl.Geom(cfg.G, cfg.H, cfg.m, cfg.W, cfg.ns, cfg.d, cfg.dv, rect=cfg.rect)


def read_state(st):
    t = torch()
    t.cuda.synchronize()
    return dict(meta=st.meta.cpu().numpy().view(np.uint32),
                ring_k=st.ring_k.cpu().numpy(), ring_v=st.ring_v.cpu().numpy(),
                mz=st.mz.cpu().numpy(), theta=st.theta.cpu().numpy())


def excess(got, want, atol=ATOL, rtol=RTOL, scale=None):
    """max over elements of |got - want| - (atol + rtol * scale)."""
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    ref = np.abs(want) if scale is None else scale
    both_inf = np.isinf(got) & np.isinf(want) & (np.sign(got) == np.sign(want))
    with np.errstate(invalid="ignore"):   # inf - inf where both are -inf (masked below)
        d = np.where(both_inf, 0.0, np.abs(got - want))
    return float(np.max(d - (atol + rtol * ref))) if d.size else -1.0


def check_out(got, want, what="out", atol=ATOL):
    """Elementwise |got - want| <= atol + RTOL |want| (atol scales with the
    values' scale when a test scales the values: the output is linear in
    them)."""
    got = np.asarray(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    e = excess(got, want, atol=atol)
    md = float(np.max(np.abs(got.astype(np.float64) - want))) if got.size else 0.0
    print(f"  {what}: max|d| {md:.3e}  excess {e:.3e}", flush=True)
    if e > 0:
        w = np.asarray(want, np.float64)
        at = np.unravel_index(np.argmax(np.abs(got - w) - (atol + RTOL * np.abs(w))), w.shape)
        raise AssertionError(f"{what}: beyond tolerance by {e:.3e} (max|d| {md:.3e}); worst at "
                             f"{tuple(int(i) for i in at)}: got {float(got[at]):.8g}, "
                             f"want {float(w[at]):.8g}, max|want| {float(np.max(np.abs(w))):.4g}")


def check_state(gpu, orc, ring=True, vscale=1.0):
    """GPU state (read_state) against a SerialOracle's state.  vscale: the
    values' scale, by which Theta's absolute bound scales."""
    np.testing.assert_array_equal(gpu["meta"][:, :3], orc.meta()[:, :3])
    if ring:
        rk, rv = orc.ring()
        for g in range(orc.G):
            meta = orc.meta()[g]
            ln, hd = int(meta[0]), int(meta[1])
            wg = orc.windows[g]
            slots = [(hd + x) % wg for x in range(ln)]
            np.testing.assert_array_equal(gpu["ring_k"][g, slots], rk[g, slots].astype(np.float32))
            np.testing.assert_array_equal(gpu["ring_v"][g, slots], rv[g, slots].astype(np.float32))
    M, Z = gpu["mz"][:, 0, :], gpu["mz"][:, 1, :]
    eM = excess(M, orc.M)
    eZ = excess(Z, orc.Z)
    sc = np.max(np.abs(orc.theta), axis=2, keepdims=True)
    eT = excess(gpu["theta"], orc.theta, atol=ATOL * vscale, scale=sc)
    th = np.asarray(gpu["theta"], np.float64)
    dT = np.abs(th - orc.theta)
    mt = float(np.max(dT)) if dT.size else 0.0
    # elementwise reading, reported beside the accumulator-scale one: the
    # excess, how many elements exceed, and how far the worst one has
    # cancelled (|Theta| of that element against its landmark's largest)
    lim = ATOL * vscale + RTOL * np.abs(orc.theta)
    over = dT - lim
    eTe = float(np.max(over)) if over.size else -1.0
    nbad = int(np.sum(over > 0))
    if over.size:
        at = np.unravel_index(np.argmax(over), over.shape)
        canc = float(abs(orc.theta[at]) / max(float(sc[at[0], at[1], 0]), 1e-300))
    else:
        canc = 1.0
    print(f"  state: M excess {eM:.3e}  Z excess {eZ:.3e}  Theta max|d| {mt:.3e} "
          f"excess {eT:.3e} (accumulator scale)  elementwise excess {eTe:.3e} "
          f"({nbad} of {over.size} over; worst |Theta|/scale {canc:.2e})", flush=True)
    assert eM <= 0 and eZ <= 0 and eT <= 0


def oracle_threads():
    return max(1, min(16, os.cpu_count() or 1))


def banner(msg):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()
