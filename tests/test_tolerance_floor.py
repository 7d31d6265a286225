"""What an fp32 far accumulator can reach: the reading of the Theta tolerance.

The far accumulator Theta_b of a landmark sums exp(l_j - M_b) v_j over every
key the window has evicted (cortiq-engine 0.8.51 src/gpu_wgpu/o1_batch.rs,
o1b_far_commit; 0.8.82 src/gpu_metal/o1c.rs, the token commit): at the
decode workload, about 35 000 signed terms of magnitude ~1 per element.  An
element is a random walk; it can end near 0 while its partial sums were of
order 100.  The layer's state keeps Theta in fp32 and rewrites it after every
sub-chunk and every token, as the pages' kernels do.

These tests measure, on one query head of the decode workload (the
max-window layer: a 32768-row prompt as 64-row sub-chunks, then 4096 single
rows), what two fp32 evaluations of the recurrence reach against the exact
float64 sum:

* exact arithmetic, with Theta only *stored* in fp32 after each sub-chunk
  and each row (the pages' state);
* fp32 arithmetic for each sub-chunk's increment (the exponentials, the
  products and the 64-term sum), summed exactly across sub-chunks (the best
  any compensated accumulation of fp32 increments can do).

Both exceed the elementwise bound 1e-5 + 1e-4 |Theta| on elements that
cancel toward 0, and both stay far inside 1e-5 + 1e-4 max_t |Theta_b[t]|,
the bound taken against the landmark's accumulator scale.  That is why the
GPU tests read the tolerance of Theta against that scale (and print the
elementwise figures beside it).  Plain numpy; no GPU and no oracle code.
"""
import numpy as np
import pytest

import synth

ATOL, RTOL = 1e-5, 1e-4


def _bounds(got, want):
    """(elementwise excess, elements over it, accumulator-scale excess, max|d|)."""
    d = np.abs(got - want)
    over = d - (ATOL + RTOL * np.abs(want))
    scale = np.max(np.abs(want), axis=1, keepdims=True)
    acc = d - (ATOL + RTOL * scale)
    return float(over.max()), int(np.sum(over > 0)), float(acc.max()), float(d.max()), float(scale.max())


@pytest.fixture(scope="module")
def stream():
    """Evicted keys' landmark scores and values of query head 0 (group 0)."""
    cfg = synth.DECODE
    host = synth.make_state(cfg)
    n = cfg.rows + cfg.decode_steps
    _, k, v = synth.rows(cfg, 0, n)
    w = cfg.window(0)
    nev = n - w                     # row r >= w evicts the key of row r - w
    K = k[:nev, 0].astype(np.float64)
    V = v[:nev, 0].astype(np.float64)
    qt = host.q_tilde[0].astype(np.float64)        # [m][d]
    L = cfg.scale * (K @ qt.T)                      # [nev][m]
    return cfg, w, L, V


def _exact(L, V, n):
    l = L[:n]
    M = l.max(axis=0)
    return np.exp(l - M).T @ V[:n]                  # [m][dv]


def test_fp32_state_exceeds_elementwise_bound(stream):
    cfg, w, L, V = stream
    m = cfg.m
    npre = cfg.rows - w
    M = np.full(m, -np.inf)
    th = np.zeros((m, cfg.dv))
    for s in range(cfg.rows // 64):
        lo, hi = max(64 * s - w, 0), 64 * s + 64 - w
        if hi <= 0:
            continue
        l = L[lo:hi]
        Mn = np.maximum(M, l.max(axis=0))
        R = np.where(Mn == M, 1.0, np.exp(M - Mn))
        th = (R[:, None] * th + np.exp(l - Mn).T @ V[lo:hi]).astype(np.float32).astype(np.float64)
        M = Mn
    pre = _bounds(th, _exact(L, V, npre))
    for t in range(npre, L.shape[0]):
        Mn = np.maximum(M, L[t])
        R = np.where(Mn == M, 1.0, np.exp(M - Mn))
        th = (R[:, None] * th + np.exp(L[t] - Mn)[:, None] * V[t][None, :]).astype(np.float32)
        th = th.astype(np.float64)
        M = Mn
    dec = _bounds(th, _exact(L, V, L.shape[0]))
    for name, (el, nb, acc, md, sc) in (("prompt end", pre), ("after 4096 rows", dec)):
        print(f"  fp32 state, exact arithmetic, {name}: max|d| {md:.3e}, elementwise excess "
              f"{el:.3e} ({nb} of {th.size} over), accumulator-scale excess {acc:.3e} "
              f"(scale {sc:.1f})")
    el, nb, acc, md, sc = dec
    assert el > 0 and nb > 0, "the fp32 state met the elementwise bound"
    assert md < 0.1 * RTOL * sc, "the fp32 state used more than a tenth of the scaled bound"
    assert pre[2] < 0 and acc < 0


def test_fp32_increments_exceed_elementwise_bound(stream):
    cfg, w, L, V = stream
    m = cfg.m
    M = np.full(m, -np.inf)
    th = np.zeros((m, cfg.dv))
    for s in range(cfg.rows // 64):
        lo, hi = max(64 * s - w, 0), 64 * s + 64 - w
        if hi <= 0:
            continue
        l = L[lo:hi]
        Mn = np.maximum(M, l.max(axis=0))
        R = np.where(Mn == M, 1.0, np.exp(M - Mn))
        E32 = np.exp((l - Mn).astype(np.float32))
        d32 = (E32.T @ V[lo:hi].astype(np.float32)).astype(np.float64)
        th = R[:, None] * th + d32
        M = Mn
    el, nb, acc, md, sc = _bounds(th, _exact(L, V, cfg.rows - w))
    print(f"  fp32 increments, exact accumulation, prompt end: max|d| {md:.3e}, elementwise "
          f"excess {el:.3e} ({nb} of {th.size} over), accumulator-scale excess {acc:.3e} "
          f"(scale {sc:.1f})")
    assert el > 0 and nb > 0, "fp32 increments met the elementwise bound"
    assert acc < 0 and md < 0.1 * RTOL * sc
