"""float64 restatement of the sub-chunk algorithm (TEST INFRASTRUCTURE ONLY).

Written from the chunk kernels of cortiq-engine 0.8.51
``src/gpu_wgpu/o1_batch.rs`` (o1b_far_e, o1b_attend, o1b_far_commit,
o1b_ring_commit, o1b_meta): a chunk of k rows is processed at once.

* far_e: row j of the chunk evicts once the ring is full (j >= j0 = w_g -
  len0); the evicted key is logical index x = j - j0 of (ring ++ chunk).
  The far max jumps to its post-chunk value M', R = 1 if M' equals the old
  M else exp(M - M'), E_j = exp(l_j - M'), and P_j = R Z + sum_{j'<=j} E_j'.
* attend: row i's window is the last min(w_g, len0+i+1) keys of ring ++
  chunk (self included) plus the sinks; the far part is read against M':
  D_far = sum_b gain_b P_bi and N_far = sum_b gain_b R_b Theta_b +
  sum_{j0<=j<=i} cf_j v_evicted(j), with cf_j = sum_b gain_b E_bj.
* commit: Theta <- R Theta + sum_j E_j v_evicted(j), M <- M', Z <- P_{k-1};
  the chunk rows enter the ring at slot (head0 + len0 + j) mod w_g (in row
  order, so the surviving rows are the last ones written); len/head/nfar
  follow the closed form after k pushes.

The pages require w_g >= 64 so that every evicted key is still in the ring
at the chunk's start; the (ring ++ chunk) source above lifts that limit with
the same arithmetic.  Used only to pin the serial oracle and to inspect
intermediate far-field values; it shares nothing with the GPU library.
"""
from __future__ import annotations

import numpy as np


class ChunkedOracle:
    def __init__(self, G, H, m, W, ns, d, dv, scale, rect, state):
        self.G, self.H, self.m, self.W, self.ns, self.d, self.dv = G, H, m, W, ns, d, dv
        self.scale, self.rect = float(scale), bool(rect)
        nh = G * H
        self.meta = np.asarray(state.meta, np.int64).reshape(G, 4).copy()
        self.ring_k = np.asarray(state.ring_k, np.float64).reshape(G, W, d).copy()
        self.ring_v = np.asarray(state.ring_v, np.float64).reshape(G, W, dv).copy()
        self.sink_k = np.asarray(state.sink_k, np.float64).reshape(G, ns, d)
        self.sink_v = np.asarray(state.sink_v, np.float64).reshape(G, ns, dv)
        self.k_tilde = np.asarray(state.k_tilde, np.float64).reshape(G, m, d)
        self.q_tilde = np.asarray(state.q_tilde, np.float64).reshape(nh, m, d)
        self.mu = np.asarray(state.mu, np.float64).reshape(nh, m, m)
        mz = np.asarray(state.mz, np.float64).reshape(nh, 2, m)
        self.M = mz[:, 0, :].copy()
        self.Z = mz[:, 1, :].copy()
        self.theta = np.asarray(state.theta, np.float64).reshape(nh, m, dv).copy()
        self.last = None  # intermediates of the last sub-chunk

    def _wg(self, g):
        w = int(self.meta[g, 3])
        return w if w else self.W

    def _key(self, g, x, len0, head0, wg, kc, vc):
        """Key and value of logical index x of ring ++ chunk."""
        if x < len0:
            s = (head0 + x) % wg
            return self.ring_k[g, s], self.ring_v[g, s]
        return kc[x - len0, g].astype(np.float64), vc[x - len0, g].astype(np.float64)

    def sub_chunk(self, q, k, v, commit=True):
        """One sub-chunk of k rows (any k >= 1). Returns out [k][nh][dv]."""
        G, H, m, ns, d, dv = self.G, self.H, self.m, self.ns, self.d, self.dv
        kk = q.shape[0]
        nh = G * H
        s = self.scale
        out = np.zeros((kk, nh, dv))
        inter = dict(E=np.zeros((nh, m, kk)), P=np.zeros((nh, m, kk)),
                     Mn=np.zeros((nh, m)), R=np.zeros((nh, m)))
        new_theta = self.theta.copy()
        for g in range(G):
            len0, head0, nfar0 = (int(x) for x in self.meta[g, :3])
            wg = self._wg(g)
            j0 = wg - len0
            ev = [self._key(g, j - j0, len0, head0, wg, k, v) if j >= j0 else None
                  for j in range(kk)]
            for h in range(H):
                gh = g * H + h
                # far_e
                l = np.full((m, kk), -np.inf)
                for j in range(kk):
                    if ev[j] is not None:
                        l[:, j] = s * (self.q_tilde[gh] @ ev[j][0])
                m_old = self.M[gh]
                mx = np.maximum(m_old, l.max(axis=1))
                with np.errstate(invalid="ignore"):   # -inf - -inf in the branch not taken
                    R = np.where(mx == m_old, 1.0, np.exp(m_old - mx))
                    E = np.where(np.isfinite(l), np.exp(l - mx[:, None]), 0.0)
                P = R[:, None] * self.Z[gh][:, None] + np.cumsum(E, axis=1)
                inter["E"][gh], inter["P"][gh], inter["Mn"][gh], inter["R"][gh] = E, P, mx, R
                # attend
                for i in range(kk):
                    qi = q[i, gh].astype(np.float64)
                    win = min(wg, len0 + i + 1)
                    lo = len0 + i + 1 - win
                    keys = [self.sink_k[g, x] for x in range(ns)]
                    vals = [self.sink_v[g, x] for x in range(ns)]
                    for x in range(lo, len0 + i + 1):
                        kx, vx = self._key(g, x, len0, head0, wg, k, v)
                        keys.append(kx)
                        vals.append(vx)
                    keys = np.array(keys).reshape(-1, d)
                    vals = np.array(vals).reshape(-1, dv)
                    sc = s * (keys @ qi)
                    c = sc.max()
                    farl = nfar0 + (i - j0 + 1 if i >= j0 else 0)
                    have = False
                    d_far = 0.0
                    n_far = np.zeros(dv)
                    if farl > 0:
                        f = s * (self.k_tilde[g] @ qi)
                        fmax = f.max()
                        u = np.exp(f - fmax) @ self.mu[gh]
                        if self.rect:
                            u = np.maximum(u, 0.0)
                        c = max(c, float((fmax + mx).max()))
                        gain = u * np.exp(fmax + mx - c)
                        d_far = float(gain @ P[:, i])
                        if d_far >= 0.0:
                            have = True
                            n_far = (gain * R) @ self.theta[gh]
                            for j in range(max(j0, 0), i + 1):
                                cf = float(gain @ E[:, j])
                                n_far = n_far + cf * ev[j][1]
                        else:
                            d_far = 0.0
                    p = np.exp(sc - c)
                    num = (n_far if have else 0.0) + p @ vals
                    den = max((d_far if have else 0.0) + p.sum(), 1e-30)
                    out[i, gh] = num / den
                # far_commit (after attend has read the old Theta)
                if j0 < kk:
                    acc = R[:, None] * self.theta[gh]
                    for j in range(max(j0, 0), kk):
                        acc = acc + E[:, j][:, None] * ev[j][1][None, :]
                    new_theta[gh] = acc
                    if commit:
                        self.M[gh] = mx
                        self.Z[gh] = P[:, kk - 1]
        self.last = inter
        if commit:
            self.theta = new_theta
            for g in range(G):
                len0, head0, nfar0 = (int(x) for x in self.meta[g, :3])
                wg = self._wg(g)
                for j in range(kk):
                    slot = (head0 + len0 + j) % wg
                    self.ring_k[g, slot] = k[j, g]
                    self.ring_v[g, slot] = v[j, g]
                tot = len0 + kk
                if tot <= wg:
                    self.meta[g, 0] = tot
                else:
                    e = tot - wg
                    self.meta[g, 0] = wg
                    self.meta[g, 1] = (head0 + e) % wg
                    self.meta[g, 2] = nfar0 + e
        return out

    def run(self, q, k, v, sub=64):
        """Rows in consecutive sub-chunks of ``sub`` rows, each committed."""
        outs = []
        for r0 in range(0, q.shape[0], sub):
            r1 = min(q.shape[0], r0 + sub)
            outs.append(self.sub_chunk(q[r0:r1], k[r0:r1], v[r0:r1], commit=True))
        return np.concatenate(outs) if outs else np.zeros((0, self.G * self.H, self.dv))


def from_config(cfg, state) -> ChunkedOracle:
    return ChunkedOracle(cfg.G, cfg.H, cfg.m, cfg.W, cfg.ns, cfg.d, cfg.dv, cfg.scale,
                         cfg.rect, state)
