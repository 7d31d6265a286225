"""Pins of the CPU oracle against what the pages and the mathematics fix.

Every check here compares the oracle with something computed another way:
textbook softmax attention, brute force over all evicted keys, closed
forms of the ring/meta recurrences, the Nystrom-exact special case, or the
chunked restatement of the method.  None calls the GPU library.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import chunked
import synth


def _cfg(**kw):
    base = dict(name="pin", G=2, H=2, d=16, dv=8, ns=2, W=16, m=4, rows=64)
    base.update(kw)
    return synth.Config(**base)


def _rand_rows(cfg, rows, seed=1):
    r = np.random.default_rng(seed)
    q = r.standard_normal((rows, cfg.nh, cfg.d)).astype(np.float32)
    k = r.standard_normal((rows, cfg.G, cfg.d)).astype(np.float32)
    v = r.standard_normal((rows, cfg.G, cfg.dv)).astype(np.float32)
    return q, k, v


def _key_stream(cfg, state, k, v, g):
    """Initial ring in logical order, then the prompt keys, as float64."""
    wg = cfg.window(g)
    len0, head0 = int(state.meta[g, 0]), int(state.meta[g, 1])
    rk = [state.ring_k[g, (head0 + x) % wg] for x in range(len0)]
    rv = [state.ring_v[g, (head0 + x) % wg] for x in range(len0)]
    K = np.concatenate([np.array(rk, np.float64).reshape(len0, cfg.d), k[:, g].astype(np.float64)])
    V = np.concatenate([np.array(rv, np.float64).reshape(len0, cfg.dv), v[:, g].astype(np.float64)])
    return K, V


def _softmax_attend(qrow, keys, vals, scale):
    s = scale * (keys @ qrow.astype(np.float64))
    p = np.exp(s - s.max())
    return (p @ vals) / p.sum()


def _window_reference(cfg, state, q, k, v, windows=None):
    """Textbook softmax over the sinks plus the last min(w_g, n) keys."""
    rows = q.shape[0]
    out = np.zeros((rows, cfg.nh, cfg.dv))
    for g in range(cfg.G):
        K, V = _key_stream(cfg, state, k, v, g)
        len0 = int(state.meta[g, 0])
        wg = cfg.window(g) if windows is None else windows[g]
        sk = state.sink_k[g].astype(np.float64)
        sv = state.sink_v[g].astype(np.float64)
        for r in range(rows):
            hi = len0 + r
            lo = max(0, hi - wg + 1)
            keys = np.concatenate([sk, K[lo:hi + 1]])
            vals = np.concatenate([sv, V[lo:hi + 1]])
            for h in range(cfg.H):
                gh = g * cfg.H + h
                out[r, gh] = _softmax_attend(q[r, gh], keys, vals, cfg.scale)
    return out


# -- near part and softmax ------------------------------------------------------

def test_no_eviction_equals_exact_causal_attention():
    """While no key has left the window the layer is exact causal softmax
    attention over the sinks plus every key so far (o1b_attend with
    nfar = 0: no far term enters)."""
    cfg = _cfg(W=64, rows=50, d=16, dv=12, ns=3)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows)
    orc = oracle.from_config(cfg, st)
    got = orc.step(q, k, v)
    want = _window_reference(cfg, st, q, k, v, windows=[10 ** 9] * cfg.G)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)
    assert (orc.meta()[:, 2] == 0).all()


def test_mu_zero_is_sliding_window_with_sinks():
    """mu = 0 gives u = 0, so the far part adds nothing: the output is exact
    softmax over the sinks and the last w_g keys.  Per-group windows (meta
    slot 3) and an initial ring whose head has wrapped pin the ring order,
    eviction and window masks."""
    cfg = _cfg(W=16, windows=(8, 16), rows=90, len0=5, head0=6, m=4)
    st = synth.make_state(cfg)
    st.mu[:] = 0.0
    q, k, v = _rand_rows(cfg, cfg.rows, seed=2)
    orc = oracle.from_config(cfg, st)
    got = orc.step(q, k, v)
    want = _window_reference(cfg, st, q, k, v)
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


# -- far readout ---------------------------------------------------------------

def _nystrom_exact_setup(H=2, d=8, w=8, m=8, ns=2, seed=3):
    """Landmark keys = the keys that will be evicted and mu = B^-1 with
    B[b][j] = exp(s q~_b . k~_j): the far estimate of every evicted key is
    then exactly its softmax weight (o1b_attend's far readout, written as
    sum_a sum_b exp(f_a) mu_ab exp(l_bj))."""
    cfg = synth.Config("nys", G=1, H=H, d=d, dv=d, ns=ns, W=w, m=m, rows=w + m)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=seed)
    r = np.random.default_rng(seed + 10)
    qt = (0.5 * r.standard_normal((H, m, d))).astype(np.float32)
    kt = k[:m, 0].astype(np.float64)          # the first m keys are the ones evicted
    mu = np.zeros((H, m, m))
    for h in range(H):
        B = np.exp(cfg.scale * (qt[h].astype(np.float64) @ kt.T))   # [b][j]
        mu[h] = np.linalg.inv(B)                                   # mu[a][b] with sum_b mu_ab B_bj = I
    st.k_tilde = kt[None].copy()
    st.q_tilde = qt
    st.mu = mu
    return cfg, st, q, k, v


def test_nystrom_exact_far_field_equals_full_causal_attention():
    cfg, st, q, k, v = _nystrom_exact_setup()
    orc = oracle.from_config(cfg, st)
    got = orc.step(q, k, v)
    want = _window_reference(cfg, st, q, k, v, windows=[10 ** 9])
    assert orc.meta()[0, 2] == cfg.m    # every landmark key was evicted
    np.testing.assert_allclose(got, want, rtol=1e-9, atol=1e-10)


def test_nystrom_exact_fails_when_a_term_is_dropped():
    """Sanity of the pin itself: the exact-attention target is far from the
    sliding-window one, so a far readout that dropped its terms could not
    pass the test above."""
    cfg, st, q, k, v = _nystrom_exact_setup()
    full = _window_reference(cfg, st, q, k, v, windows=[10 ** 9])
    window = _window_reference(cfg, st, q, k, v)
    assert np.abs(full[cfg.W:] - window[cfg.W:]).max() > 1e-2


# -- far summaries -------------------------------------------------------------

def test_far_state_matches_brute_force_over_all_evictions():
    """M_b = max_j l_bj, Z_b = sum_j exp(l_bj - M_b), Theta_b = sum_j
    exp(l_bj - M_b) v_j over every evicted key (o1b_far_e/o1b_far_commit
    summaries), independent of the order of evictions."""
    cfg = _cfg(W=16, windows=(8, 16), rows=120, len0=3, head0=2, m=5)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=4)
    orc = oracle.from_config(cfg, st)
    orc.step(q, k, v)
    for g in range(cfg.G):
        K, V = _key_stream(cfg, st, k, v, g)
        n_ev = int(st.meta[g, 0]) + cfg.rows - cfg.window(g)
        Ke, Ve = K[:n_ev], V[:n_ev]
        for h in range(cfg.H):
            gh = g * cfg.H + h
            l = cfg.scale * (st.q_tilde[gh].astype(np.float64) @ Ke.T)   # [m][n_ev]
            M = l.max(axis=1)
            e = np.exp(l - M[:, None])
            np.testing.assert_allclose(orc.M[gh], M, rtol=1e-13)
            np.testing.assert_allclose(orc.Z[gh], e.sum(axis=1), rtol=1e-12)
            np.testing.assert_allclose(orc.theta[gh], e @ Ve, rtol=1e-11, atol=1e-12)
        assert orc.meta()[g, 2] == n_ev


def test_empty_far_field_first_eviction():
    """An empty far field sits at M = -inf, Z = 0, Theta = 0 without NaN; the
    first eviction rescales that zero mass by exp(-inf) = 0 (o1b_far_e's
    R rule), leaving M_b = l_b, Z_b = 1 and Theta_b = v_e exactly."""
    cfg = _cfg(G=1, W=8, len0=8, head0=3, rows=1, m=6)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, 1, seed=5)
    orc = oracle.from_config(cfg, st)
    assert np.all(np.isneginf(orc.M)) and not np.any(orc.Z) and not np.any(orc.theta)
    out = orc.step(q, k, v)
    assert np.all(np.isfinite(out))
    ke = st.ring_k[0, 3].astype(np.float64)
    ve = st.ring_v[0, 3].astype(np.float64)
    for h in range(cfg.H):
        l = cfg.scale * (st.q_tilde[h].astype(np.float64) @ ke)
        np.testing.assert_allclose(orc.M[h], l, rtol=1e-14)  # summation order only
        np.testing.assert_array_equal(orc.Z[h], np.ones(cfg.m))
        np.testing.assert_array_equal(orc.theta[h], np.broadcast_to(ve, (cfg.m, cfg.dv)))


def test_outputs_finite_before_any_eviction_and_mass_at_least_one_after():
    cfg = _cfg(G=1, W=8, rows=20, m=6)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=6)
    orc = oracle.from_config(cfg, st)
    out = orc.step(q[:8], k[:8], v[:8])
    assert np.all(np.isfinite(out)) and np.all(np.isneginf(orc.M))
    orc.step(q[8:], k[8:], v[8:])
    # the argmax key of every landmark contributes exactly exp(0) = 1
    assert np.all(orc.Z >= 1.0)


# -- ring and meta ---------------------------------------------------------------

@pytest.mark.parametrize("wg,len0,head0,T", [
    (8, 0, 0, 3), (8, 0, 0, 8), (8, 0, 0, 9), (8, 5, 6, 2), (8, 5, 6, 70),
    (16, 10, 13, 64), (16, 16, 15, 1), (5, 5, 4, 131), (64, 0, 0, 200)])
def test_meta_and_ring_closed_form(wg, len0, head0, T):
    """After T pushes: len = min(w, len0+T), ev = max(0, len0+T-w),
    head = (head0+ev) mod w, nfar = ev, and the ring holds the last len keys
    in slot order (o1b_meta, o1b_ring_commit)."""
    cfg = _cfg(G=1, W=wg, len0=len0, head0=head0, rows=T, m=2)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, T, seed=7)
    orc = oracle.from_config(cfg, st)
    orc.step(q, k, v, want=np.zeros(T, bool))
    ev = max(0, len0 + T - wg)
    ln = min(wg, len0 + T)
    hd = (head0 + ev) % wg
    assert orc.meta()[0, :3].tolist() == [ln, hd, ev]
    K, V = _key_stream(cfg, st, k, v, 0)
    rk, rv = orc.ring()
    for x in range(ln):
        slot = (hd + x) % wg
        np.testing.assert_array_equal(rk[0, slot], K[len(K) - ln + x])
        np.testing.assert_array_equal(rv[0, slot], V[len(V) - ln + x])


@pytest.mark.parametrize("wg,len0,head0,T", [(8, 0, 0, 3), (8, 0, 0, 8), (8, 3, 5, 20), (5, 5, 4, 1)])
def test_rewind_undoes_the_last_push(wg, len0, head0, T):
    """A push followed by a rewind leaves len, head and nfar where they were
    (the rewind is the inverse of one push's bookkeeping), in a window that
    was partial or full before the push; repeated, it walks back through
    every earlier meta of a partial window."""
    cfg = _cfg(G=1, W=wg, len0=len0, head0=head0, rows=T + 1, m=2)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, T + 1, seed=9)
    orc = oracle.from_config(cfg, st)
    orc.step(q[:T], k[:T], v[:T], want=np.zeros(T, bool))
    before = orc.meta()[0, :3].tolist()
    orc.step(q[T:], k[T:], v[T:], want=np.zeros(1, bool))
    assert orc.meta()[0, :3].tolist() != before
    orc.rewind()
    assert orc.meta()[0, :3].tolist() == before
    # a partial window walks back to empty, then stays there
    cfg2 = _cfg(G=1, W=wg, rows=3, m=2)
    o2 = oracle.from_config(cfg2, synth.make_state(cfg2))
    q2, k2, v2 = _rand_rows(cfg2, 3, seed=10)
    seen = [o2.meta()[0, :3].tolist()]
    for r in range(3):
        o2.step(q2[r:r + 1], k2[r:r + 1], v2[r:r + 1], want=np.zeros(1, bool))
        seen.append(o2.meta()[0, :3].tolist())
    for r in range(3):
        o2.rewind()
        assert o2.meta()[0, :3].tolist() == seen[2 - r]
    o2.rewind()
    assert o2.meta()[0, :3].tolist() == [0, 0, 0]


@pytest.mark.parametrize("wg,N", [(8, 7), (8, 8), (8, 9), (8, 30), (5, 17), (1, 4)])
def test_rewinds_walk_back_through_every_push(wg, N):
    """From the empty state, N single pushes then N rewinds: rewind i
    restores exactly the meta that stood before push N - i, through the
    push that filled the window (it evicted nothing, so its rewind must
    shorten the window and leave head and the far count alone) and every
    evicting push after it.  The metas walked back to are the oracle's own
    after each push, which the closed-form pin above fixes."""
    cfg = _cfg(G=1, W=wg, rows=N, m=2)
    orc = oracle.from_config(cfg, synth.make_state(cfg))
    q, k, v = _rand_rows(cfg, N, seed=11)
    seen = [orc.meta()[0, :3].tolist()]
    for r in range(N):
        orc.step(q[r:r + 1], k[r:r + 1], v[r:r + 1], want=np.zeros(1, bool))
        seen.append(orc.meta()[0, :3].tolist())
    for i in range(N):
        orc.rewind()
        assert orc.meta()[0, :3].tolist() == seen[N - 1 - i], f"rewind {i + 1} of {N}"
    assert seen[0] == [0, 0, 0]


# -- rect and the negative-mass guard ----------------------------------------------

def test_rect_clamps_negative_far_weights():
    """With the rectifier on and mu <= 0 every u_b clamps to 0, so the far
    part vanishes and the output is the sliding-window softmax."""
    cfg = _cfg(W=12, rows=60, m=4, rect=True)
    st = synth.make_state(cfg)
    st.mu = -np.abs(st.mu)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=8)
    got = oracle.from_config(cfg, st).step(q, k, v)
    np.testing.assert_allclose(got, _window_reference(cfg, st, q, k, v), rtol=1e-12, atol=1e-13)


def test_negative_far_mass_is_dropped():
    """Without the rectifier, mu <= 0 makes D_far < 0: the guard drops the far
    numerator and denominator (o1b_attend), leaving the window softmax."""
    cfg = _cfg(W=12, rows=60, m=4, rect=False)
    st = synth.make_state(cfg)
    st.mu = -np.abs(st.mu)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=9)
    got = oracle.from_config(cfg, st).step(q, k, v)
    np.testing.assert_allclose(got, _window_reference(cfg, st, q, k, v), rtol=1e-12, atol=1e-13)


def test_positive_mu_far_part_is_not_negligible():
    """Sanity of the two pins above: with mu >= 0 the far part does move the
    output, so dropping it would be seen."""
    cfg = _cfg(W=12, rows=60, m=4)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=9)
    got = oracle.from_config(cfg, st).step(q, k, v)
    assert np.abs(got - _window_reference(cfg, st, q, k, v)).max() > 1e-2


# -- chunked equals serial ------------------------------------------------------

def _compare_states(a_meta, a_ring, a_M, a_Z, a_th, orc):
    np.testing.assert_array_equal(a_meta[:, :3], orc.meta()[:, :3])
    rk, rv = orc.ring()
    np.testing.assert_array_equal(a_ring[0], rk)
    np.testing.assert_array_equal(a_ring[1], rv)
    np.testing.assert_allclose(a_M, orc.M, rtol=1e-12)
    np.testing.assert_allclose(a_Z, orc.Z, rtol=1e-11)
    np.testing.assert_allclose(a_th, orc.theta, rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("head0,sizes", [(0, [64]), (13, [64, 64, 64]), (5, [7, 64, 1, 33])])
def test_chunked_equals_serial_tiny(head0, sizes):
    """The chunk form (far max at its post-chunk value, prefix mass, in-chunk
    causal coefficients) equals the serial steps up to rounding (o1_batch.rs
    module doc), including w = 16 < 64 rows where evicted keys come from the
    chunk itself."""
    cfg = synth.TINY.replace(head0=head0)
    st = synth.make_state(cfg)
    T = sum(sizes)
    q, k, v = synth.rows(cfg, 0, T)
    ser = oracle.from_config(cfg, st)
    want = ser.step(q, k, v)
    ch = chunked.from_config(cfg, st)
    outs, r0 = [], 0
    for n in sizes:
        outs.append(ch.sub_chunk(q[r0:r0 + n], k[r0:r0 + n], v[r0:r0 + n]))
        r0 += n
    np.testing.assert_allclose(np.concatenate(outs), want, rtol=1e-11, atol=1e-12)
    _compare_states(ch.meta, (ch.ring_k, ch.ring_v), ch.M, ch.Z, ch.theta, ser)


@pytest.mark.parametrize("w,w2,chunks", [(64, 64, [70, 9]), (64, 128, [70, 40])])
def test_chunked_equals_serial_reference_shapes(w, w2, chunks):
    """The pages' own chunk-vs-serial shapes (d 8, m 4, 2 sinks, 2 heads a
    group, a 100-row prompt first) with their deterministic jit inputs."""
    d, m, ns, H, t = 8, 4, 2, 2, 100
    cfg = synth.Config("ref", G=2, H=H, d=d, dv=d, ns=ns, W=max(w, w2), m=m, rows=t,
                       windows=(w, w2))
    st = synth.make_state(cfg)
    q, k, v = synth.jit_rows(2, H, d, 0, t + sum(chunks))
    ser = oracle.from_config(cfg, st)
    ser.step(q[:t], k[:t], v[:t])
    ch = chunked.from_config(cfg, st)
    ch.run(q[:t], k[:t], v[:t])
    r0 = t
    for n in chunks:
        want = ser.step(q[r0:r0 + n], k[r0:r0 + n], v[r0:r0 + n])
        got = ch.run(q[r0:r0 + n], k[r0:r0 + n], v[r0:r0 + n])
        np.testing.assert_allclose(got, want, rtol=1e-11, atol=1e-12)
        r0 += n
    _compare_states(ch.meta, (ch.ring_k, ch.ring_v), ch.M, ch.Z, ch.theta, ser)


# -- the oracle's own plumbing ----------------------------------------------------

def test_threads_and_resume_are_bit_identical():
    """Splitting heads over threads and stepping in pieces leave the float64
    results unchanged (same operations, same order)."""
    cfg = _cfg(G=2, H=4, W=16, rows=100, m=4)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=11)
    a = oracle.from_config(cfg, st, threads=1)
    oa = a.step(q, k, v)
    b = oracle.from_config(cfg, st, threads=8)
    ob = np.concatenate([b.step(q[:37], k[:37], v[:37]), b.step(q[37:], k[37:], v[37:])])
    np.testing.assert_array_equal(oa, ob)
    np.testing.assert_array_equal(a.theta, b.theta)
    np.testing.assert_array_equal(a.meta(), b.meta())


def test_sampled_outputs_match_full_outputs():
    cfg = _cfg(W=16, rows=80, m=4)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=12)
    full = oracle.from_config(cfg, st).step(q, k, v)
    want = np.zeros(cfg.rows, bool)
    want[[0, 17, 63, 79]] = True
    part = oracle.from_config(cfg, st).step(q, k, v, want=want)
    np.testing.assert_array_equal(part, full[want])


def test_rope_is_a_rotation():
    x = np.random.default_rng(0).standard_normal((5, 3, 16))
    y = synth.rope_rotate(x, np.arange(5) + 7)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_allclose(synth.rope_rotate(x, np.zeros(5)), x)


# ---- fused ingest (RoPE) and output gate ---------------------------------

def test_rope_rows_equals_complex_multiplication():
    """Pair (x_j, x_{j+d/2}) as the complex number x_j + i x_{j+d/2}: the
    rotate-half step is its product with c_j + i s_j, for any table."""
    from oracle import fused
    r = np.random.default_rng(3)
    x = r.standard_normal((6, 3, 16))
    tab = r.standard_normal((6, 16))
    z = (x[..., :8] + 1j * x[..., 8:]) * (tab[:, None, :8] + 1j * tab[:, None, 8:])
    got = fused.rope_rows(x, tab)
    np.testing.assert_allclose(got[..., :8], z.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(got[..., 8:], z.imag, rtol=0, atol=1e-13)


def test_rope_rows_with_an_angle_table_matches_the_angle_rotation():
    """With the table of positions p (cos, then sin of p * 10000^(-2j/d)) the
    oracle's rotation is the rotation by those angles, which keeps norms,
    is the identity at p = 0, and leaves <R_a q, R_b k> a function of a - b."""
    from oracle import fused
    r = np.random.default_rng(4)
    d = 32
    x = r.standard_normal((5, 2, d))
    pos = np.array([0, 3, 17, 1000, 40000])
    tab = np.concatenate([np.cos(pos[:, None] * 10000.0 ** (-2.0 * np.arange(d // 2) / d)),
                          np.sin(pos[:, None] * 10000.0 ** (-2.0 * np.arange(d // 2) / d))], axis=1)
    got = fused.rope_rows(x, tab)
    np.testing.assert_allclose(got, synth.rope_rotate(x, pos), rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.linalg.norm(got, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    np.testing.assert_array_equal(got[0], x[0])
    q, k = r.standard_normal(d), r.standard_normal(d)

    def at(v, p):
        a = p * 10000.0 ** (-2.0 * np.arange(d // 2) / d)
        return fused.rope_rows(v[None, None], np.concatenate([np.cos(a), np.sin(a)])[None])[0, 0]
    base = at(q, 9) @ at(k, 4)
    for t in (1, 50, 777):
        assert abs(at(q, 9 + t) @ at(k, 4 + t) - base) < 1e-12


def test_rope_rows_catches_a_swapped_sign():
    """A sign flip in either half of the rotation breaks the complex-product
    identity (the pin above would catch it)."""
    from oracle import fused
    r = np.random.default_rng(5)
    x = r.standard_normal((2, 1, 8))
    tab = np.concatenate([np.full((2, 4), 0.6), np.full((2, 4), 0.8)], axis=1)
    good = fused.rope_rows(x, tab)
    z = (x[..., :4] + 1j * x[..., 4:]) * (0.6 + 0.8j)
    wrong = np.concatenate([x[..., :4] * 0.6 + x[..., 4:] * 0.8, x[..., 4:] * 0.6 + x[..., :4] * 0.8], -1)
    np.testing.assert_allclose(good[..., :4], z.real, atol=1e-14)
    assert np.max(np.abs(wrong[..., :4] - z.real)) > 0.1


def test_gate_matches_the_logistic_function():
    """The gate is out * expit(z s): scipy's logistic function, 1/2 at 0,
    sigma(x) + sigma(-x) = 1, and finite at +-1000."""
    from scipy.special import expit
    from oracle import fused
    r = np.random.default_rng(6)
    out = r.standard_normal((4, 3, 8))
    z = r.standard_normal((4, 3, 8)) * 5
    s = r.uniform(0.5, 2.0, (3, 8))
    np.testing.assert_allclose(fused.gate_rows(out, z, s), out * expit(z * s[None]), rtol=1e-14)
    np.testing.assert_array_equal(fused.gate_rows(out, np.zeros_like(z), s), out / 2)
    xs = np.array([-1000.0, -30.0, -1.5, 0.0, 2.5, 40.0, 1000.0])
    np.testing.assert_allclose(fused.sigmoid(xs) + fused.sigmoid(-xs), 1.0, rtol=1e-15)
    assert fused.sigmoid(-1000.0) == 0.0 and fused.sigmoid(1000.0) == 1.0


def test_step_fused_is_rotate_step_gate():
    """The fused step with an identity table and no gate is the plain step;
    with a table it is the plain step on rotated rows, and the gate scales
    the plain output element by element."""
    from oracle import fused
    cfg = _cfg(rows=40)
    st = synth.make_state(cfg)
    q, k, v = _rand_rows(cfg, cfg.rows, seed=9)
    ident = np.concatenate([np.ones((cfg.rows, cfg.d // 2)), np.zeros((cfg.rows, cfg.d // 2))], 1)
    plain = oracle.from_config(cfg, st).step(q, k, v)
    np.testing.assert_array_equal(fused.step_fused(oracle.from_config(cfg, st), q, k, v, rope=ident), plain)
    tab = synth.rope_table(np.arange(cfg.rows) + 100, cfg.d)
    rq = synth.rope_rotate(q.astype(np.float64), np.arange(cfg.rows) + 100).astype(np.float32)
    rk = synth.rope_rotate(k.astype(np.float64), np.arange(cfg.rows) + 100).astype(np.float32)
    want = oracle.from_config(cfg, st).step(rq, rk, v)
    got = fused.step_fused(oracle.from_config(cfg, st), q, k, v, rope=tab)
    np.testing.assert_allclose(got, want, rtol=1e-5, atol=1e-6)   # fp32 table vs fp64 angles
    z, s = synth.gate_inputs(cfg, 0, cfg.rows)
    gated = fused.step_fused(oracle.from_config(cfg, st), q, k, v, gate=z, gate_scale=s)
    np.testing.assert_allclose(gated, plain / (1 + np.exp(-(z.astype(np.float64) * s))), rtol=1e-13)
