"""The allocation-free token call (swl_attend_token_noalloc) against the
token call that takes a scratch buffer (swl_attend_token /
swl_attend_token_fused), through the C ABI: the same outputs and states, bit
for bit (the same kernels on the same inputs), and the outputs within the
stated tolerance of the oracle.  Two geometries in a row, the second one
smaller, so that the second call runs on a static scratch still holding the
first one's larger partials."""
import numpy as np
import pytest

import oracle
import synth
import sink_window_landmark_amd as swl

from swl_gpu import banner, check_out, check_state, dev, geom_of, read_state, torch

pytestmark = pytest.mark.gpu


def _prefilled(cfg, T):
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, T + 8)
    st = swl.LayerState.from_host(geom_of(cfg), host)
    t = torch()
    out = t.empty((T, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    swl.swl_prefill(st, dev(q[:T]), dev(k[:T]), dev(v[:T]), out, swl.alloc_scratch(st.geom, T))
    orc = oracle.from_config(cfg, host)
    orc.step(q[:T], k[:T], v[:T], want=np.zeros(T, bool))
    return st, orc, (q[T:], k[T:], v[T:])


def _run(cfg, st, rows, noalloc, fuse=None):
    t = torch()
    q, k, v = (dev(x) for x in rows)
    n = q.shape[0]
    out = t.empty((n, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    scratch = None if noalloc else swl.alloc_scratch(st.geom, 1)
    for i in range(n):
        f = {} if fuse is None else {kk: (x[i:i + 1] if kk != "gate_scale" else x)
                                      for kk, x in fuse.items()}
        if noalloc:
            swl.swl_attend_token_noalloc(st, q[i:i + 1], k[i:i + 1], v[i:i + 1], out[i:i + 1], **f)
        elif fuse is None:
            swl.swl_attend_token(st, q[i:i + 1], k[i:i + 1], v[i:i + 1], out[i:i + 1], scratch)
        else:
            swl.swl_attend_token_fused(st, q[i:i + 1], k[i:i + 1], v[i:i + 1], out[i:i + 1],
                                       scratch, **f)
    t.cuda.synchronize()
    return out.cpu().numpy()


def _same(cfg, T, fuse_rows=False):
    st, orc, rows = _prefilled(cfg, T)
    a, b = st.clone(), st.clone()
    fuse = None
    if fuse_rows:
        n = rows[0].shape[0]
        pos = cfg.ns + T + np.arange(n)
        z, s = synth.gate_inputs(cfg, T, n)
        fuse = dict(rope=dev(synth.rope_table(pos, cfg.d)), gate=dev(z), gate_scale=dev(s))
    want = _run(cfg, a, rows, noalloc=False, fuse=fuse)
    got = _run(cfg, b, rows, noalloc=True, fuse=fuse)
    np.testing.assert_array_equal(got, want)
    sa, sb = read_state(a), read_state(b)
    for f in sa:
        np.testing.assert_array_equal(sb[f], sa[f], err_msg=f)
    if not fuse_rows:
        check_out(got, orc.step(*rows), "noalloc tokens")
        check_state(sb, orc)


def test_noalloc_tokens_match_the_scratch_call_large_then_small():
    big = synth.MAXWIN.replace(rows=3000)
    banner("noalloc tokens: max-window geometry after 3000 rows")
    _same(big, 3000)
    small = synth.Config("small-noalloc", G=2, H=3, d=64, dv=64, ns=3, W=300, m=16, rows=500,
                         windows=(300, 200), rope=True, landmark_scale=0.125)
    banner("noalloc tokens: a smaller geometry next, on the same static scratch")
    _same(small, 500)


def test_noalloc_fused_tokens_match_the_scratch_call():
    cfg = synth.Config("fused-noalloc", G=2, H=4, d=128, dv=128, ns=4, W=512, m=32, rows=700,
                       landmark_scale=1.0 / 128 ** 0.5)
    banner("noalloc fused tokens (RoPE table and gate)")
    _same(cfg, 700, fuse_rows=True)


def test_noalloc_refuses_a_geometry_beyond_its_scratch():
    """SWL_ESIZE before anything is enqueued: the state is unchanged."""
    cfg = synth.Config("huge", G=64, H=16, d=16, dv=16, ns=4, W=65536, m=4, rows=0)
    banner("noalloc: oversized geometry")
    host = synth.make_state(cfg)
    st = swl.LayerState.from_host(geom_of(cfg), host)
    before = read_state(st)
    t = torch()
    q = t.zeros((1, cfg.nh, cfg.d), device="cuda")
    k = t.zeros((1, cfg.G, cfg.d), device="cuda")
    v = t.zeros((1, cfg.G, cfg.dv), device="cuda")
    out = t.zeros((1, cfg.nh, cfg.dv), device="cuda")
    with pytest.raises(swl.SwlError, match="static scratch"):
        swl.swl_attend_token_noalloc(st, q, k, v, out)
    after = read_state(st)
    for f in before:
        np.testing.assert_array_equal(after[f], before[f])
