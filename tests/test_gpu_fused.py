"""Fused ingest (RoPE) and output gate, through the C ABI, against the oracle.

The rows are drawn before RoPE; the GPU turns q and k by the table inside
its kernels and gates the output on its way out, and the float64 oracle
(``oracle.fused.step_fused``) rotates, steps and gates on the CPU.  The ring
then holds computed (turned) keys, so it is compared at rounding level
instead of bit for bit; meta stays exact.
"""
import numpy as np
import pytest

import oracle
import synth
import sink_window_landmark_amd as swl
from oracle import fused

from swl_gpu import banner, check_out, check_state, dev, geom_of, oracle_threads, read_state, torch

pytestmark = pytest.mark.gpu


def _raw(cfg):
    """The same workload with rows drawn before RoPE."""
    return cfg.replace(rope=False)


def _inputs(cfg, rows, pos0, rope=True, gate=True):
    tab = synth.rope_table(np.arange(rows) + pos0, cfg.d) if rope else None
    z, s = synth.gate_inputs(cfg, 0, rows) if gate else (None, None)
    return tab, z, s


def _opt(a):
    return dev(a) if a is not None else None


def check_ring(gpu, orc):
    """Occupied ring slots against the oracle's at fp32 rounding level (the
    GPU turns the keys in fp32, the oracle in float64)."""
    rk, rv = orc.ring()
    for g in range(orc.G):
        meta = orc.meta()[g]
        ln, hd = int(meta[0]), int(meta[1])
        slots = [(hd + x) % orc.windows[g] for x in range(ln)]
        np.testing.assert_allclose(gpu["ring_k"][g, slots], rk[g, slots], rtol=1e-6, atol=1e-6)
        np.testing.assert_array_equal(gpu["ring_v"][g, slots], rv[g, slots].astype(np.float32))


@pytest.mark.parametrize("rope,gate", [(True, True), (True, False), (False, True)])
def test_fused_prefill(rope, gate):
    cfg = synth.SMALL.replace(rows=1500)   # several sub-chunks; evictions start at row 1024
    banner(f"fused prefill rope={rope} gate={gate} T={cfg.rows}")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(_raw(cfg), 0, cfg.rows)
    tab, z, s = _inputs(cfg, cfg.rows, 5000, rope, gate)
    st = swl.LayerState.from_host(geom_of(cfg), host)
    t = torch()
    out = t.empty((cfg.rows, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    scratch = swl.alloc_scratch(st.geom, cfg.rows)
    swl.swl_prefill_fused(st, dev(q), dev(k), dev(v), out, scratch, rope=_opt(tab), gate=_opt(z),
                          gate_scale=_opt(s))
    t.cuda.synchronize()
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    want = fused.step_fused(orc, q, k, v, rope=tab, gate=z, gate_scale=s)
    check_out(out.cpu().numpy(), want)
    gs = read_state(st)
    check_state(gs, orc, ring=False)
    check_ring(gs, orc)


def test_fused_identity_table_is_the_plain_path():
    """cos = 1, sin = 0 turns nothing: x*1 - y*0 and y*1 + x*0 are exact in
    fp32, so the fused prefill gives the plain prefill's bits."""
    cfg = synth.SMALL.replace(rows=700)
    banner("fused prefill with the identity table")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    ident = np.concatenate([np.ones((cfg.rows, cfg.d // 2)), np.zeros((cfg.rows, cfg.d // 2))],
                           1).astype(np.float32)
    t = torch()
    outs, states = [], []
    for use in (False, True):
        st = swl.LayerState.from_host(geom_of(cfg), host)
        out = t.empty((cfg.rows, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
        scratch = swl.alloc_scratch(st.geom, cfg.rows)
        if use:
            swl.swl_prefill_fused(st, dev(q), dev(k), dev(v), out, scratch, rope=dev(ident))
        else:
            swl.swl_prefill(st, dev(q), dev(k), dev(v), out, scratch)
        t.cuda.synchronize()
        outs.append(out.cpu().numpy())
        states.append(read_state(st))
    np.testing.assert_array_equal(outs[1], outs[0])
    for f in ("meta", "ring_k", "ring_v", "mz", "theta"):
        np.testing.assert_array_equal(states[1][f], states[0][f], err_msg=f)


@pytest.mark.parametrize("sizes", [[64, 7, 33, 64], [1] * 12])
def test_fused_chunks_then_commit(sizes):
    cfg = synth.Config("fchunks", G=2, H=2, d=64, dv=64, ns=4, W=96, m=16,
                       rows=int(np.sum(sizes)))
    banner(f"fused attend_chunk + commit sizes={sizes}")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    tab, z, s = _inputs(cfg, cfg.rows, 77)
    st = swl.LayerState.from_host(geom_of(cfg), host)
    t = torch()
    scratch = swl.alloc_scratch(st.geom, 64)
    orc = oracle.from_config(cfg, host)
    r0 = 0
    for n in sizes:
        sl = slice(r0, r0 + n)
        out = t.empty((n, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
        kd, vd, td = dev(k[sl]), dev(v[sl]), dev(tab[sl])
        swl.swl_attend_chunk_fused(st, dev(q[sl]), kd, vd, out, scratch, rope=td, gate=dev(z[sl]),
                                   gate_scale=dev(s))
        swl.swl_commit_fused(st, kd, vd, scratch, rope=td)
        t.cuda.synchronize()
        want = fused.step_fused(orc, q[sl], k[sl], v[sl], rope=tab[sl], gate=z[sl], gate_scale=s)
        check_out(out.cpu().numpy(), want, f"rows {r0}..{r0 + n - 1}")
        r0 += n
    gs = read_state(st)
    check_state(gs, orc, ring=False)
    check_ring(gs, orc)


def test_fused_verify_then_commit_rows():
    """A verify over 64 speculative rows leaves the state alone; committing
    the first 37 with the same table gives the state of 37 turned rows."""
    cfg = synth.Config("fverify", G=2, H=2, d=64, dv=64, ns=4, W=64, m=16, rows=164)
    banner("fused verify + commit_rows")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    tab, z, s = _inputs(cfg, cfg.rows, 300)
    st = swl.LayerState.from_host(geom_of(cfg), host)
    t = torch()
    scratch = swl.alloc_scratch(st.geom, 100)
    swl.swl_prefill_fused(st, dev(q[:100]), dev(k[:100]), dev(v[:100]),
                          t.empty((100, cfg.nh, cfg.dv), dtype=t.float32, device="cuda"), scratch,
                          rope=dev(tab[:100]))
    sp = slice(100, 164)
    out = t.empty((64, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    swl.swl_attend_chunk_fused(st, dev(q[sp]), dev(k[sp]), dev(v[sp]), out, scratch,
                               rope=dev(tab[sp]), gate=dev(z[sp]), gate_scale=dev(s))
    acc = slice(100, 137)
    swl.swl_commit_rows_fused(st, dev(k[acc]), dev(v[acc]), scratch, rope=dev(tab[acc]))
    t.cuda.synchronize()
    orc = oracle.from_config(cfg, host)
    fused.step_fused(orc, q[:100], k[:100], v[:100], rope=tab[:100])
    probe = oracle.from_config(cfg, host)
    fused.step_fused(probe, q[:100], k[:100], v[:100], rope=tab[:100])
    want = fused.step_fused(probe, q[sp], k[sp], v[sp], rope=tab[sp], gate=z[sp], gate_scale=s)
    check_out(out.cpu().numpy(), want, "speculative rows")
    fused.step_fused(orc, q[acc], k[acc], v[acc], rope=tab[acc])
    gs = read_state(st)
    check_state(gs, orc, ring=False)
    check_ring(gs, orc)


def test_fused_tokens():
    """Decode with the row's table and gate, after a fused prompt: the
    window fills and then evicts."""
    cfg = synth.Config("ftok", G=2, H=4, d=128, dv=128, ns=4, W=64, m=16, rows=40)
    steps = 60
    banner(f"fused tokens: prompt {cfg.rows}, {steps} tokens")
    host = synth.make_state(cfg)
    n = cfg.rows + steps
    q, k, v = synth.rows(cfg, 0, n)
    tab, z, s = _inputs(cfg, n, 11)
    st = swl.LayerState.from_host(geom_of(cfg), host)
    t = torch()
    scratch = swl.alloc_scratch(st.geom, cfg.rows)
    swl.swl_prefill_fused(st, dev(q[:cfg.rows]), dev(k[:cfg.rows]), dev(v[:cfg.rows]),
                          t.empty((cfg.rows, cfg.nh, cfg.dv), dtype=t.float32, device="cuda"),
                          scratch, rope=dev(tab[:cfg.rows]))
    outs = t.empty((steps, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    qd, kd, vd, td, zd = (dev(a[cfg.rows:]) for a in (q, k, v, tab, z))
    sd = dev(s)
    for i in range(steps):
        swl.swl_attend_token_fused(st, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], outs[i:i + 1],
                                   scratch, rope=td[i:i + 1], gate=zd[i:i + 1], gate_scale=sd)
    t.cuda.synchronize()
    orc = oracle.from_config(cfg, host)
    fused.step_fused(orc, q[:cfg.rows], k[:cfg.rows], v[:cfg.rows], rope=tab[:cfg.rows])
    tl = slice(cfg.rows, n)
    want = fused.step_fused(orc, q[tl], k[tl], v[tl], rope=tab[tl], gate=z[tl], gate_scale=s)
    check_out(outs.cpu().numpy(), want, "tokens")
    gs = read_state(st)
    check_state(gs, orc, ring=False)
    check_ring(gs, orc)


def test_fused_small_heads():
    """d = 8 (a float4 on each side of the halves) and d = 16."""
    for d in (8, 16):
        cfg = synth.Config(f"fsmall{d}", G=1, H=2, d=d, dv=d, ns=2, W=32, m=4, rows=150)
        banner(f"fused prefill d={d}")
        host = synth.make_state(cfg)
        q, k, v = synth.rows(cfg, 0, cfg.rows)
        tab, z, s = _inputs(cfg, cfg.rows, 3)
        st = swl.LayerState.from_host(geom_of(cfg), host)
        t = torch()
        out = t.empty((cfg.rows, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
        scratch = swl.alloc_scratch(st.geom, cfg.rows)
        swl.swl_prefill_fused(st, dev(q), dev(k), dev(v), out, scratch, rope=dev(tab), gate=dev(z),
                              gate_scale=dev(s))
        t.cuda.synchronize()
        orc = oracle.from_config(cfg, host)
        check_out(out.cpu().numpy(), fused.step_fused(orc, q, k, v, rope=tab, gate=z, gate_scale=s))
        gs = read_state(st)
        check_state(gs, orc, ring=False)
        check_ring(gs, orc)
