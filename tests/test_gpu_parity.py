"""GPU path (through the C ABI) against the CPU oracle.

Inputs are the seeded synthetic workloads of ``synth`` (and the pages' own
deterministic ``jit`` rows for their test shapes); expected values are the
float64 serial oracle's.  Every test compares every output row it
produces and the whole final state.
"""
import numpy as np
import pytest

import oracle
import synth
import sink_window_landmark_amd as swl

from swl_gpu import (ATOL, banner, check_out, check_state, dev, excess, geom_of, oracle_threads,
                     read_state, torch)

pytestmark = pytest.mark.gpu


def _state(cfg, host):
    return swl.LayerState.from_host(geom_of(cfg), host)


def _prefill(cfg, st, q, k, v, poison=False):
    t = torch()
    out = t.empty((q.shape[0], cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    scratch = swl.alloc_scratch(st.geom, q.shape[0])
    if poison:
        scratch.view(t.float32)[: scratch.numel() // 4].fill_(float("nan"))
        out.fill_(float("nan"))
    swl.swl_prefill(st, dev(q), dev(k), dev(v), out, scratch)
    t.cuda.synchronize()
    return out.cpu().numpy()


def _chunks(cfg, st, q, k, v, sizes, poison=False):
    """attend_chunk + commit over consecutive chunks of the given sizes."""
    t = torch()
    outs = []
    scratch = swl.alloc_scratch(st.geom, 64)
    r0 = 0
    for n in sizes:
        out = t.empty((n, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
        if poison:
            scratch.view(t.float32)[: scratch.numel() // 4].fill_(float("nan"))
        qd, kd, vd = dev(q[r0:r0 + n]), dev(k[r0:r0 + n]), dev(v[r0:r0 + n])
        swl.swl_attend_chunk(st, qd, kd, vd, out, scratch)
        swl.swl_commit(st, kd, vd, scratch)
        outs.append(out)
        r0 += n
    t.cuda.synchronize()
    return np.concatenate([o.cpu().numpy() for o in outs])


# -- tiny layer (w = 16 < 64 rows, ring 10/16, empty far field) ----------------

def test_tiny_attend_commit():
    banner("tiny attend_chunk + commit")
    cfg = synth.TINY
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    got = _chunks(cfg, st, q, k, v, [64], poison=True)
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


def test_tiny_prefill():
    banner("tiny prefill")
    cfg = synth.TINY
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q, k, v, poison=True)
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


@pytest.mark.parametrize("head0,sizes", [(13, [64, 64, 64]), (5, [7, 64, 1, 33]), (0, [1] * 40)])
def test_tiny_chunk_sizes_and_wrapped_head(head0, sizes):
    banner(f"tiny chunks head0={head0} sizes={sizes[:4]}...")
    cfg = synth.TINY.replace(head0=head0)
    host = synth.make_state(cfg)
    T = sum(sizes)
    q, k, v = synth.rows(cfg, 0, T)
    st = _state(cfg, host)
    got = _chunks(cfg, st, q, k, v, sizes, poison=True)
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)
    # the same rows in one prefill call
    st2 = _state(cfg, host)
    got2 = _prefill(cfg, st2, q, k, v)
    check_out(got2, oracle.from_config(cfg, host).step(q, k, v), "prefill")
    check_state(read_state(st2), orc)


# -- the pages' chunk-vs-serial shapes, with their jit inputs ---------------------

@pytest.mark.parametrize("w,w2,chunks", [(64, 64, [70, 9]), (64, 128, [70, 40])])
def test_reference_shapes(w, w2, chunks):
    banner(f"reference shapes w={w}/{w2} chunks={chunks}")
    d, m, ns, H, t0 = 8, 4, 2, 2, 100
    cfg = synth.Config("ref", G=2, H=H, d=d, dv=d, ns=ns, W=max(w, w2), m=m, rows=t0,
                       windows=(w, w2))
    host = synth.make_state(cfg)
    q, k, v = synth.jit_rows(2, H, d, 0, t0 + sum(chunks))
    orc = oracle.from_config(cfg, host)
    st = _state(cfg, host)
    got0 = _prefill(cfg, st, q[:t0], k[:t0], v[:t0])
    check_out(got0, orc.step(q[:t0], k[:t0], v[:t0]), "prompt")
    r0 = t0
    for n in chunks:
        sl = slice(r0, r0 + n)
        got = _prefill(cfg, st, q[sl], k[sl], v[sl])
        check_out(got, orc.step(q[sl], k[sl], v[sl]), f"chunk {n}")
        r0 += n
    check_state(read_state(st), orc)


@pytest.mark.parametrize("w,w2,chunks,tokens", [(128, 512, [64, 64], 0), (128, 128, [5], 1)])
def test_reference_production_head(w, w2, chunks, tokens):
    """The pages' production head geometry (d = dv = 256, m = 32, 4 sinks, 6
    query heads, a 300-row prompt), continued through attend_chunk + commit
    and, in the second case, a token after a 5-row verify chunk."""
    banner(f"production head d=256 w={w}/{w2} chunks={chunks} tokens={tokens}")
    d, m, ns, H, t0 = 256, 32, 4, 6, 300
    cfg = synth.Config("prod", G=2, H=H, d=d, dv=d, ns=ns, W=max(w, w2), m=m, rows=t0,
                       windows=(w, w2))
    host = synth.make_state(cfg)
    n = t0 + sum(chunks) + tokens
    q, k, v = synth.jit_rows(2, H, d, 0, n)
    orc = oracle.from_config(cfg, host)
    st = _state(cfg, host)
    got0 = _prefill(cfg, st, q[:t0], k[:t0], v[:t0], poison=True)
    check_out(got0, orc.step(q[:t0], k[:t0], v[:t0]), "prompt")
    r0 = t0 + sum(chunks)
    got1 = _chunks(cfg, st, q[t0:r0], k[t0:r0], v[t0:r0], chunks, poison=True)
    check_out(got1, orc.step(q[t0:r0], k[t0:r0], v[t0:r0]), f"chunks {chunks}")
    if tokens:
        got2 = _tokens(cfg, st, q[r0:], k[r0:], v[r0:])
        check_out(got2, orc.step(q[r0:], k[r0:], v[r0:]), "token")
    check_state(read_state(st), orc)


# -- verify: speculative rows, then a commit of the accepted ones --------------------

@pytest.mark.parametrize("spec,accepted", [(64, 37), (64, 64), (20, 1)])
def test_verify_then_commit_accepted_rows(spec, accepted):
    """attend_chunk over speculative rows leaves the state as it was; the
    accepted rows are then committed with swl_commit_rows (far_e over them
    only), and the layer continues from that state."""
    banner(f"verify spec={spec} accepted={accepted}")
    cfg = synth.Config("verify", G=2, H=4, d=64, dv=64, ns=4, W=128, m=16, rows=300,
                       windows=(96, 128), rope=True, landmark_scale=0.125)
    host = synth.make_state(cfg)
    t0, nxt = 300, 80
    q, k, v = synth.rows(cfg, 0, t0 + spec + nxt)
    st = _state(cfg, host)
    _prefill(cfg, st, q[:t0], k[:t0], v[:t0])
    before = read_state(st)
    sp = slice(t0, t0 + spec)
    t = torch()
    out = t.empty((spec, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    scratch = swl.alloc_scratch(st.geom, 64)
    kd, vd = dev(k[sp]), dev(v[sp])
    swl.swl_attend_chunk(st, dev(q[sp]), kd, vd, out, scratch)
    t.cuda.synchronize()
    after = read_state(st)
    for f in before:
        assert np.array_equal(before[f], after[f], equal_nan=True), f"attend_chunk changed {f}"
    spec_orc = oracle.from_config(cfg, host)
    spec_orc.step(q[:t0], k[:t0], v[:t0], want=np.zeros(t0, bool))
    check_out(out.cpu().numpy(), spec_orc.step(q[sp], k[sp], v[sp]), "speculative rows")
    # accept the first rows: the state of that many serial steps
    swl.swl_commit_rows(st, kd[:accepted].contiguous(), vd[:accepted].contiguous(),
                        swl.alloc_scratch(st.geom, accepted))
    orc = oracle.from_config(cfg, host)
    orc.step(q[:t0], k[:t0], v[:t0], want=np.zeros(t0, bool))
    orc.step(q[t0:t0 + accepted], k[t0:t0 + accepted], v[t0:t0 + accepted],
             want=np.zeros(accepted, bool))
    check_state(read_state(st), orc)
    # the layer goes on with new rows
    nx = slice(t0 + spec, t0 + spec + nxt)
    got = _prefill(cfg, st, q[nx], k[nx], v[nx])
    check_out(got, orc.step(q[nx], k[nx], v[nx]), "rows after the commit")
    check_state(read_state(st), orc)


def test_commit_rows_matches_prefill_state():
    """swl_commit_rows over several sub-chunks gives prefill's state."""
    banner("commit_rows over 150 rows vs prefill")
    cfg = synth.SMALL.replace(rows=500, W=256, m=16)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 500)
    a = _state(cfg, host)
    _prefill(cfg, a, q[:350], k[:350], v[:350])
    b = a.clone()
    swl.swl_commit_rows(a, dev(k[350:]), dev(v[350:]), swl.alloc_scratch(a.geom, 150))
    _prefill(cfg, b, q[350:], k[350:], v[350:])
    orc = oracle.from_config(cfg, host)
    orc.step(q, k, v, want=np.zeros(500, bool))
    check_state(read_state(a), orc)
    check_state(read_state(b), orc)


# -- seal from exact rows, rewind one push ------------------------------------------

def test_seal_from_exact_rows():
    """swl_seal builds the state of the rows (ring = the last w_g of them,
    M/Z/Theta over the rest) without attending them; the layer then goes on
    as the oracle does."""
    banner("seal 700 rows, then 100 more")
    cfg = synth.Config("seal", G=2, H=4, d=64, dv=64, ns=4, W=256, m=16, rows=800,
                       windows=(128, 256), rope=True, landmark_scale=0.125)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 800)
    st = _state(cfg, host)
    swl.swl_seal(st, dev(k[:700]), dev(v[:700]), swl.alloc_scratch(st.geom, 700),
                 windows=cfg.meta_windows())
    orc = oracle.from_config(cfg, host)
    orc.step(q[:700], k[:700], v[:700], want=np.zeros(700, bool))
    check_state(read_state(st), orc)
    got = _prefill(cfg, st, q[700:], k[700:], v[700:])
    check_out(got, orc.step(q[700:], k[700:], v[700:]), "rows after the seal")
    check_state(read_state(st), orc)


@pytest.mark.parametrize("T", [30, 47, 63, 64, 200])
def test_rewind_one_push(T):
    """swl_rewind moves meta back by one push in every group, as the
    oracle's rewind does: after T rows with windows 48 / 64 (partial, the
    push that filled a window -- T = 47 then a token for the first group,
    T = 63 for the second -- and full windows), then a token followed by a
    rewind, then a second rewind."""
    banner(f"rewind after {T} rows")
    cfg = synth.Config("rewind", G=2, H=2, d=32, dv=32, ns=2, W=64, m=8, rows=T,
                       windows=(48, 64))
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, T + 1)
    st = _state(cfg, host)
    _prefill(cfg, st, q[:T], k[:T], v[:T])
    orc = oracle.from_config(cfg, host)
    orc.step(q[:T], k[:T], v[:T], want=np.zeros(T, bool))
    swl.swl_rewind(st)
    orc.rewind()
    check_state(read_state(st), orc, ring=False)
    out = torch().empty((1, cfg.nh, cfg.dv), device="cuda")
    swl.swl_attend_token(st, dev(q[T:]), dev(k[T:]), dev(v[T:]), out,
                         swl.alloc_scratch(st.geom, 1))
    orc.step(q[T:], k[T:], v[T:], want=np.zeros(1, bool))
    swl.swl_rewind(st)
    orc.rewind()
    got = read_state(st)
    np.testing.assert_array_equal(got["meta"][:, :3], orc.meta()[:, :3])
    swl.swl_rewind(st)
    orc.rewind()
    got = read_state(st)
    np.testing.assert_array_equal(got["meta"][:, :3], orc.meta()[:, :3])
    assert np.all(got["meta"][:, 2] < 1 << 30), "far count wrapped around"


# -- the small layer, every row ------------------------------------------------------

def test_small_full():
    cfg = synth.SMALL
    banner(f"small layer prefill T={cfg.rows}")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    # reset through the library: the synthetic state is the empty one
    swl.swl_init_state(st, cfg.meta_windows())
    got = _prefill(cfg, st, q, k, v, poison=True)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


def test_split_window_calls():
    """Calls with few attention work items split the window over several
    blocks and merge their partial softmax states: prefills of 1500 and 700
    rows (2 and 5 splits; the far field starts at row 2048), then 64-, 37-
    and 64-row attend_chunk + commit calls (12 splits; the far score's
    landmark-row tiles over 8 blocks per group, four waves per tile), at the
    max-window geometry, every output against the oracle."""
    cfg = synth.CONFIGS["maxwin"]
    banner("maxwin split-window calls: prefill 1500 + 700, chunks 64/37/64")
    host = synth.make_state(cfg)
    sizes = [64, 37, 64]
    n = 2200 + sum(sizes)
    q, k, v = synth.rows(cfg, 0, n)
    st = _state(cfg, host)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    for a, b in ((0, 1500), (1500, 2200)):
        got = _prefill(cfg, st, q[a:b], k[a:b], v[a:b], poison=True)
        check_out(got, orc.step(q[a:b], k[a:b], v[a:b]), f"prefill rows {a}..{b - 1}")
    got = _chunks(cfg, st, q[2200:], k[2200:], v[2200:], sizes, poison=True)
    check_out(got, orc.step(q[2200:], k[2200:], v[2200:]), f"chunks {sizes}")
    check_state(read_state(st), orc)


@pytest.mark.parametrize("d", [32, 64])
def test_split_window_small_heads(d):
    """The split-window path at d = 32 and 64 (m = 16: one landmark tile),
    three query heads per group (an idle head slot in every block) and
    per-group windows 256/128: a 700-row prompt (3 splits per work item),
    then 64- and 20-row attend_chunk + commit calls, against the oracle."""
    import math
    cfg = synth.Config("splitd", G=2, H=3, d=d, dv=d, ns=4, W=256, m=16, rows=700, windows=(256, 128),
                       rope=True, landmark_scale=1.0 / math.sqrt(d))
    banner(f"split-window d={d}: prefill 700, chunks 64/20")
    host = synth.make_state(cfg)
    sizes = [64, 20]
    n = cfg.rows + sum(sizes)
    q, k, v = synth.rows(cfg, 0, n)
    st = _state(cfg, host)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    T = cfg.rows
    got = _prefill(cfg, st, q[:T], k[:T], v[:T], poison=True)
    check_out(got, orc.step(q[:T], k[:T], v[:T]), "prefill")
    got = _chunks(cfg, st, q[T:], k[T:], v[T:], sizes, poison=True)
    check_out(got, orc.step(q[T:], k[T:], v[T:]), f"chunks {sizes}")
    check_state(read_state(st), orc)


@pytest.mark.parametrize("rect", [False, True])
def test_split_merge_landmark_tiles(rect):
    """Merges of few heads split each head's query rows over two blocks and
    the landmarks over their two waves: m = 48 (a second landmark tile with 16
    landmarks), mu of mixed signs (the two tiles' far masses of either sign;
    head 0 all negative, so its far part is dropped by the guard on the total),
    a 300-row prompt (5 sub-chunks, 30 merge heads), then 64-, 20- (no rows in
    the second half) and 33-row attend_chunk + commit calls, against the
    oracle."""
    banner(f"split merge m=48 rect={rect}: prefill 300, chunks 64/20/33")
    cfg = synth.Config("mtiles", G=2, H=3, d=64, dv=64, ns=4, W=128, m=48, rows=300,
                       windows=(128, 96), rect=rect)
    host = synth.make_state(cfg)
    r = np.random.default_rng(11)
    host.mu = (r.standard_normal(host.mu.shape) / cfg.m).astype(np.float32)
    host.mu[0] = -np.abs(host.mu[0])
    sizes = [64, 20, 33]
    n = cfg.rows + sum(sizes)
    q, k, v = synth.rows(cfg, 0, n)
    st = _state(cfg, host)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    T = cfg.rows
    got = _prefill(cfg, st, q[:T], k[:T], v[:T], poison=True)
    check_out(got, orc.step(q[:T], k[:T], v[:T]), "prefill")
    got = _chunks(cfg, st, q[T:], k[T:], v[T:], sizes, poison=True)
    check_out(got, orc.step(q[T:], k[T:], v[T:]), f"chunks {sizes}")
    check_state(read_state(st), orc)


def test_split_merge_wide_heads():
    """The split merge at d = 256 with two landmark tiles (m = 64; two heads
    per attention block, the largest staging of the far readout): a 200-row
    prompt (4 sub-chunks, 16 merge heads), then 64- and 20-row
    attend_chunk + commit calls, against the oracle."""
    import math
    banner("split merge d=256 m=64: prefill 200, chunks 64/20")
    cfg = synth.Config("wide", G=2, H=2, d=256, dv=256, ns=4, W=128, m=64, rows=200, windows=(128, 72),
                       landmark_scale=1.0 / math.sqrt(256))
    host = synth.make_state(cfg)
    sizes = [64, 20]
    n = cfg.rows + sum(sizes)
    q, k, v = synth.rows(cfg, 0, n)
    st = _state(cfg, host)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    T = cfg.rows
    got = _prefill(cfg, st, q[:T], k[:T], v[:T], poison=True)
    check_out(got, orc.step(q[:T], k[:T], v[:T]), "prefill")
    got = _chunks(cfg, st, q[T:], k[T:], v[T:], sizes, poison=True)
    check_out(got, orc.step(q[T:], k[T:], v[T:]), f"chunks {sizes}")
    check_state(read_state(st), orc)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["maxwin", "mixed"])
def test_full_size_every_row(name):
    """The max-window (32768 rows) and mixed-window (131072 rows, windows
    512/1024/2048/2048) prompts in one swl_prefill call each, every output
    row against the oracle, then the whole final state."""
    cfg = synth.CONFIGS[name]
    banner(f"{name} prefill T={cfg.rows}")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q, k, v)
    banner(f"{name} oracle over all {cfg.rows} rows")
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    want = orc.step(q, k, v)
    check_out(got, want)
    # the rows around each group's first eviction, reported on their own
    for g in range(cfg.G):
        w = cfg.window(g)
        rs = [x for x in (w - 1, w, w + 1, w + 63, w + 64) if 0 <= x < cfg.rows]
        hs = slice(g * cfg.H, (g + 1) * cfg.H)
        check_out(got[rs][:, hs], want[rs][:, hs], f"group {g} (window {w}) rows {rs}")
    check_state(read_state(st), orc)


# -- decode: one row at a time after a long prompt ----------------------------------------

@pytest.mark.timeout(600)
def test_decode_after_prompt():
    """The decode workload: the max-window state after its 32768-row prompt,
    then all 4096 single-row steps, every output and the final state against
    the oracle."""
    cfg = synth.DECODE
    steps = cfg.decode_steps
    banner(f"decode: prefill {cfg.rows} then {steps} tokens")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows + steps)
    st = _state(cfg, host)
    _prefill(cfg, st, q[:cfg.rows], k[:cfg.rows], v[:cfg.rows])
    t = torch()
    scratch = swl.alloc_scratch(st.geom, 1)
    outs = t.empty((steps, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    qd, kd, vd = dev(q[cfg.rows:]), dev(k[cfg.rows:]), dev(v[cfg.rows:])
    for i in range(steps):
        swl.swl_attend_token(st, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], outs[i:i + 1], scratch)
    t.cuda.synchronize()
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    orc.step(q[:cfg.rows], k[:cfg.rows], v[:cfg.rows], want=np.zeros(cfg.rows, bool))
    want = orc.step(q[cfg.rows:], k[cfg.rows:], v[cfg.rows:])
    check_out(outs.cpu().numpy(), want)
    check_state(read_state(st), orc)


# -- edge cases ------------------------------------------------------------------------------

@pytest.mark.parametrize("rect", [False, True])
def test_negative_mu_guard_and_rect(rect):
    banner(f"negative mu, rect={rect}")
    cfg = synth.Config("neg", G=2, H=3, d=32, dv=32, ns=3, W=48, m=16, rows=200,
                       windows=(40, 48), rect=rect)
    host = synth.make_state(cfg)
    r = np.random.default_rng(3)
    host.mu = (r.standard_normal(host.mu.shape) / cfg.m).astype(np.float32)  # mixed signs
    host.mu[0] = -np.abs(host.mu[0])                                          # head 0: D_far < 0
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q, k, v)
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


def test_no_sinks():
    """A layer without sinks: no sink tiles, the window tiles start the key
    tiles, and the decode path runs on from the prefilled state."""
    banner("no sinks")
    cfg = synth.Config("nosink", G=2, H=2, d=32, dv=32, ns=0, W=96, m=8, rows=400,
                       windows=(70, 96))
    host = synth.make_state(cfg)
    T = 360
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q[:T], k[:T], v[:T])
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q[:T], k[:T], v[:T]), "prefill")
    check_out(_tokens(cfg, st, q[T:], k[T:], v[T:]), orc.step(q[T:], k[T:], v[T:]), "tokens")
    check_state(read_state(st), orc)


@pytest.mark.parametrize("vscale", [1e-5, 1e-20, 1e5, 1e20])
def test_value_scales(vscale):
    """Values far from unit scale (below fp16's normal range, and above its
    largest value) through the fp16 hi/lo value products, which split them
    after a power-of-two scale per pass and group: the stated bound,
    elementwise, with its absolute part scaled by the values' scale (the
    output and Theta are linear in the values), through prefill, chunks and
    tokens."""
    banner(f"value scale x {vscale:g}")
    cfg = synth.Config("vscale", G=2, H=2, d=64, dv=64, ns=4, W=128, m=16, rows=500,
                       windows=(96, 128), rope=True, landmark_scale=0.125)
    host = synth.make_state(cfg)
    host.sink_v = (host.sink_v.astype(np.float64) * vscale).astype(np.float32)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    v = (v.astype(np.float64) * vscale).astype(np.float32)
    st = _state(cfg, host)
    orc = oracle.from_config(cfg, host)
    a = ATOL * vscale
    T = 400
    check_out(_prefill(cfg, st, q[:T], k[:T], v[:T], poison=True), orc.step(q[:T], k[:T], v[:T]),
              "prefill", atol=a)
    check_state(read_state(st), orc, vscale=vscale)
    check_out(_chunks(cfg, st, q[T:T + 80], k[T:T + 80], v[T:T + 80], [64, 16], poison=True),
              orc.step(q[T:T + 80], k[T:T + 80], v[T:T + 80]), "chunks", atol=a)
    check_out(_tokens(cfg, st, q[T + 80:], k[T + 80:], v[T + 80:]),
              orc.step(q[T + 80:], k[T + 80:], v[T + 80:]), "tokens", atol=a)
    check_state(read_state(st), orc, vscale=vscale)


@pytest.mark.parametrize("kq", [2.0 ** 13, 2.0 ** -15])
def test_key_query_range(kq):
    """Keys (sinks, rows, landmark keys) times kq and queries (rows, landmark
    queries) divided by it, so every score is unchanged: keys up to about
    2^15 (the fp16 splits' range is 65504), or queries up to about
    2^14 / (scale log2 e) with keys in fp16's subnormal range.  The stated
    bound, elementwise."""
    banner(f"keys x {kq:g}, queries / {kq:g}")
    cfg = synth.Config("kqrange", G=2, H=2, d=64, dv=64, ns=4, W=128, m=16, rows=400,
                       windows=(128, 96), landmark_scale=0.125)
    host = synth.make_state(cfg)
    up = lambda x, f: (x.astype(np.float64) * f).astype(np.float32)
    host.sink_k = up(host.sink_k, kq)
    host.k_tilde = up(host.k_tilde, kq)
    host.q_tilde = up(host.q_tilde, 1.0 / kq)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    q, k = up(q, 1.0 / kq), up(k, kq)
    print(f"  max|k| {np.abs(k).max():.4g}  max|q| {np.abs(q).max():.4g}  "
          f"max|q~| {np.abs(host.q_tilde).max():.4g}", flush=True)
    st = _state(cfg, host)
    orc = oracle.from_config(cfg, host)
    T = 360
    check_out(_prefill(cfg, st, q[:T], k[:T], v[:T]), orc.step(q[:T], k[:T], v[:T]), "prefill")
    check_out(_tokens(cfg, st, q[T:], k[T:], v[T:]), orc.step(q[T:], k[T:], v[T:]), "tokens")
    check_state(read_state(st), orc)


def test_peaked_softmax_large_values():
    """Keys x 20 and values x 1000: a very peaked near softmax (scores spread
    over about +-80 in log2 units) with large values.  Beyond the stated
    contract (unit-scale scores), so the bound here is taken norm-wise: 1e-4
    of the largest |output| of the same (row, head) plus 1e-5 times the
    value scale.  Elementwise it is beyond any fp32 evaluation: a score
    carries an fp32 rounding error of order 2^-24 * sum_i |q_i k_i| (about
    1e-5 with keys x 20) into its weight, and values of order 1000 carry
    that into outputs that cancel to order 10; the elementwise figures are
    printed beside it.  (Far logits spread by more than about 87, the fp32
    exp range, underflow for the rows of a sub-chunk before the eviction
    that sets its post-sub-chunk max: there fp32 and the fp64 oracle part
    ways by the method's construction, so the key scale stops short of
    that.)"""
    kscale, vscale = 20.0, 1000.0
    banner(f"peaked softmax: k x {kscale:g}, v x {vscale:g}")
    cfg = synth.Config("scale", G=2, H=2, d=64, dv=64, ns=4, W=128, m=16, rows=400)
    host = synth.make_state(cfg)
    host.sink_k = (host.sink_k * kscale).astype(np.float32)
    host.sink_v = (host.sink_v * vscale).astype(np.float32)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    k = (k * kscale).astype(np.float32)
    v = (v * vscale).astype(np.float32)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q, k, v)
    orc = oracle.from_config(cfg, host)
    want = orc.step(q, k, v)
    assert np.all(np.isfinite(got))
    rowmax = np.max(np.abs(want), axis=2, keepdims=True)
    e = excess(got, want, atol=ATOL * vscale, scale=rowmax)
    ee = excess(got, want, atol=ATOL * vscale)
    rel = float(np.max(np.abs(got - want) / rowmax))
    print(f"  max |d| / max|out of its row and head| = {rel:.3e}  excess {e:.3e} "
          f"(elementwise: {ee:.3e})", flush=True)
    assert e <= 0, f"beyond the norm-wise tolerance by {e:.3e}"
    check_state(read_state(st), orc, vscale=vscale)


def test_resume_from_copied_state():
    banner("resume from a copied state")
    cfg = synth.SMALL.replace(rows=1500, W=256, m=16)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    a = _state(cfg, host)
    full = _prefill(cfg, a, q, k, v)
    b = _state(cfg, host)
    cut = 704  # a sub-chunk boundary: both runs then see the same sub-chunks
    first = _prefill(cfg, b, q[:cut], k[:cut], v[:cut])
    saved = {f: getattr(b, f).cpu() for f in swl.LayerState.FIELDS}
    c = swl.LayerState(b.geom, **{f: x.to("cuda") for f, x in saved.items()})
    rest = _prefill(cfg, c, q[cut:], k[cut:], v[cut:])
    # The far mass Z is a scan over the call's sub-chunks whose association
    # order depends on where the call starts, and Theta is carried with a
    # compensation term within a call but stored as one fp32 number between
    # calls, so Z, Theta (and through them the outputs) agree up to rounding;
    # the max M, the ring and meta are exact.
    np.testing.assert_allclose(np.concatenate([first, rest]), full, rtol=1e-6, atol=1e-7)
    sa, sc = read_state(a), read_state(c)
    for f in sa:
        if f == "mz":
            m = cfg.m
            za = sa[f].reshape(-1, 2, m)
            zc = sc[f].reshape(-1, 2, m)
            np.testing.assert_array_equal(za[:, 0], zc[:, 0])
            np.testing.assert_allclose(za[:, 1], zc[:, 1], rtol=1e-6, atol=0)
        elif f == "theta":
            scale = np.max(np.abs(sa[f]), axis=2, keepdims=True)
            assert np.all(np.abs(sa[f] - sc[f]) <= 1e-6 * scale), "Theta beyond rounding"
        else:
            np.testing.assert_array_equal(sa[f], sc[f])


def test_prefill_passes_match_one_long_call():
    """More rows than one prefill pass holds (32768) against the oracle."""
    cfg = synth.Config("long", G=1, H=2, d=32, dv=32, ns=4, W=512, m=8, rows=36000, rope=True,
                       landmark_scale=0.2)
    banner(f"long prefill T={cfg.rows}")
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, cfg.rows)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q, k, v)
    orc = oracle.from_config(cfg, host)
    want = orc.step(q, k, v)
    check_out(got, want)
    check_out(got[32768 - 70:32768 + 70], want[32768 - 70:32768 + 70], "rows around the pass boundary")
    check_state(read_state(st), orc)


# -- limits of the geometry ------------------------------------------------------------

def test_largest_heads_sinks_landmarks():
    """H = 16 query heads, ns = 256 sinks, m = 64 landmarks, three groups with
    windows 300 / 130 / 64 (not multiples of the tile sizes), a ragged
    777-row prompt, then tokens."""
    banner("limits: H=16 ns=256 m=64, windows 300/130/64")
    cfg = synth.Config("limits", G=3, H=16, d=64, dv=64, ns=256, W=300, m=64, rows=777,
                       windows=(300, 130, 64), rope=True, landmark_scale=0.125)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 777 + 24)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q[:777], k[:777], v[:777], poison=True)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    check_out(got, orc.step(q[:777], k[:777], v[:777]))
    check_state(read_state(st), orc)
    got_t = _tokens(cfg, st, q[777:], k[777:], v[777:])
    check_out(got_t, orc.step(q[777:], k[777:], v[777:]), "tokens")
    check_state(read_state(st), orc)


def test_many_groups():
    """G = 64 KV groups (the limit) of two heads, a prompt and tokens."""
    banner("limits: G=64")
    cfg = synth.Config("groups", G=64, H=2, d=16, dv=16, ns=2, W=40, m=8, rows=150)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 150 + 6)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q[:150], k[:150], v[:150])
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    check_out(got, orc.step(q[:150], k[:150], v[:150]))
    got_t = _tokens(cfg, st, q[150:], k[150:], v[150:])
    check_out(got_t, orc.step(q[150:], k[150:], v[150:]), "tokens")
    check_state(read_state(st), orc)


@pytest.mark.parametrize("d,H", [(64, 16), (256, 4)])
def test_more_landmark_tiles_than_waves(d, H):
    """A prompt of 64 sub-chunks in two groups, whose far-score launch keeps
    one block per sub-chunk (it already has 128), with more landmark-row
    tiles per group (H * m / 32) than the block has waves: each wave then
    scores several tiles, loading their query halves in turn."""
    banner(f"far score, tiles over waves: d={d} H={H} m=64, 4096 rows")
    cfg = synth.Config("tiles", G=2, H=H, d=d, dv=d, ns=4, W=128, m=64, rows=4096)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 4096)
    st = _state(cfg, host)
    got = _prefill(cfg, st, q, k, v, poison=True)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


@pytest.mark.parametrize("W,T", [(65536, 3000), (5000, 6000)])
def test_tokens_over_many_splits(W, T):
    """Decode with the window split into more than 64 partials per head (the
    merge folds them in several batches): the widest ring stride with a
    partial window, and a full 5000-key window."""
    banner(f"tokens over many splits: W={W} after {T} rows")
    cfg = synth.Config("splits", G=1, H=2, d=32, dv=32, ns=3, W=W, m=8, rows=T)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, T + 12)
    st = _state(cfg, host)
    _prefill(cfg, st, q[:T], k[:T], v[:T])
    orc = oracle.from_config(cfg, host)
    orc.step(q[:T], k[:T], v[:T], want=np.zeros(T, bool))
    got = _tokens(cfg, st, q[T:], k[T:], v[T:])
    check_out(got, orc.step(q[T:], k[T:], v[T:]), "tokens")
    check_state(read_state(st), orc)


def test_zero_rows_is_a_noop():
    cfg = synth.TINY
    host = synth.make_state(cfg)
    st = _state(cfg, host)
    before = read_state(st)
    t = torch()
    z = lambda *s: t.empty(s, dtype=t.float32, device="cuda")
    swl.swl_prefill(st, z(0, cfg.nh, cfg.d), z(0, cfg.G, cfg.d), z(0, cfg.G, cfg.dv),
                    z(0, cfg.nh, cfg.dv), swl.alloc_scratch(st.geom, 0))
    after = read_state(st)
    for f in before:
        np.testing.assert_array_equal(before[f], after[f])


def _tokens(cfg, st, q, k, v):
    t = torch()
    scratch = swl.alloc_scratch(st.geom, 1)
    scratch.view(t.float32)[: scratch.numel() // 4].fill_(float("nan"))
    n = q.shape[0]
    outs = t.empty((n, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    qd, kd, vd = dev(q), dev(k), dev(v)
    for i in range(n):
        swl.swl_attend_token(st, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], outs[i:i + 1], scratch)
    t.cuda.synchronize()
    return outs.cpu().numpy()


@pytest.mark.parametrize("head0", [0, 13])
def test_tokens_fill_then_evict(head0):
    """The one-row path from a ring 10/16 with an empty far field: the ring
    fills, the first eviction meets M = -inf, then every row evicts."""
    banner(f"tokens on the tiny layer, head0={head0}")
    cfg = synth.TINY.replace(head0=head0)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 40)
    st = _state(cfg, host)
    got = _tokens(cfg, st, q, k, v)
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


@pytest.mark.parametrize("rect", [False, True])
def test_tokens_windows_and_guard(rect):
    banner(f"tokens with per-group windows and mixed-sign mu, rect={rect}")
    cfg = synth.Config("tokw", G=2, H=3, d=64, dv=64, ns=3, W=20, m=16, rows=0,
                       windows=(12, 20), len0=0, rect=rect)
    host = synth.make_state(cfg)
    r = np.random.default_rng(5)
    host.mu = (r.standard_normal(host.mu.shape) / cfg.m).astype(np.float32)
    host.mu[1] = -np.abs(host.mu[1])
    q, k, v = synth.rows(cfg, 0, 70)
    st = _state(cfg, host)
    got = _tokens(cfg, st, q, k, v)
    orc = oracle.from_config(cfg, host)
    check_out(got, orc.step(q, k, v))
    check_state(read_state(st), orc)


def test_tokens_after_chunks_match_chunk_path():
    """Tokens and one-row chunks agree from the same state."""
    banner("tokens vs one-row chunks")
    cfg = synth.SMALL.replace(rows=1100, W=1024)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 1100)
    a = _state(cfg, host)
    _prefill(cfg, a, q[:1000], k[:1000], v[:1000])
    b = a.clone()
    got_t = _tokens(cfg, a, q[1000:], k[1000:], v[1000:])
    got_c = _chunks(cfg, b, q[1000:], k[1000:], v[1000:], [1] * 100)
    orc = oracle.from_config(cfg, host, threads=oracle_threads())
    orc.step(q[:1000], k[:1000], v[:1000], want=np.zeros(1000, bool))
    want = orc.step(q[1000:], k[1000:], v[1000:])
    check_out(got_t, want, "tokens")
    check_out(got_c, want, "chunks")
    check_state(read_state(a), orc)


def test_token_graph_replays_match_eager():
    """Tokens captured in a HIP graph, replayed several times with eager work
    in between, give the eager results every time."""
    banner("token path under HIP graph replay")
    t = torch()
    cfg = synth.SMALL.replace(rows=300, W=256, m=16)
    host = synth.make_state(cfg)
    q, k, v = synth.rows(cfg, 0, 300 + 8)
    base = _state(cfg, host)
    _prefill(cfg, base, q[:300], k[:300], v[:300])
    qd, kd, vd = dev(q[300:]), dev(k[300:]), dev(v[300:])
    n = 8
    # eager reference: three consecutive passes over the same 8 rows
    ref = base.clone()
    scr = swl.alloc_scratch(ref.geom, 1)
    want = []
    for rep in range(3):
        o = t.empty((n, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
        for i in range(n):
            swl.swl_attend_token(ref, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], o[i:i + 1], scr)
        want.append(o.cpu().numpy())
    want_state = read_state(ref)
    # the same three passes as replays of one captured pass
    st = base.clone()
    scr2 = swl.alloc_scratch(st.geom, 1)
    out = t.zeros((n, cfg.nh, cfg.dv), dtype=t.float32, device="cuda")
    swl.swl_attend_token(st.clone(), qd[0:1], kd[0:1], vd[0:1], out[0:1], scr2)   # first-call set-up
    t.cuda.synchronize()
    g = t.cuda.CUDAGraph()
    with t.cuda.graph(g):
        for i in range(n):
            swl.swl_attend_token(st, qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], out[i:i + 1], scr2)
    for rep in range(3):
        g.replay()
        t.cuda.synchronize()
        got = out.cpu().numpy()
        np.testing.assert_array_equal(got, want[rep])
        _ = (dev(np.ones(1000, np.float32)) * 2).sum().item()   # eager work between replays
    got_state = read_state(st)
    for f in want_state:
        np.testing.assert_array_equal(got_state[f], want_state[f])
