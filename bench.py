"""Benchmark of the sink + window + landmark layer on one MI355X.

A step is one pass of the whole hot path over the max-window workload
(4 KV groups x 4 query heads, d = dv = 128, 4 sinks, w = 2048, m = 64
landmarks): the empty state (swl_init_state), then a 32768-row prompt
through swl_prefill as 512 consecutive 64-row sub-chunks (far scores,
far scan, far accumulator, near attention, far readout, ring and meta
commit).  Inputs are synthetic (seeded N(0,1) with RoPE), already resident
in HBM when the timed region starts.

Prints one JSON line: prefill rows/s (whole job, one GPU), the near
kernel's achieved TFLOP/s against its matrix-core roofline (timed live with
HIP events around its launches): the near products, the far readout's
landmark scores and its far numerator run as three fp16 products of hi/lo
splits (2.5 PFLOP/s / 3 of fp32-accurate work), the far readout's u and
in-chunk coefficients on fp32 MFMA (157.3 TFLOP/s), the decode path's
us/token after the
32768-row prompt, the per-sub-chunk API's rate, an exact-attention timing
for context, and the CPU oracle timed on a bounded sample.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

MFMA_FP32_PEAK_TFLOPS = 157.3   # MI355X dense fp32 matrix
MFMA_FP16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix
# an fp32-accurate product from fp16 hi/lo splits takes three fp16 products
MFMA_SPLIT_PEAK_TFLOPS = MFMA_FP16_PEAK_TFLOPS / 3
HBM_PEAK_GBS = 8000.0           # MI355X HBM3E


def near_flops(cfg, T, len0=0):
    """Algorithmic near flops of T rows: each row and head scores and sums
    ns + min(w_g, len0 + i + 1) keys, 2d + 2dv flops each."""
    tot = 0
    r = np.arange(T, dtype=np.int64)
    for g in range(cfg.G):
        w = cfg.window(g)
        keys = cfg.ns + np.minimum(w, len0 + r + 1)
        tot += int(keys.sum()) * cfg.H * (2 * cfg.d + 2 * cfg.dv)
    return tot


def far_flops(cfg, T, len0=0, nfar0=0, split=False):
    """Algorithmic far flops of T rows: evicted-key scores and accumulator
    updates (2 d m H and 2 dv m H per evicted key and group), and per row and
    head with a non-empty far field: f (2 m d), u (2 m m), N (2 m dv) and the
    in-chunk terms (2 n (m + dv), n = rows of the sub-chunk evicted so far).
    With split=True the readout figure comes as (the part on fp16 splits:
    f, N and the in-chunk value terms 2 n dv; the part on fp32 MFMA: u and
    the in-chunk coefficients 2 n m)."""
    m, d, dv, H = cfg.m, cfg.d, cfg.dv, cfg.H
    fe = fc = ro = rf = 0
    for g in range(cfg.G):
        w = cfg.window(g)
        ln, nf = len0, nfar0
        for r0 in range(0, T, 64):
            k = min(64, T - r0)
            j0 = w - ln
            ev = max(0, k - max(j0, 0))
            fe += ev * 2 * d * m * H
            fc += ev * 2 * dv * m * H
            for i in range(k):
                n_in = max(0, i - max(j0, 0) + 1) if i >= j0 else 0
                if nf + n_in > 0:
                    ro += H * (2 * m * d + 2 * m * m + 2 * m * dv + 2 * n_in * (m + dv))
                    rf += H * (2 * m * d + 2 * m * dv + 2 * n_in * dv)
            tot = ln + k
            if tot > w:
                nf += tot - w
            ln = min(w, tot)
    if split:
        return fe, fc, (rf, ro - rf)
    return fe, fc, ro


def attend_bytes(cfg, T, len0=0):
    """Algorithmic HBM bytes of the near-attention + far-readout kernel over
    T rows, each input counted once per 64-row sub-chunk: the sinks and the
    ring rows it starts from, the chunk's own k and v, q in and out written,
    and the far readout's inputs (Theta before the sub-chunk, the exp-mass
    and prefix planes, and the per-landmark max, rescale and mass)."""
    G, H, d, dv, m, ns = cfg.G, cfg.H, cfg.d, cfg.dv, cfg.m, cfg.ns
    nh = G * H
    f = 0
    for g in range(G):
        w = cfg.window(g)
        ln = len0
        for r0 in range(0, T, 64):
            k = min(64, T - r0)
            f += (ns + ln) * (d + dv) + k * (d + dv)
            ln = min(w, ln + k)
    for r0 in range(0, T, 64):
        k = min(64, T - r0)
        f += k * nh * (d + dv) + nh * m * (dv + 2 * k + 3)
    return 4 * f


def source_sha256():
    """sha256 over every source of the HIP library (csrc/*.hip, *.h and the
    C ABI header), in name order: a profile summary taken on other sources
    does not describe the kernels that run."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sink_window_landmark_amd", "csrc")
    files = sorted(os.path.join(csrc, f) for f in os.listdir(csrc) if f.endswith((".hip", ".h")))
    files.append(os.path.join(ROOT, "include", "swl.h"))
    for f in files:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + b"\0" + fh.read())
    return h.hexdigest()


def profile_values(name):
    """The `key = value` lines of a committed profile summary, or None when
    it is missing or was taken on other library sources."""
    try:
        text = open(os.path.join(ROOT, "profiles", name)).read()
    except OSError:
        return None
    kv = {}
    for line in text.splitlines():
        if " = " in line and not line.startswith(("    ", "|")):
            k, v = line.split(" = ", 1)
            kv[k.strip().strip("`")] = v.strip().strip("`")
    if kv.get("source_sha256") != source_sha256():
        return None
    return kv


def attend_counters(launch_bytes):
    """HBM traffic of one attend launch from the committed counter summary,
    or None when the library's sources have changed since it was taken."""
    kv = profile_values("attend_maxwin_counters.md")
    if kv is None:
        return None
    read = float(kv["fetch_kib_per_launch"]) * float(kv["fetch_factor"]) * 1024
    write = float(kv["write_kib_per_launch"]) * float(kv["write_factor"]) * 1024
    return dict(bytes=read + write, read_bytes=read, write_bytes=write,
                vs_algorithmic=(read + write) / launch_bytes,
                source="profiles/attend_maxwin_counters.md (rocprofv3 FETCH_SIZE and WRITE_SIZE, "
                       "scaled by a 256 MiB copy)")


def decode_bytes(cfg):
    """Algorithmic HBM bytes of one decode token at a full window: the
    group's sinks and window K/V, the far skeleton (k~, q~, mu, M/Z, Theta
    read and Theta/M/Z written), q/k/v in, out and the pushed row written."""
    G, H, d, dv, m, ns = cfg.G, cfg.H, cfg.d, cfg.dv, cfg.m, cfg.ns
    nh = G * H
    f = 0
    for g in range(G):
        f += (ns + cfg.window(g)) * (d + dv)
    f += G * m * d + nh * m * d + nh * m * m + nh * 2 * m * 2 + nh * m * dv * 2
    f += nh * d + G * (d + dv) + nh * dv + G * (d + dv)
    return 4 * f


def run_gpu(args, cfg):
    import torch
    import synth
    import sink_window_landmark_amd as swl

    dev = "cuda"
    T = cfg.rows
    geom = swl.Geom(cfg.G, cfg.H, cfg.m, cfg.W, cfg.ns, cfg.d, cfg.dv)
    host = synth.make_state(cfg)
    st = swl.LayerState.from_host(geom, host, device=dev)
    nd = args.decode_steps
    qh, kh, vh = synth.rows(cfg, 0, T + nd)
    q = torch.from_numpy(qh[:T]).to(dev)
    k = torch.from_numpy(kh[:T]).to(dev)
    v = torch.from_numpy(vh[:T]).to(dev)
    out = torch.empty((T, cfg.nh, cfg.dv), dtype=torch.float32, device=dev)
    scratch = swl.alloc_scratch(geom, T, device=dev)
    windows = cfg.meta_windows()

    stage_ev = []   # (stage, start_event, end_event) of the timed steps
    recording = [False]

    def on_stage(name, begin):
        if not recording[0]:
            return
        ev = torch.cuda.Event(enable_timing=True)
        ev.record()
        if begin:
            stage_ev.append([name, ev, None])
        else:
            stage_ev[-1][2] = ev

    def step():
        swl.swl_init_state(st, windows)
        swl.swl_prefill(st, q, k, v, out, scratch)

    def traced_step():
        swl.swl_init_state(st, windows)
        swl.swl_prefill_traced(st, q, k, v, out, scratch, on_stage)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the headline: K steps with nothing else on the stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    for _ in range(args.steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    # then K more steps with an event pair around each launch (the stage
    # times and the attention kernel's launch time come from these)
    recording[0] = True
    for _ in range(args.steps):
        traced_step()
    torch.cuda.synchronize()
    recording[0] = False
    stages = {}
    for name, a, b in stage_ev:
        stages.setdefault(name, []).append(a.elapsed_time(b))
    near_ms = stages["attend"]
    near_launch_ms = float(np.mean(near_ms))
    near_step_flops = near_flops(cfg, T)
    fe, fc, ro = far_flops(cfg, T)
    launches_per_step = len(near_ms) / args.steps
    # the attend kernel computes the near part and the far readout
    near_flops_per_launch = (near_step_flops + ro) / launches_per_step
    achieved = near_flops_per_launch / (near_launch_ms * 1e-3) / 1e12
    # the kernel's peak for its own mix: the near products and the readout's
    # split parts at the split rate, its u and in-chunk coefficients at the
    # fp32 rate
    _, _, (ro_s, ro_32) = far_flops(cfg, T, split=True)
    t_peak = ((near_step_flops + ro_s) / MFMA_SPLIT_PEAK_TFLOPS + ro_32 / MFMA_FP32_PEAK_TFLOPS) / launches_per_step
    peak = near_flops_per_launch / t_peak
    near_bytes_per_launch = attend_bytes(cfg, T) / launches_per_step
    step_flops = near_step_flops + fe + fc + ro

    res = dict(
        value=T * args.steps / (ms_total * 1e-3),
        ms_per_step=ms_per_step,
        wall_s=wall,
        stages_ms_per_step={n: float(np.sum(x)) / args.steps for n, x in stages.items()},
        near=dict(avg_launch_ms=near_launch_ms, launches_per_step=launches_per_step,
                  flops_per_launch=near_flops_per_launch, achieved_tflops=achieved,
                  peak_tflops=peak, near_flops_per_launch=near_step_flops / launches_per_step,
                  readout_flops_per_launch=ro / launches_per_step,
                  bytes_per_launch=near_bytes_per_launch),
        step_flops=step_flops,
        step_tflops=step_flops / (ms_per_step * 1e-3) / 1e12,
    )

    # decode: one row at a time after the 32768-row prompt (the state left by
    # the last timed step), through swl_attend_token.  Timed two ways: a host
    # loop through the Python binding, and HIP-graph replays of captured
    # 256-token segments (the GPU time of the path, without Python).
    if nd > 0:
        qd = torch.from_numpy(qh[T:]).to(dev)
        kd = torch.from_numpy(kh[T:]).to(dev)
        vd = torch.from_numpy(vh[T:]).to(dev)
        od = torch.empty((nd, cfg.nh, cfg.dv), dtype=torch.float32, device=dev)
        tscr = swl.alloc_scratch(geom, 1, device=dev)
        views = [(qd[i:i + 1], kd[i:i + 1], vd[i:i + 1], od[i:i + 1]) for i in range(nd)]
        sh = torch.cuda.current_stream().cuda_stream
        nw = min(16, nd)
        for i in range(nw):
            swl.swl_attend_token(st, *views[i], tscr, stream=sh)
        torch.cuda.synchronize()
        d0, d1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        d0.record()
        for i in range(nw, nd):
            swl.swl_attend_token(st, *views[i], tscr, stream=sh)
        d1.record()
        torch.cuda.synchronize()
        us_host = d0.elapsed_time(d1) * 1e3 / (nd - nw)
        seg = min(256, nd)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            gs = torch.cuda.current_stream().cuda_stream
            for i in range(seg):
                swl.swl_attend_token(st, *views[i], tscr, stream=gs)
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, (nd - nw) // seg)
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g0.record()
        for _ in range(reps):
            graph.replay()
        g1.record()
        torch.cuda.synchronize()
        us = g0.elapsed_time(g1) * 1e3 / (reps * seg)
        db = decode_bytes(cfg)
        res["decode"] = dict(tokens=reps * seg, us_per_token=us, timing="HIP graph replay of "
                             f"{seg}-token segments", us_per_token_host_loop=us_host,
                             bytes_per_token=db, achieved_gbs=db / (us * 1e-6) / 1e9,
                             frac_hbm=db / (us * 1e-6) / 1e9 / HBM_PEAK_GBS)
        if args.cold_states > 0:
            res["decode"]["cold"] = decode_cold(args, cfg, st, views[:seg], tscr, db)
        res["decode"]["launch_floor_us"] = launch_floor_us()

    # the fused ingest and output steps: the same prompt through
    # swl_prefill_fused with q, k taken before RoPE (a cos/sin table row per
    # prompt row) and the sigmoid output gate (pre-activations per output
    # element, a scale per head and column)
    if args.fused:
        tab = torch.from_numpy(synth.rope_table(np.arange(T), cfg.d)).to(dev)
        zh, sh_ = synth.gate_inputs(cfg, 0, T)
        z = torch.from_numpy(zh).to(dev)
        gsc = torch.from_numpy(sh_).to(dev)
        del zh

        def fstep():
            swl.swl_init_state(st, windows)
            swl.swl_prefill_fused(st, q, k, v, out, scratch, rope=tab, gate=z, gate_scale=gsc)

        for _ in range(max(1, args.warmup)):
            fstep()
        torch.cuda.synchronize()
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        f0.record()
        for _ in range(args.steps):
            fstep()
        f1.record()
        torch.cuda.synchronize()
        fms = f0.elapsed_time(f1) / args.steps
        res["fused"] = dict(ms_per_step=fms, rows_per_s=T / (fms * 1e-3),
                            vs_plain_step=fms / ms_per_step,
                            extra_bytes_per_step=(tab.numel() + z.numel() + gsc.numel()) * 4,
                            what="swl_prefill_fused: q, k before RoPE (table rows) and the "
                                 "sigmoid output gate, fused into the kernels")
        del tab, z, gsc

    # the per-sub-chunk API (attend_chunk + commit per 64 rows), for comparison
    if args.chunk_api:
        cscr = swl.alloc_scratch(geom, 64, device=dev)
        swl.swl_init_state(st, windows)
        torch.cuda.synchronize()
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for r0 in range(0, T, 64):
            sl = slice(r0, min(T, r0 + 64))
            swl.swl_attend_chunk(st, q[sl], k[sl], v[sl], out[sl], cscr)
            swl.swl_commit(st, k[sl], v[sl], cscr)
        c1.record()
        torch.cuda.synchronize()
        res["chunk_api_rows_per_s"] = T / (c0.elapsed_time(c1) * 1e-3)

    if args.exact:
        res["exact_attention"] = exact_attention(cfg, host, q, k, v)
    return res


def decode_cold(args, cfg, st, views, tscr, db):
    """us/token with the state out of every cache: token i of a captured
    segment runs on state copy i mod N (N byte copies of the prefilled
    state, every array its own), so that the other N - 1 states' ~10 MB
    each pass through the caches between two visits to one state (N = 32:
    ~330 MB, above the 256 MB Infinity Cache)."""
    import torch
    import sink_window_landmark_amd as swl
    n = args.cold_states
    states = [st.clone() for _ in range(n)]
    state_bytes = sum(getattr(st, f).numel() * 4 for f in swl.LayerState.FIELDS)
    seg = len(views)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        gs = torch.cuda.current_stream().cuda_stream
        for i in range(seg):
            swl.swl_attend_token(states[i % n], *views[i], tscr, stream=gs)
    graph.replay()
    torch.cuda.synchronize()
    reps = 8
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    us = a.elapsed_time(b) * 1e3 / (reps * seg)
    del graph, states
    torch.cuda.empty_cache()
    return dict(us_per_token=us, states=n, bytes_rotated=n * state_bytes,
                achieved_gbs=db / (us * 1e-6) / 1e9, frac_hbm=db / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                timing=f"HIP graph replay of {seg}-token segments, token i on state copy i mod {n}")


def launch_floor_us():
    """The time of two dependent launches of a trivial kernel (a one-element
    add), per pair, under HIP-graph replay: the floor of any two-launch
    token path on this GPU and runtime."""
    import torch
    x = torch.zeros(1, device="cuda")
    seg = 256
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(seg):
            x.add_(1.0)
            x.add_(1.0)
    graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(8):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (8 * seg)


def exact_attention(cfg, host, q, k, v):
    """Exact fp32 causal softmax attention over sinks + every key, same heads,
    blockwise torch.matmul (for the "faster than exact" comparison only)."""
    import torch
    T, G, H, d = q.shape[0], cfg.G, cfg.H, cfg.d
    sk = torch.from_numpy(host.sink_k).to(q.device)      # [G][ns][d]
    sv = torch.from_numpy(host.sink_v).to(q.device)
    Q = q.permute(1, 0, 2).contiguous()                    # [nh][T][d]
    K = torch.cat([sk, k.permute(1, 0, 2)], dim=1)         # [G][ns+T][d]
    V = torch.cat([sv, v.permute(1, 0, 2)], dim=1)
    K = K.repeat_interleave(H, dim=0).contiguous()         # [nh][ns+T][d]
    V = V.repeat_interleave(H, dim=0).contiguous()
    Kt = K.transpose(1, 2).contiguous()                    # [nh][d][ns+T]
    out = torch.empty_like(Q)
    B = 2048
    ns = cfg.ns

    def run():
        for b0 in range(0, T, B):
            b1 = min(T, b0 + B)
            nk = ns + b1
            s = torch.matmul(Q[:, b0:b1], Kt[:, :, :nk]) * cfg.scale
            rows = torch.arange(b0, b1, device=q.device)[:, None]
            cols = torch.arange(nk, device=q.device)[None, :] - ns
            s.masked_fill_(cols > rows, float("-inf"))
            p = torch.softmax(s, dim=-1)
            out[:, b0:b1] = torch.matmul(p, V[:, :nk])

    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    run()
    e1.record()
    torch.cuda.synchronize()
    return dict(ms=e0.elapsed_time(e1), backend="torch.matmul fp32 blockwise + softmax",
                rows=T)


def _oracle_rate(cfg, fill, batch, budget_s, threads):
    """Rows/s of the oracle on `cfg` after `fill` rows stepped without
    outputs: rows with outputs in batches of `batch` until ~budget_s."""
    import oracle
    import synth
    host = synth.make_state(cfg)
    orc = oracle.from_config(cfg, host, threads=threads)
    if fill:
        q, k, v = synth.rows(cfg, 0, fill)
        orc.step(q, k, v, want=np.zeros(fill, bool))
    done, r0 = 0, fill
    el = 0.0
    while el < budget_s:
        q, k, v = synth.rows(cfg, r0, r0 + batch)
        ts = time.perf_counter()
        orc.step(q, k, v)
        el += time.perf_counter() - ts
        done += batch
        r0 += batch
    return done / el, done, el, orc.threads


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, budget_s):
    """The oracle (float64 serial steps, threads = min(G*H, cores, 16)) on
    the max-window layer: the ring is filled (2048 rows, no outputs), then
    rows with outputs are stepped in 256-row batches for ~budget_s (timed:
    the stepping only).  Beside it, bounded samples of the other workloads:
    the tiny layer's 64-row chunk and the small layer at a full window,
    each also on one thread, and the mixed-window layer once every window
    is full; a decode token is one serial row step at the max-window layer's
    full window, so its us/token is the inverse of the main rate."""
    import synth
    cores = min(cfg.nh, os.cpu_count() or 1, 16)
    fill = max(cfg.window(g) for g in range(cfg.G))
    rate, done, el, thr = _oracle_rate(cfg, fill, 256, budget_s, cores)
    per = {}
    for name, c, fl, batch, bud, single in (
            ("tiny", synth.TINY, 0, 64, 1.0, True),
            ("small", synth.SMALL, synth.SMALL.W, 256, 2.0, True),
            ("mixed", synth.MIXED, synth.MIXED.W, 256, 3.0, False)):
        r, n, e, t = _oracle_rate(c, fl, batch, bud, min(c.nh, cores))
        per[name] = dict(rows_per_s=r, threads=t, rows=n, seconds=e,
                         sample=f"rows {fl}..{fl + n}" + (" (full window)" if fl else
                                                          " from its 10/16 ring, in 64-row chunks"))
        if single:
            r1, n1, e1, _ = _oracle_rate(c, fl, batch, bud, 1)
            per[name]["rows_per_s_1_thread"] = r1
    per["maxwin"] = dict(rows_per_s=rate, threads=thr)
    per["decode"] = dict(us_per_token=1e6 / rate, threads=thr,
                         sample="a token is one serial row step at the max-window layer's full "
                                "window: the inverse of the max-window rate")
    return dict(value=rate, unit="rows/s", cores=thr, kind="oracle",
                sample=f"max-window layer rows {fill}..{fill + done} (full window, every row "
                       f"evicting), after a {fill}-row fill; {el:.1f} s of stepping",
                cpu_model=cpu_model(), host_cores=os.cpu_count(), per_config=per)


def hbm_copy_gbs():
    """Achievable HBM bandwidth on this GPU: a 1 GiB device-to-device copy
    (read + write counted), best of 10 after 2 warm-up copies."""
    import torch
    a = torch.empty(256 << 20, dtype=torch.float32, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    best = float("inf")
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1))
    gbs = 2 * a.numel() * 4 / (best * 1e-3) / 1e9
    del a, b
    torch.cuda.empty_cache()
    return gbs


def other_configs(args):
    """The other workloads of the layer, timed through the same entry points:
    the tiny layer's one 64-row chunk from its 10/16 ring (attend_chunk +
    commit, the state restored between repetitions outside the timed
    region), the small layer's 4096-row prompt and the mixed-window layer's
    131072-row prompt from the empty state (swl_init_state + swl_prefill)."""
    import torch
    import synth
    import sink_window_landmark_amd as swl

    dev = "cuda"
    res = {}

    def tensors(cfg, T):
        q, k, v = synth.rows(cfg, 0, T)
        return [torch.from_numpy(x).to(dev) for x in (q, k, v)]

    # tiny: one chunk, latency per call pair
    cfg = synth.TINY
    geom = swl.Geom(cfg.G, cfg.H, cfg.m, cfg.W, cfg.ns, cfg.d, cfg.dv)
    host = synth.make_state(cfg)
    st = swl.LayerState.from_host(geom, host, device=dev)
    saved = {n: getattr(st, n).clone() for n in ("meta", "ring_k", "ring_v", "mz", "theta")}
    q, k, v = tensors(cfg, cfg.rows)
    out = torch.empty((cfg.rows, cfg.nh, cfg.dv), dtype=torch.float32, device=dev)
    scr = swl.alloc_scratch(geom, cfg.rows, device=dev)
    times = []
    for rep in range(25):
        for n, t in saved.items():
            getattr(st, n).copy_(t)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        swl.swl_attend_chunk(st, q, k, v, out, scr)
        swl.swl_commit(st, k, v, scr)
        b.record()
        torch.cuda.synchronize()
        if rep >= 5:
            times.append(a.elapsed_time(b) * 1e3)
    res["tiny"] = dict(us_per_chunk=float(np.median(times)), rows=cfg.rows,
                       what="attend_chunk + commit of one 64-row chunk, median of 20")

    for cfg, steps in ((synth.SMALL, 10), (synth.MIXED, 3)):
        T = cfg.rows
        geom = swl.Geom(cfg.G, cfg.H, cfg.m, cfg.W, cfg.ns, cfg.d, cfg.dv)
        st = swl.LayerState.from_host(geom, synth.make_state(cfg), device=dev)
        q, k, v = tensors(cfg, T)
        out = torch.empty((T, cfg.nh, cfg.dv), dtype=torch.float32, device=dev)
        scr = swl.alloc_scratch(geom, T, device=dev)
        windows = cfg.meta_windows()

        def step():
            swl.swl_init_state(st, windows)
            swl.swl_prefill(st, q, k, v, out, scr)

        step()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(steps):
            step()
        b.record()
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / steps
        fl = near_flops(cfg, T) + sum(far_flops(cfg, T))
        tf = fl / (ms * 1e-3) / 1e12
        res[cfg.name] = dict(ms_per_prompt=ms, rows=T, rows_per_s=T / (ms * 1e-3),
                             algorithmic_tflops=tf, frac_split_peak=tf / MFMA_SPLIT_PEAK_TFLOPS,
                             windows=[cfg.window(g) for g in range(cfg.G)])
        del q, k, v, out, scr, st
        torch.cuda.empty_cache()
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--cold-states", type=int, default=32,
                    help="state copies the cold decode figure rotates over (0: skip it)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-exact", dest="exact", action="store_false")
    ap.add_argument("--no-chunk-api", dest="chunk_api", action="store_false")
    ap.add_argument("--no-fused", dest="fused", action="store_false",
                    help="skip the fused RoPE + gate prefill leg")
    ap.add_argument("--no-configs", dest="configs", action="store_false",
                    help="skip the tiny, small and mixed-window workloads")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 256 MiB device-to-device copy (the reference kernel "
                         "for scaling HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this layer runs on a single MI355X here "
              "(no multi-GPU path is built); run it with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import synth
    cfg = synth.MAXWIN
    if args.calibrate_copy:
        import torch
        a = torch.ones(64 << 20, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    res = run_gpu(args, cfg)
    near = res["near"]
    line = {
        "metric": "prefill rows/sec per layer (64-row chunks) at w=2048; µs/token decode; % roofline",
        "value": res["value"],
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "mfma_dtype": "f16 hi/lo splits (three products per fp32-accurate product, f32 accumulation) "
                      "for the near part, the landmark and evicted-key scores and the accumulator "
                      "increments, the far readout's landmark scores and far numerator; f32 for the far "
                      "readout's u and in-chunk coefficients",
        "data": "synthetic",
        "config": {"workload": "max-window layer: 4 KV groups x 4 query heads, d=dv=128, 4 sinks, "
                               "w=2048, m=64 landmarks, 32768-row prompt from the empty state as "
                               "64-row sub-chunks (swl_init_state + swl_prefill)",
                   "rows_per_step": cfg.rows},
        "roofline": {"bound": "mfma", "kernel": "k_attend<128,2> (near attention + far readout)",
                     "achieved": near["achieved_tflops"], "peak": near["peak_tflops"],
                     "unit": "TFLOP/s", "frac": near["achieved_tflops"] / near["peak_tflops"],
                     "peak_basis": "near flops and the far readout's landmark scores and far numerator "
                                   "at 2500/3 TFLOP/s (fp16 MFMA, three split products per fp32-accurate "
                                   "product), its u and in-chunk coefficients at 157.3 TFLOP/s (fp32 MFMA)",
                     "near_flops_per_launch": near["near_flops_per_launch"],
                     "readout_flops_per_launch": near["readout_flops_per_launch"],
                     "traffic": None,
                     "avg_launch_ms": near["avg_launch_ms"],
                     "flops_per_launch": near["flops_per_launch"],
                     "algorithmic_bytes_per_launch": near["bytes_per_launch"]},
        "step": {"algorithmic_flops": res["step_flops"], "tflops": res["step_tflops"],
                 "frac_split_peak": res["step_tflops"] / MFMA_SPLIT_PEAK_TFLOPS,
                 "stages_ms": res["stages_ms_per_step"]},
    }
    rf = line["roofline"]
    rf["frac_dense_fp16"] = near["achieved_tflops"] / MFMA_FP16_PEAK_TFLOPS
    kt = profile_values("prefill_maxwin_kernel_trace.md")
    if kt is not None and "attend_avg_ns" in kt:
        traced_ms = float(kt["attend_avg_ns"]) * 1e-6
        ach = near["flops_per_launch"] / (traced_ms * 1e-3) / 1e12
        rf["traced"] = dict(avg_launch_ms=traced_ms, achieved=ach, frac=ach / near["peak_tflops"],
                            frac_dense_fp16=ach / MFMA_FP16_PEAK_TFLOPS,
                            source="profiles/prefill_maxwin_kernel_trace.md (rocprofv3 kernel "
                                   "trace of the same command)")
    tr = attend_counters(near["bytes_per_launch"])
    if tr is not None:
        line["roofline"]["traffic"] = tr["bytes"]
        line["roofline"]["traffic_detail"] = tr
    copy_gbs = hbm_copy_gbs()
    line["hbm_copy_gbs"] = copy_gbs
    if "decode" in res:
        line["decode"] = res["decode"]
        line["decode"]["frac_copy_bandwidth"] = res["decode"]["achieved_gbs"] / copy_gbs
    if "fused" in res:
        line["fused"] = res["fused"]
    if "chunk_api_rows_per_s" in res:
        line["chunk_api_rows_per_s"] = res["chunk_api_rows_per_s"]
    if "exact_attention" in res:
        line["exact_attention"] = res["exact_attention"]
    if args.configs:
        line["other_configs"] = other_configs(args)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
