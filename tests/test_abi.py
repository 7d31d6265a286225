"""The C ABI on the host: the library loads, exports what include/swl.h
declares, and rejects bad arguments before it enqueues anything.

No call here reaches a kernel: every call is either pure host arithmetic
(swl_scratch_bytes, swl_status_str) or one that validation must refuse.
"""
import ctypes
import os
import re

import pytest

import sink_window_landmark_amd as swl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    text = open(os.path.join(ROOT, "include", "swl.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swl_[a-z_]+)\s*\(", text)))


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


# Calls that must fail validation get fake (never dereferenced) pointers;
# keep them off machines with a GPU so a validation bug cannot reach one.
needs_no_gpu = pytest.mark.skipif(_gpu_visible(), reason="fake-pointer checks run without a GPU")


def test_library_exports_every_declared_function():
    lib = swl.load_library()
    declared = _header_functions()
    assert set(declared) == set(swl.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name


GOOD = dict(G=2, H=4, m=32, W=1024, ns=4, d=128, dv=128)


def _geom(**kw):
    a = dict(GOOD)
    a.update(kw)
    return swl.Geom(**a)


def test_scratch_bytes_grows_then_caps():
    g = _geom()
    b1 = swl.swl_scratch_bytes(g, 1)
    b64 = swl.swl_scratch_bytes(g, 64)
    b65 = swl.swl_scratch_bytes(g, 65)
    assert 0 < b1 == b64 < b65
    assert swl.swl_scratch_bytes(g, 32768) == swl.swl_scratch_bytes(g, 10 ** 7)
    assert swl.swl_scratch_bytes(g, 0) == b1


@pytest.mark.parametrize("bad", [dict(G=0), dict(G=65), dict(H=0), dict(H=17), dict(m=0), dict(m=65),
                                 dict(W=0), dict(ns=-1), dict(ns=257), dict(d=24, dv=24),
                                 dict(d=64, dv=128), dict(d=512, dv=512), dict(rect=2),
                                 dict(scale=float("nan"))])
def test_invalid_geometry_has_no_scratch(bad):
    assert swl.swl_scratch_bytes(_geom(**bad), 64) == 0


def test_status_strings():
    lib = swl.load_library()
    assert lib.swl_status_str(0) == b"ok"
    assert lib.swl_status_str(1) == b"invalid argument"
    assert lib.swl_status_str(2) == b"HIP launch failed"
    assert b"static scratch" in lib.swl_status_str(3)


@needs_no_gpu
def test_noalloc_token_rejects_oversized_geometry_and_null_pointers():
    """The allocation-free token call refuses, before any HIP call, a geometry
    whose decode partials outgrow its static scratch (SWL_ESIZE), and null
    pointers (SWL_EINVAL)."""
    lib = swl.load_library()
    st = _fake_state()
    big = swl.Geom(G=64, H=16, m=8, W=65536, ns=4, d=128, dv=128).c()
    rc = lib.swl_attend_token_noalloc(ctypes.byref(big), ctypes.byref(st), FAKE, FAKE, FAKE, None,
                                      FAKE, None)
    assert rc == swl.SWL_ESIZE
    g = _geom().c()
    for args in ((None, FAKE, FAKE, FAKE), (FAKE, None, FAKE, FAKE), (FAKE, FAKE, None, FAKE),
                 (FAKE, FAKE, FAKE, None)):
        q, k, v, out = args
        rc = lib.swl_attend_token_noalloc(ctypes.byref(g), ctypes.byref(st), q, k, v, None, out,
                                          None)
        assert rc == swl.SWL_EINVAL
    rc = lib.swl_attend_token_noalloc(ctypes.byref(g), ctypes.byref(_fake_state(theta=True)),
                                      FAKE, FAKE, FAKE, None, FAKE, None)
    assert rc == swl.SWL_EINVAL


FAKE = 0x10000


def _fake_state(**null):
    vals = {f: (None if null.get(f) else FAKE) for f in swl.LayerState.FIELDS}
    return swl._State(*[vals[f] for f in swl.LayerState.FIELDS])


@needs_no_gpu
@pytest.mark.parametrize("rows", [0, -1, 65])
def test_attend_chunk_rejects_rows(rows):
    lib = swl.load_library()
    g = _geom().c()
    st = _fake_state()
    n = swl.swl_scratch_bytes(_geom(), 64)
    rc = lib.swl_attend_chunk(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, rows, FAKE,
                              FAKE, n, None)
    assert rc == swl.SWL_EINVAL
    rc = lib.swl_commit(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, rows, FAKE, n, None)
    assert rc == swl.SWL_EINVAL


@needs_no_gpu
def test_calls_reject_small_scratch_and_null_pointers():
    lib = swl.load_library()
    g = _geom().c()
    st = _fake_state()
    n = swl.swl_scratch_bytes(_geom(), 64)
    assert lib.swl_attend_chunk(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, 64, FAKE,
                                FAKE, n - 1, None) == swl.SWL_EINVAL
    assert lib.swl_attend_chunk(ctypes.byref(g), ctypes.byref(st), None, FAKE, FAKE, 64, FAKE,
                                FAKE, n, None) == swl.SWL_EINVAL
    n_big = swl.swl_scratch_bytes(_geom(), 1000)
    assert lib.swl_prefill(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, 1000, FAKE, FAKE,
                           n_big - 256, None) == swl.SWL_EINVAL
    assert lib.swl_prefill(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, -5, FAKE, FAKE,
                           n_big, None) == swl.SWL_EINVAL
    # zero rows is a no-op that needs nothing
    assert lib.swl_prefill(ctypes.byref(g), ctypes.byref(st), None, None, None, 0, None, None, 0,
                           None) == swl.SWL_OK
    for f in ("meta", "ring_k", "mz", "theta", "mu", "q_tilde", "k_tilde", "sink_k"):
        bad = _fake_state(**{f: True})
        assert lib.swl_attend_chunk(ctypes.byref(g), ctypes.byref(bad), FAKE, FAKE, FAKE, 64,
                                    FAKE, FAKE, n, None) == swl.SWL_EINVAL, f
    assert lib.swl_attend_token(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, FAKE, FAKE,
                                0, None) == swl.SWL_EINVAL
    assert lib.swl_commit_rows(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, -1, FAKE, n_big,
                               None) == swl.SWL_EINVAL
    assert lib.swl_commit_rows(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, 1000, FAKE,
                               n_big - 256, None) == swl.SWL_EINVAL
    assert lib.swl_commit_rows(ctypes.byref(g), ctypes.byref(st), None, FAKE, 10, FAKE, n_big,
                               None) == swl.SWL_EINVAL
    assert lib.swl_commit_rows(ctypes.byref(g), ctypes.byref(st), None, None, 0, None, 0,
                               None) == swl.SWL_OK


@needs_no_gpu
def test_init_rejects_window_wider_than_stride():
    lib = swl.load_library()
    g = _geom().c()
    st = _fake_state()
    win = (ctypes.c_uint32 * 2)(512, 1025)
    assert lib.swl_init_state(ctypes.byref(g), ctypes.byref(st), ctypes.cast(win, ctypes.c_void_p),
                              None) == swl.SWL_EINVAL
    bad = _geom(G=0).c()
    assert lib.swl_init_state(ctypes.byref(bad), ctypes.byref(st), None, None) == swl.SWL_EINVAL


@needs_no_gpu
def test_fused_calls_reject_a_gate_without_its_scale():
    lib = swl.load_library()
    g = _geom().c()
    st = _fake_state()
    n = swl.swl_scratch_bytes(_geom(), 64)
    bad = swl._Fuse(FAKE, FAKE, None)
    assert lib.swl_prefill_fused(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, 64,
                                 ctypes.byref(bad), FAKE, FAKE, n, None) == swl.SWL_EINVAL
    assert lib.swl_attend_chunk_fused(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, 64,
                                      ctypes.byref(bad), FAKE, FAKE, n, None) == swl.SWL_EINVAL
    assert lib.swl_attend_token_fused(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE,
                                      ctypes.byref(bad), FAKE, FAKE, n, None) == swl.SWL_EINVAL
    assert lib.swl_commit_fused(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, 64,
                                ctypes.byref(bad), FAKE, n, None) == swl.SWL_EINVAL
    assert lib.swl_commit_rows_fused(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, 64,
                                     ctypes.byref(bad), FAKE, n, None) == swl.SWL_EINVAL
    # the fused calls keep their plain counterparts' checks
    ok = swl._Fuse(FAKE, None, None)
    assert lib.swl_attend_chunk_fused(ctypes.byref(g), ctypes.byref(st), FAKE, FAKE, FAKE, 65,
                                      ctypes.byref(ok), FAKE, FAKE, n, None) == swl.SWL_EINVAL
    assert lib.swl_prefill_fused(ctypes.byref(g), ctypes.byref(st), None, None, None, 0,
                                 ctypes.byref(ok), None, None, 0, None) == swl.SWL_OK
