"""The C ABI: the library loads, exports every declared symbol, and rejects bad arguments
on the host (status codes, nothing launched).  Runs without a GPU: every call here fails
validation before touching the device."""
import ctypes
import os
import re

import pytest

import draft_verify_sampling_step_amd as ds

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "dspark.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dspark_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    names = _declared()
    assert {"dspark_draft_markov", "dspark_confidence", "dspark_schedule", "dspark_verify",
            "dspark_accept_rate_tv", "dspark_workspace_bytes"} <= set(names)
    L = ds.lib()
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version():
    L = ds.lib()
    for s in range(7):
        assert L.dspark_status_string(s).startswith(b"DSPARK_")
    assert L.dspark_version() >= 100


def _dims(B=4, G=4, V=1024, r=16, d=64):
    return ds.Dims(B, G, V, r, d)


P = ctypes.c_void_p(256)   # a non-null pointer; never dereferenced on these error paths


def _draft(dm, temp=1.0, wdt=0, ws=P, ws_bytes=1 << 30, U=P):
    return ds.lib().dspark_draft_markov(ctypes.byref(dm) if dm is not None else None, U, P, P,
                                        wdt, P, None, temp, 1, P, P, P, ws, ws_bytes, None)


def test_draft_argument_validation():
    assert _draft(None) == 1
    assert _draft(_dims(), U=None) == 1
    for bad in (_dims(B=0), _dims(G=0), _dims(G=65), _dims(V=1), _dims(r=12), _dims(r=0),
                _dims(V=(1 << 28) + 1), _dims(B=70000)):
        assert _draft(bad) == 2
    assert _draft(_dims(), wdt=7) == 3
    for t in (0.0, -1.0, float("inf"), float("nan")):
        assert _draft(_dims(), temp=t) == 4
    assert _draft(_dims(), ws=None) == 5
    assert _draft(_dims(), ws_bytes=16) == 5


def test_schedule_argument_validation():
    L = ds.lib()
    assert L.dspark_schedule(4, 4, None, P, 0, P, P, P, None, 0, None) == 1
    assert L.dspark_schedule(0, 4, P, P, 0, P, P, P, None, 0, None) == 2
    assert L.dspark_schedule(4097, 1, P, P, 0, P, P, P, None, 0, None) == 2
    assert L.dspark_schedule(4, 4, P, P, 2, P, P, P, None, 0, None) == 4


def test_schedule_topk_argument_validation():
    L = ds.lib()
    assert L.dspark_schedule_topk(4, 4, None, P, 3, P, P, P, None, 0, None) == 1
    assert L.dspark_schedule_topk(4, 4, P, P, 3, None, P, P, None, 0, None) == 1
    assert L.dspark_schedule_topk(0, 4, P, P, 3, P, P, P, None, 0, None) == 2
    assert L.dspark_schedule_topk(4, 65, P, P, 3, P, P, P, None, 0, None) == 2
    assert L.dspark_schedule_topk(4097, 1, P, P, 3, P, P, P, None, 0, None) == 2
    assert L.dspark_schedule_topk(4, 4, P, P, -1, P, P, P, None, 0, None) == 4


def test_sts_and_calibrated_confidence_validation():
    L = ds.lib()
    ws = 1 << 30
    assert L.dspark_sts_calibrate(100, 4, None, P, P, 8, 15, P, P, P, ws, None) == 1
    assert L.dspark_sts_calibrate(100, 4, P, P, P, 8, 15, P, None, P, ws, None) == 1
    assert L.dspark_sts_calibrate(0, 4, P, P, P, 8, 15, P, P, P, ws, None) == 2
    assert L.dspark_sts_calibrate((1 << 22) + 1, 4, P, P, P, 8, 15, P, P, P, ws, None) == 2
    assert L.dspark_sts_calibrate(100, 65, P, P, P, 8, 15, P, P, P, ws, None) == 2
    assert L.dspark_sts_calibrate(100, 4, P, P, P, 0, 15, P, P, P, ws, None) == 2
    assert L.dspark_sts_calibrate(100, 4, P, P, P, 8, 257, P, P, P, ws, None) == 2
    need = L.dspark_sts_workspace_bytes(100, 8, 15)
    assert need >= 100 * 8 + 8 * 15 * 3 * 8
    assert L.dspark_sts_calibrate(100, 4, P, P, P, 8, 15, P, P, P, need - 1, None) == 5
    assert L.dspark_sts_calibrate(100, 4, P, P, P, 8, 15, P, P, None, need, None) == 5
    dm = _dims()
    assert L.dspark_confidence_calibrated(ctypes.byref(dm), P, 0, P, 0, P, 0, P, P, None, P,
                                          None) == 1


def test_draft_loss_validation():
    L = ds.lib()
    ws = 1 << 30
    f = L.dspark_draft_loss
    assert f(2, 4, 100, None, P, P, P, 0.1, 0.9, 1.0, P, None, P, P, P, ws, None) == 1
    assert f(2, 4, 100, P, P, P, P, 0.1, 0.9, 1.0, None, None, P, P, P, ws, None) == 1
    assert f(0, 4, 100, P, P, P, P, 0.1, 0.9, 1.0, P, None, P, P, P, ws, None) == 2
    assert f(2, 65, 100, P, P, P, P, 0.1, 0.9, 1.0, P, None, P, P, P, ws, None) == 2
    assert f(2, 4, (1 << 22) + 1, P, P, P, P, 0.1, 0.9, 1.0, P, None, P, P, P, ws, None) == 2
    assert f(2, 4, 100, P, P, P, P, float("nan"), 0.9, 1.0, P, None, P, P, P, ws, None) == 4
    assert f(2, 4, 100, P, P, P, P, 0.1, float("inf"), 1.0, P, None, P, P, P, ws, None) == 4
    need = L.dspark_loss_workspace_bytes(2, 4, 100)
    assert need >= 8 * (6 + 1) * 8 + 8 * 2 * 4
    assert L.dspark_loss_workspace_bytes(2, 4, 0) == 0
    assert f(2, 4, 100, P, P, P, P, 0.1, 0.9, 1.0, P, None, P, P, P, need - 1, None) == 5
    assert f(2, 4, 100, P, P, P, P, 0.1, 0.9, 1.0, P, None, P, P, None, need, None) == 5
    # the vocabulary is split into ceil(V / 8192) chunks of published partials per row
    assert L.dspark_loss_workspace_bytes(128, 16, 151936) >= 2048 * 19 * 6 * 8


def test_closed_loop_validation():
    L = ds.lib()
    dm = _dims()
    ws = 1 << 34
    f = L.dspark_closed_loop

    def call(dims=ctypes.byref(dm), U=P, anchor=P, rounds=3, sigma=0.5, temp=1.0, mode=0,
             wsb=ws, tokens=P):
        return f(dims, U, P, P, 1, P, 1, P, 1, anchor, P, mode, temp, 1, sigma, 2, rounds,
                 None, tokens, P, P, None, P, P, P, None, P, wsb, None)
    assert call(U=None) == 1
    assert call(tokens=None) == 1
    assert call(rounds=0) == 2
    assert call(rounds=65537) == 2
    assert call(sigma=-1.0) == 4
    assert call(sigma=float("nan")) == 4
    assert call(temp=0.0) == 4
    assert call(mode=7) == 4
    assert call(mode=-1) == 4
    # the scheduler's candidate limit is checked before anything is enqueued
    big = _dims(B=128, G=64)
    assert call(dims=ctypes.byref(big), wsb=1 << 40) == 2
    need = L.dspark_loop_workspace_bytes(ctypes.byref(dm))
    assert need >= dm.batch * (dm.gamma + 1) * dm.vocab * 4
    assert call(wsb=need - 1) == 5


def test_verify_confidence_tv_validation():
    L = ds.lib()
    dm = _dims()
    assert L.dspark_verify(ctypes.byref(dm), P, P, P, 0, P, P, P, P, None, P, 1.0, 1, P, P,
                           None, P, 1 << 30, None) == 1
    assert L.dspark_verify(ctypes.byref(dm), P, P, P, 0, P, P, P, P, P, P, 0.0, 1, P, P, None,
                           P, 1 << 30, None) == 4
    assert L.dspark_verify(ctypes.byref(dm), P, P, P, 0, P, P, P, P, P, P, 1.0, 1, P, P, None,
                           P, 8, None) == 5
    assert L.dspark_confidence(ctypes.byref(dm), P, 0, P, 0, P, 3, P, P, P, None) == 3
    assert L.dspark_confidence(ctypes.byref(dm), None, 0, P, 0, P, 0, P, P, P, None) == 1
    assert L.dspark_accept_rate_tv(ctypes.byref(dm), P, P, P, 0, P, P, P, P, -2.0, P, P,
                                   1 << 30, None) == 4
    assert L.dspark_rng_uniforms(1, 0, 1, 0, 0, -5, P, None) == 2


def test_workspace_sizes_are_consistent():
    L = ds.lib()
    for (B, G, V, r) in [(4, 4, 1024, 16), (1, 16, 151936, 256), (128, 16, 151936, 256),
                         (256, 5, 129280, 256), (64, 16, 262144, 256)]:
        for op in (ds.OP_DRAFT, ds.OP_VERIFY, ds.OP_TV):
            n = ds.workspace_bytes(op, B, G, V, r)
            assert n > 0 and n % 256 == 0
        assert ds.workspace_bytes(ds.OP_SCHEDULE, B, G, V, r) == 0
        assert ds.workspace_bytes(ds.OP_CONFIDENCE, B, G, V, r) == 0
    assert ds.workspace_bytes(0, 0, 4, 1024, 16) == 0        # invalid dims -> 0
    assert ds.workspace_bytes(9, 4, 4, 1024, 16) == 0        # unknown op -> 0


def test_binding_fails_loudly_without_library(monkeypatch):
    monkeypatch.setattr(ds, "_lib", None)
    monkeypatch.setattr(ds, "LIB_PATH", "/nonexistent/libdspark.so")
    with pytest.raises(RuntimeError, match="missing"):
        ds.lib()


def test_noalloc_draft_validation_and_size_limit():
    """The allocation-free draft validates like the draft and refuses, before touching the
    device, a shape whose scratch exceeds its 32 MiB array."""
    L = ds.lib()

    def call(dm, temp=1.0, wdt=1, U=P):
        return L.dspark_draft_markov_noalloc(ctypes.byref(dm) if dm is not None else None, U,
                                             P, P, wdt, P, None, temp, 1, P, P, P, None)
    assert call(None) == 1
    assert call(_dims(), U=None) == 1
    assert call(_dims(B=0)) == 2
    assert call(_dims(), wdt=5) == 3
    assert call(_dims(), temp=-1.0) == 4
    # 256 requests, 64 positions on the matrix-core path: 64 x 256 slices x 256 x 8 bytes
    assert call(ds.Dims(256, 64, 151936, 256, 0)) == 5


def test_gumbel_lattice_validation():
    L = ds.lib()
    assert L.dspark_gumbel_lattice(0, None, None) == 1
    assert L.dspark_gumbel_lattice(2, P, None) == 4
    assert L.dspark_gumbel_lattice(-1, P, None) == 4


def test_profile_switch_validation():
    import ctypes
    L = ds.lib()
    assert L.dspark_profile_start(0) == 4            # DSPARK_E_VALUE, no HIP call made
    assert L.dspark_profile_start(1 << 17) == 4
    assert L.dspark_profile_stop(None, None, None) == 1    # DSPARK_E_NULL


def test_stream_read_probe_validation():
    import ctypes
    L = ds.lib()
    ms = ctypes.c_double()
    buf = ctypes.c_void_p(4096)      # never dereferenced: validation fails first
    sink = ctypes.c_void_p(8192)
    assert L.dspark_stream_read_probe(None, 64, 16, 1, sink, ctypes.byref(ms), None) == 1
    assert L.dspark_stream_read_probe(buf, 64, 16, 1, None, ctypes.byref(ms), None) == 1
    assert L.dspark_stream_read_probe(buf, 64, 16, 1, sink, None, None) == 1
    assert L.dspark_stream_read_probe(buf, 64, 24, 1, sink, ctypes.byref(ms), None) == 2
    assert L.dspark_stream_read_probe(buf, 64, 128, 1, sink, ctypes.byref(ms), None) == 2
    assert L.dspark_stream_read_probe(ctypes.c_void_p(4100), 64, 16, 1, sink,
                                      ctypes.byref(ms), None) == 2
    assert L.dspark_stream_read_probe(buf, 64, 16, 0, sink, ctypes.byref(ms), None) == 4
    assert L.dspark_stream_read_probe(buf, 64, 16, 10001, sink, ctypes.byref(ms), None) == 4
