"""The draft entry point that allocates nothing, dspark_draft_markov_noalloc (its scratch is
the library's static device array): called through the C ABI, its outputs equal those of
dspark_draft_markov with a caller workspace bit for bit, call after call, with each next
call on a smaller input (the array keeps the previous call's contents), on the matrix-core
and the row paths, free-running and teacher-forced."""
import ctypes

import numpy as np
import pytest
import torch

import draft_verify_sampling_step_amd as ds
import workload
from gpu_round import DeviceInputs

pytestmark = pytest.mark.gpu

CASES = {
    # matrix-core path (16-column kernel), 8.4 MB of the array at gamma = 16
    "mfma_b128_v151936": workload.custom(name="na_big", B=128, gamma=16, V=151936, r=256, d=8,
                                         bf16=True, logits="zipf", table="serve"),
    # matrix-core path with fewer requests and a smaller vocabulary
    "mfma_b40_v5000": workload.custom(name="na_mid", B=40, gamma=3, V=5000, r=256, d=8,
                                      bf16=True, wsigma=0.1, logits="zipf", table="serve"),
    # row path, fp32 weights
    "rows_b3_v1000": workload.custom(name="na_rows", B=3, gamma=5, V=1000, r=8, d=8),
}


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _noalloc_c_abi(D, cfg, seed, forced):
    """One call of dspark_draft_markov_noalloc through ctypes, outputs pre-filled with junk."""
    B, G, V = cfg.B, cfg.gamma, cfg.V
    tok = torch.full((B, G), -7, dtype=torch.int32, device="cuda")
    logp = torch.full((B, G), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((B, G), float("nan"), dtype=torch.float32, device="cuda")
    dm = ds.Dims(B, G, V, cfg.r, 0)
    wdt = ds.BF16 if cfg.bf16 else ds.F32
    st = torch.cuda.current_stream().cuda_stream
    rc = ds.lib().dspark_draft_markov_noalloc(
        ctypes.byref(dm), _p(D.U), _p(D.W1), _p(D.W2t), wdt, _p(D.anchor), _p(forced),
        float(cfg.temperature), int(seed), _p(tok), _p(logp), _p(lse), ctypes.c_void_p(st))
    assert rc == 0, ds.lib().dspark_status_string(rc)
    return tok, logp, lse


def _check(name, seed, forced_too):
    cfg = CASES[name]
    print(f"noalloc draft {name} seed {seed}", flush=True)
    inp = workload.generate(cfg, seed)
    D = DeviceInputs(inp)
    ref = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed)
    got = _noalloc_c_abi(D, cfg, inp.seed, None)
    torch.cuda.synchronize()
    for what, a, b in zip(("tokens", "logp", "lse"), ref, got):
        assert torch.equal(a, b), f"{name}: {what} differs from the workspace draft"
    if forced_too:
        forced = torch.roll(ref[0], 1, dims=1).contiguous()
        ref_f = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed,
                                       forced=forced)
        got_f = _noalloc_c_abi(D, cfg, inp.seed, forced)
        torch.cuda.synchronize()
        for what, a, b in zip(("tokens", "logp", "lse"), ref_f, got_f):
            assert torch.equal(a, b), f"{name} forced: {what} differs"


def test_noalloc_draft_equals_the_workspace_draft_call_after_call():
    _check("mfma_b128_v151936", 1, True)
    _check("mfma_b40_v5000", 2, True)     # smaller than the call before, same array
    _check("rows_b3_v1000", 3, True)      # smaller again, the row path
    _check("mfma_b40_v5000", 4, False)


def test_noalloc_draft_in_a_graph_replays_like_eager():
    """Captured in a HIP graph (it allocates nothing and clears with a kernel), every replay
    equals the eager call."""
    cfg = CASES["mfma_b40_v5000"]
    inp = workload.generate(cfg, 5)
    D = DeviceInputs(inp)
    out = tuple(torch.empty((cfg.B, cfg.gamma), dtype=dt, device="cuda")
                for dt in (torch.int32, torch.float32, torch.float32))
    ref = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        ds.dspark_draft_markov_noalloc(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed,
                                       out=out)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ds.dspark_draft_markov_noalloc(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed,
                                       out=out)
    for i in range(3):
        for t in out:
            t.fill_(-3)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, out):
            assert torch.equal(a, b), f"replay {i}"
        # eager work on the same array between replays
        _check("rows_b3_v1000", 6 + i, False)
    del g
