"""Helpers of the GPU parity tests: run the library on seeded inputs and compare with the
oracle to the stated tolerances.

Protocol (no oracle input ever comes from the HIP path):
  * the oracle drafts freely; the GPU drafts with the oracle's tokens as teacher-forced
    prefix, so every position is compared on the same conditioning token;
  * sampled tokens must match except where the oracle's top-2 Gumbel-score gap is below
    1e-4 (an excused near-tie; these are counted);
  * probabilities (p_d(x), p_t(x), c, alpha) match to 1e-4 relative; lse to 1e-4 absolute
    (a relative 1e-4 on exp(lse));
  * scheduler and accept decisions given identical inputs are bit-exact; an accept test is
    excused only if the oracle's margin |u p_d - p_t| / p_t is below 1e-5.

The oracle is plain single-threaded C called through ctypes, which releases the
interpreter lock, so the helpers below split the requests over a thread pool (threads of
this process: nothing is forked from a process that has touched the GPU).  Every request
keys its random numbers with its global id, so a split reproduces the whole batch.
"""
from __future__ import annotations

import concurrent.futures
import os

import numpy as np

import draft_verify_sampling_step_amd as ds
import oracle
import workload

REL = 1e-4          # relative tolerance on probabilities
GAP_TIE = 1e-4      # near-tie threshold on the oracle's top-2 score gap
MARGIN_TIE = 1e-5   # accept-test decisions within this relative margin are excused

# Session-wide tally, reported in the pytest terminal summary:
#   samples          sampled tokens compared (draft tokens and final verify tokens)
#   flagged          of those, the oracle's top-2 gap is below GAP_TIE (a near-tie)
#   excused          of the flagged, the GPU's token differs from the oracle's
#   accept_tests     accept decisions compared
#   accept_flagged   of those, the oracle's margin is below MARGIN_TIE
#   accept_excused   of the flagged, the GPU decided otherwise
TALLY = {"samples": 0, "flagged": 0, "excused": 0, "accept_tests": 0, "accept_flagged": 0,
         "accept_excused": 0}


def dev(a):
    return ds.to_device(a)


def host(t):
    return t.detach().cpu().numpy()


def workers() -> int:
    """Oracle threads: the host's cores, at most 16 (the share of one GPU on a box)."""
    return max(1, min(16, os.cpu_count() or 1))


def compare_tokens(gpu, ref, gap, what):
    gpu = np.asarray(gpu)
    ref = np.asarray(ref)
    gap = np.asarray(gap)
    mism = gpu != ref
    bad = mism & (gap >= GAP_TIE)
    assert not bad.any(), (
        f"{what}: {int(bad.sum())} token mismatches with oracle gap >= {GAP_TIE}: "
        f"at {np.argwhere(bad)[:5].tolist()} gpu {gpu[bad][:5]} ref {ref[bad][:5]} "
        f"gap {gap[bad][:5]}")
    TALLY["samples"] += int(mism.size)
    TALLY["flagged"] += int((gap < GAP_TIE).sum())
    TALLY["excused"] += int(mism.sum())
    return mism


def assert_rel(gpu, ref, what, rel=REL, mask=None):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        gpu, ref = gpu[mask], ref[mask]
    err = np.abs(gpu - ref) / np.maximum(np.abs(ref), 1e-300)
    assert np.all(err <= rel), (
        f"{what}: max rel err {err.max():.3e} at {np.argmax(err)} "
        f"(gpu {gpu.flat[np.argmax(err)]!r} ref {ref.flat[np.argmax(err)]!r})")
    return float(err.max()) if err.size else 0.0


def assert_abs(gpu, ref, what, tol, mask=None):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if mask is not None:
        gpu, ref = gpu[mask], ref[mask]
    err = np.abs(gpu - ref)
    assert np.all(err <= tol), f"{what}: max abs err {err.max():.3e}"
    return float(err.max()) if err.size else 0.0


class DeviceInputs:
    """The round's inputs resident on the GPU."""

    def __init__(self, inp: workload.RoundInputs):
        self.inp = inp
        self.U = dev(inp.U)
        self.W1 = dev(inp.W1)
        self.W2t = dev(inp.W2t)
        self.h = dev(inp.h)
        self.w = dev(inp.w)
        self.anchor = dev(inp.anchor)
        self.sps = dev(inp.sps)


# ------------------------------------------------------------------------------------
# the oracle over many requests, on a thread pool
# ------------------------------------------------------------------------------------
def _split(rows, parts):
    rows = np.asarray(rows)
    parts = max(1, min(parts, rows.size))
    return [c for c in np.array_split(rows, parts) if c.size]


def _pool_map(fn, chunks):
    if len(chunks) == 1:
        return [fn(chunks[0])]
    with concurrent.futures.ThreadPoolExecutor(max_workers=workers()) as ex:
        return list(ex.map(fn, chunks))


def _weights64(inp):
    return oracle.widen(inp.W1), oracle.widen(inp.W2t)


def par_draft(inp, rows=None, forced=None):
    """oracle.draft for the requests `rows` (default all), keyed by their global ids.
    `forced` [B][gamma] (indexed by request) teacher-forces the prefix.  Returns the
    oracle's dict with one row per entry of `rows`."""
    cfg = inp.cfg
    rows = np.arange(cfg.B) if rows is None else np.asarray(rows)
    W1, W2t = _weights64(inp)

    def one(r):
        return oracle.draft(inp.U[r], W1, W2t, inp.anchor[r], cfg.temperature, inp.seed,
                            forced=None if forced is None else np.asarray(forced)[r], gid=r)

    parts = _pool_map(one, _split(rows, 4 * workers()))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def par_confidence(inp, tokens_by_row, rows=None):
    rows = np.arange(inp.cfg.B) if rows is None else np.asarray(rows)
    return oracle.confidence(inp.h[rows], inp.W1, inp.w, inp.anchor[rows], tokens_by_row)


def par_verify(inp, tokens, T_rows, ell, rows=None):
    """oracle.verify for `rows`: tokens and ell indexed by request, T_rows by position in
    `rows` (T_rows[i] is request rows[i])."""
    cfg = inp.cfg
    rows = np.arange(cfg.B) if rows is None else np.asarray(rows)
    W1, W2t = _weights64(inp)
    tokens = np.asarray(tokens)
    ell = np.asarray(ell)
    pos = {int(b): i for i, b in enumerate(rows)}

    def one(r):
        ti = np.array([pos[int(b)] for b in r])
        return oracle.verify(inp.U[r], W1, W2t, inp.anchor[r], tokens[r], T_rows[ti], ell[r],
                             cfg.temperature, inp.seed, gid=r)

    parts = _pool_map(one, _split(rows, 4 * workers()))
    return {k: np.concatenate([p[k] for p in parts]) for k in parts[0]}


def par_accept_tv(inp, tokens, T_rows, rows=None):
    cfg = inp.cfg
    rows = np.arange(cfg.B) if rows is None else np.asarray(rows)
    W1, W2t = _weights64(inp)
    tokens = np.asarray(tokens)
    pos = {int(b): i for i, b in enumerate(rows)}

    def one(r):
        ti = np.array([pos[int(b)] for b in r])
        return oracle.accept_tv(inp.U[r], W1, W2t, inp.anchor[r], tokens[r], T_rows[ti],
                                cfg.temperature)

    parts = _pool_map(one, _split(rows, 4 * workers()))
    return (np.concatenate([p[0] for p in parts]), np.concatenate([p[1] for p in parts]))


def check_verify(inp, tokens_ref, T, ell, gpu_n, gpu_out, gpu_pt, rows=None, rel=REL):
    """Compare GPU verification outputs with the oracle for `rows` (default: all).
    T holds either every request or exactly the requests `rows`, in that order."""
    cfg = inp.cfg
    rows = np.arange(cfg.B) if rows is None else np.asarray(rows)
    T_rows = T if T.shape[0] == len(rows) else T[rows]
    ref = par_verify(inp, tokens_ref, T_rows, ell, rows)
    n_g = np.asarray(gpu_n)[rows]
    out_g = np.asarray(gpu_out)[rows]
    pt_g = np.asarray(gpu_pt)[rows]
    # p_t(x_k) for k <= ell_b
    G = cfg.gamma
    kmask = np.arange(G)[None, :] < ell[rows][:, None]
    assert_rel(pt_g, ref["pt_tok"], "p_t(x_k)", rel=rel, mask=kmask)
    assert np.all(np.isnan(pt_g[~kmask])), "p_t beyond ell must be NaN"
    for i, b in enumerate(rows):
        n_r = int(ref["n_accept"][i])
        n_gb = int(n_g[i])
        tests = min(n_r + 1, int(ell[b]))
        TALLY["accept_tests"] += tests
        TALLY["accept_flagged"] += int(np.sum(ref["margin"][i][:tests] < MARGIN_TIE))
        if n_gb != n_r:
            # only a decision inside the rounding margin may differ
            kdec = min(n_gb, n_r)     # 0-based index of the first differing test
            m = ref["margin"][i][kdec]
            assert m < MARGIN_TIE, (f"request {b}: n_accept gpu {n_gb} ref {n_r}, "
                                    f"oracle margin {m:.3e}")
            TALLY["accept_excused"] += 1
            continue
        assert np.array_equal(out_g[i][:n_r], ref["out_tokens"][i][:n_r])
        assert np.all(out_g[i][n_r + 1:] == -1)
        y_g, y_r = out_g[i][n_r], ref["out_tokens"][i][n_r]
        compare_tokens(np.array([y_g]), np.array([y_r]), np.array([ref["gap"][i]]),
                       f"request {b} final token (kind {ref['kind'][i]})")
    return ref
