"""GPU parity: the HIP library against the fp64 oracle on seeded inputs.

Small shapes compare every output element.  The multi-tile shapes do the same at
V = 131072, where every matrix-core workgroup streams 8 or 16 vocabulary tiles, so the
steady state of the tile pipeline (its prefetch ring, waits and register rotation) is
compared element by element, with weights large enough (s.d. 0.5, a bias of s.d. about 4)
that a stale tile would move the normaliser and the tokens.  The workload configurations
at full size run in the benchmark's launch configuration and compare every request (the
oracle runs on a thread pool).  See tests/gpu_round.py for the protocol and tolerances.
"""
import dataclasses

import numpy as np
import pytest
import torch

import draft_verify_sampling_step_amd as ds
import oracle
import workload
from gpu_round import (REL, TALLY, DeviceInputs, assert_abs, assert_rel, check_verify,
                       compare_tokens, dev, host, par_accept_tv, par_draft)

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


# ------------------------------------------------------------------------------------
# random numbers
# ------------------------------------------------------------------------------------
@pytest.mark.parametrize("seed,b,k,s,v0,n", [
    (0, 0, 1, 0, 0, 1 << 20),
    (0xD5A4005EED0000, 127, 16, 0, 150000, 1936),
    (0x0123456789ABCDEF, 3, 5, 1, 0, 4),
    (2**64 - 1, 65535, 64, 2, 262100, 44),
    (77, 9, 2, 2, 7, 100003),
])
def test_rng_bit_exact(seed, b, k, s, v0, n):
    _flush(f"rng seed={seed} b={b} k={k} s={s} v0={v0} n={n}")
    g = host(ds.dspark_rng_uniforms(seed, b, k, s, v0, n))
    o = oracle.uniforms(seed, b, k, s, v0, n).astype(np.float32)
    assert np.array_equal(g, o)


@pytest.mark.parametrize("form", [0, 1])
def test_gumbel_transform_on_the_whole_lattice(form):
    """The kernels' fp32 Gumbel transform on all 2^23 uniforms u = (2m + 1) 2^-24 against
    fp64: within 3 * 2^-23 * (1 + |value|) everywhere, including u -> 1 where the largest
    scores (the winners of the races) come from.  Form 0 is -ln(-ln u) (row kernels),
    form 1 is -log2(-log2 u) (matrix-core kernels)."""
    g = host(ds.dspark_gumbel_lattice(form)).astype(np.float64)
    m = np.arange(1 << 23, dtype=np.float64)
    u = (2.0 * m + 1.0) * 2.0 ** -24
    e = -np.log1p(u - 1.0)                       # -ln u, exact argument (u - 1 is exact)
    exact = -np.log(e) if form == 0 else -np.log2(e / np.log(2.0))
    err = np.abs(g - exact)
    ratio = err / (3 * 2.0 ** -23 * (1.0 + np.abs(exact)))
    i = int(np.argmax(ratio))
    tail = err[-(1 << 16):]                      # the u closest to 1
    _flush(f"gumbel form {form}: max abs err {err.max():.3e}, max err/bound {ratio.max():.3f} "
           f"at u={u[i]!r} (value {exact[i]:.6f}); max abs err over the top 2^16 u "
           f"{tail.max():.3e}")
    assert np.all(np.isfinite(g))
    assert ratio.max() <= 1.0, (err[i], exact[i], u[i])


# ------------------------------------------------------------------------------------
# whole round, every element, small shapes
# ------------------------------------------------------------------------------------
def run_round_parity(cfg, seed=0, extra_ells=True):
    _flush(f"round parity cfg={cfg} seed={seed}")
    inp = workload.generate(cfg, seed)
    D = DeviceInputs(inp)
    temp = cfg.temperature
    od = par_draft(inp)
    tok_o = od["tokens"]
    forced = dev(tok_o)
    tg, lg, sg = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, temp, inp.seed,
                                        forced=forced)
    tg_h, lg_h, sg_h = host(tg), host(lg), host(sg)
    mism = compare_tokens(tg_h, tok_o, od["gap"], "draft tokens")
    # the logits' fp32 error (the rank-r bias is accumulated in fp32) is divided by the
    # temperature: below T = 1 the tolerances on lse and probabilities scale by 1/T
    tscale = max(1.0, 1.0 / temp)
    assert_abs(sg_h, od["lse"], "draft lse", 1e-4 * tscale)
    assert_rel(np.exp(lg_h.astype(np.float64)), np.exp(od["logp"]), "p_d(x_k)",
               rel=REL * tscale, mask=~mism)

    # free-running draft: identical to the forced one up to (and including) the first
    # position whose token differs from the oracle's
    tf, lf, sf = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, temp, inp.seed)
    tf_h, lf_h, sf_h = host(tf), host(lf), host(sf)
    for b in range(cfg.B):
        diff = np.nonzero(tf_h[b] != tok_o[b])[0]
        m = diff[0] + 1 if diff.size else cfg.gamma
        assert np.array_equal(tf_h[b, :m], tg_h[b, :m])
        assert np.array_equal(lf_h[b, :m], lg_h[b, :m])
        assert np.array_equal(sf_h[b, :m], sg_h[b, :m])

    c_o = oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tok_o)
    c_g = host(ds.dspark_confidence(D.h, D.W1, D.w, D.anchor, forced))
    assert_rel(c_g, c_o, "confidence")

    c32 = c_o.astype(np.float32)
    ell_o, th_o, n_o = oracle.schedule(c32, inp.sps, cfg.sched_mode)
    ell_g, th_g, n_g = ds.dspark_schedule(dev(c32), D.sps, cfg.sched_mode)
    assert np.array_equal(host(ell_g), ell_o)
    assert host(th_g)[0] == th_o and host(n_g)[0] == n_o

    T = workload.synthesize_target(inp, tok_o)
    Td = dev(T)
    ells = [ell_o]
    if extra_ells:
        ells += [np.full(cfg.B, cfg.gamma, np.int32),
                 (np.arange(cfg.B) % (cfg.gamma + 1)).astype(np.int32)]
    for ell in ells:
        n_g, out_g, pt_g = ds.dspark_verify(D.U, D.W1, D.W2t, D.anchor, forced, lg, sg, Td,
                                            dev(ell), temp, inp.seed)
        check_verify(inp, tok_o, T, ell, host(n_g), host(out_g), host(pt_g),
                     rel=REL * tscale)

    if cfg.tv:
        a_o, l1 = par_accept_tv(inp, tok_o, T)
        a_g = host(ds.dspark_accept_rate_tv(D.U, D.W1, D.W2t, D.anchor, forced, sg, Td, temp))
        assert_rel(a_g, a_o, "TV accept rate", rel=REL * tscale)
    torch.cuda.synchronize()


SMALL = {
    "tiny": workload.CONFIGS["tiny"],
    "tiny_t07_ragged": workload.custom(B=3, gamma=5, V=1000, r=8, d=40, temperature=0.7),
    "fp32_odd_vocab": workload.custom(B=5, gamma=3, V=4099, r=24, d=33, wsigma=0.3),
    "bf16_rows_b1": workload.custom(B=1, gamma=6, V=3001, r=64, d=96, bf16=True, wsigma=0.2,
                                    logits="zipf", sigma0=0.3, sigma1=0.05, table="serve"),
    "bf16_rows_b16": workload.custom(B=16, gamma=4, V=2048, r=256, d=64, bf16=True,
                                     wsigma=0.1, logits="zipf", table="serve"),
    "gamma1_v2": workload.custom(B=2, gamma=1, V=2, r=8, d=8),
    "no_hidden_d0": workload.custom(B=4, gamma=3, V=500, r=16, d=0),   # h empty: W1 part only
    # the longest draft (gamma = 64: one decision lane per row, 65 output slots), on the
    # row kernels and on the resident draft
    "gamma64_rows": workload.custom(B=2, gamma=64, V=300, r=8, d=8, wsigma=0.3,
                                    logits="zipf", table="serve"),
    "gamma64_resident": workload.custom(B=3, gamma=64, V=1024, r=256, d=16, bf16=True,
                                        wsigma=0.3, logits="zipf", table="serve"),
    # gamma = 64 at 64 requests: 4096 candidates, the scheduler's limit; the 4-wave draft
    # kernel, 32 TV launches
    "gamma64_b64_mfma": workload.custom(B=64, gamma=64, V=2048, r=256, d=16, bf16=True,
                                        wsigma=0.3, logits="zipf", table="serve"),
    # the largest rank (row kernels) and a wide hidden state with odd d, so the confidence
    # head's bf16 rows are not 16-byte aligned (element loads, several batches of rounds)
    "wide_r1024_d5001": workload.custom(B=3, gamma=3, V=700, r=1024, d=5001, bf16=True,
                                        wsigma=0.05, logits="zipf", table="serve"),
    "wide_r1024_fp32": workload.custom(B=2, gamma=2, V=513, r=1024, d=4608, wsigma=0.05),
    # a vocabulary of 2^22 + 3 entries (row kernels; every index past 2^22)
    "huge_vocab_fp32": workload.custom(B=2, gamma=2, V=(1 << 22) + 3, r=8, d=8, wsigma=0.3,
                                       logits="zipf", table="serve"),
    "mfma_b32": workload.custom(B=32, gamma=3, V=3072, r=256, d=128, bf16=True, wsigma=0.1,
                                logits="zipf", table="serve"),
    # the 32-column matrix-core kernels below 32 columns: one request with V % 4 != 0 (no
    # resident or streaming kernel for it), and 20 requests (draft, residual and TV)
    "mfma_b1_v_odd": workload.custom(B=1, gamma=5, V=3001, r=256, d=64, bf16=True,
                                     wsigma=0.3, logits="zipf", table="serve"),
    "mfma_b20": workload.custom(B=20, gamma=3, V=4096, r=256, d=64, bf16=True, wsigma=0.3,
                                logits="zipf", sigma_mix=True, table="serve"),
    "mfma_b40_ragged": workload.custom(B=40, gamma=4, V=5000, r=256, d=64, bf16=True,
                                       wsigma=0.1, logits="zipf", sigma_mix=True,
                                       table="serve"),
    "mfma_b64_v_odd": workload.custom(B=64, gamma=3, V=4099, r=256, d=64, bf16=True,
                                      wsigma=0.1, temperature=0.7, table="serve15"),
    "mfma_b128": workload.custom(B=128, gamma=3, V=2500, r=256, d=64, bf16=True, wsigma=0.1,
                                 logits="peaked_flat", table="serve"),
    # 16-column-wave draft kernel with idle columns inside the last waves, ragged last tile
    "mfma_b100_ragged": workload.custom(B=100, gamma=3, V=3004, r=256, d=64, bf16=True,
                                        wsigma=0.1, logits="zipf", sigma_mix=True,
                                        table="serve"),
    "mfma_b200_t07": workload.custom(B=200, gamma=2, V=1100, r=256, d=48, bf16=True,
                                     wsigma=0.1, temperature=0.7, table="serve15"),
    # temperature extremes on the matrix-core path: sharply peaked and nearly flat
    "mfma_b64_t005": workload.custom(B=64, gamma=3, V=3000, r=256, d=16, bf16=True,
                                     wsigma=0.3, temperature=0.05, logits="zipf",
                                     table="serve"),
    "mfma_b64_t5": workload.custom(B=64, gamma=3, V=3000, r=256, d=16, bf16=True, wsigma=0.3,
                                   temperature=5.0, logits="zipf", table="serve"),
    "mfma_b256": workload.custom(B=256, gamma=2, V=1600, r=256, d=64, bf16=True, wsigma=0.1,
                                 logits="zipf", table="serve"),
    "mfma_b300": workload.custom(B=300, gamma=2, V=1100, r=256, d=32, bf16=True, wsigma=0.1,
                                 table="serve"),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_round_parity(name):
    run_round_parity(SMALL[name], seed=3)


def test_round_parity_second_seed():
    run_round_parity(SMALL["mfma_b40_ragged"], seed=11, extra_ells=False)


# V = 131072 is 4096 tiles of 32 rows: 8 tiles per workgroup for 33-128 columns (512
# workgroups), 16 for 32 or more than 128 columns (256 workgroups).
MULTI_TILE = {
    # 16-column draft kernel, 4-wave workgroups (up to 64 requests); TV over 192 columns
    # (two launches)
    "mt_b64_g3": workload.custom(name="mt_b64_g3", B=64, gamma=3, V=131072, r=256, d=64,
                                 bf16=True, wsigma=0.5, logits="zipf", sigma_mix=True,
                                 table="serve"),
    # ... with 24 idle columns (the last wave has none live) and a ragged last tile
    "mt_b40_v131076": workload.custom(name="mt_b40_v131076", B=40, gamma=2, V=131076, r=256,
                                      d=64, bf16=True, wsigma=0.5, logits="peaked_flat",
                                      table="serve"),
    # 16-column draft kernel, 8-wave workgroups with 28 idle columns, a ragged last tile
    # (V % 32 == 4: one run of four live rows) and workgroups of 8 and 9 steps
    "mt_b100_v131076": workload.custom(name="mt_b100_v131076", B=100, gamma=2, V=131076,
                                       r=256, d=64, bf16=True, wsigma=0.5, logits="zipf",
                                       table="serve"),
    # 16-column draft kernel, 16-wave workgroups; TV over 400 columns (the last 16 on the
    # 32-column kernel)
    "mt_b200_g2_t07": workload.custom(name="mt_b200_g2_t07", B=200, gamma=2, V=131072, r=256,
                                      d=48, bf16=True, wsigma=0.5, temperature=0.7,
                                      table="serve15"),
    # 32-column kernel (one column block), V % 4 != 0: scalar logit loads, ragged last tile
    "mt_b32_odd": workload.custom(name="mt_b32_odd", B=32, gamma=2, V=131075, r=256, d=64,
                                  bf16=True, wsigma=0.5, logits="zipf", table="serve"),
    # 32-column kernel with eight column blocks (more than 128 requests, V % 4 != 0)
    "mt_b150_odd": workload.custom(name="mt_b150_odd", B=150, gamma=2, V=131073, r=256,
                                   d=64, bf16=True, wsigma=0.5, logits="peaked_flat",
                                   table="serve"),
    # the resident draft for few requests: one workgroup per compute unit, 32 blocks of 16
    # rows each, all in accumulation registers
    "mt_gemv_b3_g4": workload.custom(name="mt_gemv_b3", B=3, gamma=4, V=131072, r=256, d=64,
                                     bf16=True, wsigma=0.5, logits="zipf", sigma_mix=True,
                                     table="serve"),
    # ... with 7 or 8 blocks per workgroup in LDS and a ragged last block (V % 16 == 4)
    "mt_res_b5_v160004": workload.custom(name="mt_res_b5", B=5, gamma=3, V=160004, r=256,
                                         d=64, bf16=True, wsigma=0.5, logits="zipf",
                                         table="serve"),
    # ... at its largest vocabulary (40 blocks per workgroup, 8 in LDS) and 16 requests
    "mt_res_b16_v163840": workload.custom(name="mt_res_b16", B=16, gamma=2, V=163840, r=256,
                                          d=64, bf16=True, wsigma=0.5, logits="peaked_flat",
                                          table="serve"),
    # beyond the resident draft's vocabulary: two requests on the 32-column matrix-core
    # kernels (30 idle columns; residual and TV passes too)
    "mt_b2_v262144": workload.custom(name="mt_b2_v262144", B=2, gamma=3, V=262144, r=256,
                                     d=64, bf16=True, wsigma=0.5, logits="peaked_flat",
                                     table="serve"),
    # ... and one request on the streaming kernel: two 224-row chunks per workgroup (more
    # than 768 chunks)
    "mt_gemv_b1_v262144": workload.custom(name="mt_gemv_b1", B=1, gamma=3, V=262144, r=256,
                                          d=64, bf16=True, wsigma=0.5, logits="zipf",
                                          table="serve"),
    # the row kernels (fp32 weights, r = 64): slices of 1280 rows, i.e. a step of four
    # 256-row tiles and a step of one, one Philox call per four rows; the last slice ends
    # one row into its third tile, and the target-row pass (V % 4 != 0) ends on a one-entry
    # slice
    "mt_rows_fp32_b16_odd": workload.custom(name="mt_rows_fp32", B=16, gamma=2, V=131073,
                                            r=64, d=64, wsigma=0.5, logits="zipf",
                                            table="serve"),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(MULTI_TILE))
def test_round_parity_multi_tile(name):
    run_round_parity(MULTI_TILE[name], seed=4)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("nrej,V,wsigma", [(0, 4096, 0.1), (1, 4096, 0.1), (2, 4096, 0.1),
                                           (3, 4096, 0.1), (5, 4096, 0.1), (40, 4096, 0.1),
                                           (1, 131072, 0.5), (2, 131072, 0.5),
                                           (5, 131072, 0.5), (40, 131072, 0.5)])
def test_residual_pass_by_rejection_count(nrej, V, wsigma):
    """Verification with exactly `nrej` requests rejected at their first draft row: 1 or 2
    take the thin residual pass, more the matrix-core pass, and with none neither pass has
    work.  The target rows 1..gamma are the draft logits themselves (every test accepts),
    except that the chosen requests get +40 on one token other than x_1 in row 1, so x_1 is
    rejected there and the residual mass sits on that token."""
    _flush(f"residual pass with {nrej} rejected requests, V={V}")
    cfg = workload.custom(name=f"rej{nrej}", B=96, gamma=3, V=V, r=256, d=64, bf16=True,
                          wsigma=wsigma, logits="zipf", table="serve")
    inp = workload.generate(cfg, 5)
    D = DeviceInputs(inp)
    od = par_draft(inp)
    tok = od["tokens"]
    T = workload.synthesize_target(inp, tok).astype(np.float32)
    W1f, W2f = oracle.widen(inp.W1), oracle.widen(inp.W2t)
    prev = np.concatenate([inp.anchor[:, None], tok[:, :-1]], axis=1)
    for k in range(cfg.gamma):
        T[:, k, :] = (inp.U[:, k, :].astype(np.float64) + W1f[prev[:, k]] @ W2f.T)
    rej = np.random.default_rng(nrej).permutation(cfg.B)[:nrej]
    for b in rej:
        T[b, 0, (tok[b, 0] + 1) % cfg.V] += 40.0
    ell = np.full(cfg.B, cfg.gamma, np.int32)
    forced = dev(tok)
    _, lg, sg = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, 1.0, inp.seed,
                                       forced=forced)
    n_g, out_g, pt_g = ds.dspark_verify(D.U, D.W1, D.W2t, D.anchor, forced, lg, sg, dev(T),
                                        dev(ell), 1.0, inp.seed)
    ref = check_verify(inp, tok, T, ell, host(n_g), host(out_g), host(pt_g))
    assert sorted(np.nonzero(ref["n_accept"] < ell)[0].tolist()) == sorted(rej.tolist())
    assert np.array_equal(host(n_g), ref["n_accept"])
    torch.cuda.synchronize()


# more requests than the target-row pass maps in LDS (8192): the rows are listed by the
# plan kernel; the matrix-core kernels run 33 column groups per position
MANY = {
    "many_rows_fp32": workload.custom(B=8200, gamma=2, V=200, r=8, d=16, wsigma=0.3,
                                      logits="zipf", table="serve"),
    "many_mfma_bf16": workload.custom(B=8200, gamma=2, V=1024, r=256, d=16, bf16=True,
                                      wsigma=0.3, logits="zipf", table="serve"),
    # the largest batch the calls accept (65535 requests: the row kernels' grid height)
    "max_batch_fp32": workload.custom(B=65535, gamma=1, V=64, r=8, d=8, wsigma=0.3,
                                      logits="zipf", table="serve"),
    "max_batch_bf16": workload.custom(B=65535, gamma=1, V=256, r=256, d=8, bf16=True,
                                      wsigma=0.3, logits="zipf", table="serve"),
}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", list(MANY))
def test_many_requests(name):
    """Draft, confidence and verification (a ragged budget and the full block) for every
    request; the scheduler's own limit (B * gamma <= 4096) keeps it out of this shape."""
    cfg = MANY[name]
    _flush(f"many requests {name}: {cfg}")
    inp = workload.generate(cfg, 3)
    D = DeviceInputs(inp)
    od = par_draft(inp)
    tok_o = od["tokens"]
    forced = dev(tok_o)
    tg, lg, sg = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature,
                                        inp.seed, forced=forced)
    tg_h, lg_h, sg_h = host(tg), host(lg), host(sg)
    mism = compare_tokens(tg_h, tok_o, od["gap"], "draft tokens")
    assert_abs(sg_h, od["lse"], "draft lse", 1e-4)
    assert_rel(np.exp(lg_h.astype(np.float64)), np.exp(od["logp"]), "p_d(x_k)", mask=~mism)
    c_o = oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tok_o)
    assert_rel(host(ds.dspark_confidence(D.h, D.W1, D.w, D.anchor, forced)), c_o, "confidence")
    T = workload.synthesize_target(inp, tok_o)
    Td = dev(T)
    for ell in ((np.arange(cfg.B) % (cfg.gamma + 1)).astype(np.int32),
                np.full(cfg.B, cfg.gamma, np.int32)):
        _flush(f"many requests {name}: verify, ell sum {int(ell.sum())}")
        n_g, out_g, pt_g = ds.dspark_verify(D.U, D.W1, D.W2t, D.anchor, forced, lg, sg, Td,
                                            dev(ell), cfg.temperature, inp.seed)
        check_verify(inp, tok_o, T, ell, host(n_g), host(out_g), host(pt_g))
    torch.cuda.synchronize()


def test_graph_replay_matches_eager():
    """A round (draft, confidence, schedule, verify) captured in a HIP graph: every replay,
    with eager work and synchronisation between replays, equals the eager round bit for bit."""
    _flush("graph replay of a round")
    cfg = SMALL["mfma_b128"]
    inp = workload.generate(cfg, 3)
    D = DeviceInputs(inp)
    B, G = cfg.B, cfg.gamma
    dev_ = torch.device("cuda")
    tok = torch.empty((B, G), dtype=torch.int32, device=dev_)
    lp = torch.empty((B, G), dtype=torch.float32, device=dev_)
    ls = torch.empty((B, G), dtype=torch.float32, device=dev_)
    cf = torch.empty((B, G), dtype=torch.float32, device=dev_)
    ell = torch.empty(B, dtype=torch.int32, device=dev_)
    th = torch.empty(1, dtype=torch.float64, device=dev_)
    nt = torch.empty(1, dtype=torch.int32, device=dev_)
    na = torch.empty(B, dtype=torch.int32, device=dev_)
    ot = torch.empty((B, G + 1), dtype=torch.int32, device=dev_)
    ws_d = torch.empty(ds.workspace_bytes(ds.OP_DRAFT, B, G, cfg.V, cfg.r), dtype=torch.uint8,
                       device=dev_)
    ws_v = torch.empty(ds.workspace_bytes(ds.OP_VERIFY, B, G, cfg.V, cfg.r),
                       dtype=torch.uint8, device=dev_)
    temp = cfg.temperature
    ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, temp, inp.seed, out=(tok, lp, ls),
                           ws=ws_d)
    torch.cuda.synchronize()
    Td = dev(workload.synthesize_target(inp, host(tok)))

    def step():
        ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, temp, inp.seed, out=(tok, lp, ls),
                               ws=ws_d)
        ds.dspark_confidence(D.h, D.W1, D.w, D.anchor, tok, out=cf)
        ds.dspark_schedule(cf, D.sps, cfg.sched_mode, out=(ell, th, nt))
        ds.dspark_verify(D.U, D.W1, D.W2t, D.anchor, tok, lp, ls, Td, ell, temp, inp.seed,
                         out=(na, ot, None), ws=ws_v)

    outs = (tok, lp, ls, cf, ell, th, nt, na, ot)
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for i in range(4):
        for t in outs:
            t.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(ref, outs):
            assert torch.equal(a, b), f"replay {i} differs from the eager round"
        step()
        torch.cuda.synchronize()
    del g


def test_deterministic():
    cfg = SMALL["mfma_b64_v_odd"]
    inp = workload.generate(cfg, 1)
    D = DeviceInputs(inp)
    outs = []
    for _ in range(2):
        t, l, s = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed)
        outs.append((host(t), host(l), host(s)))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_schedule_edge_cases_bit_exact():
    rng = np.random.default_rng(5)
    cases = []
    B, G = 128, 16
    sps = workload.sps_table(workload.CONFIGS["serve128"])
    c = rng.uniform(0, 1, size=(B, G)).astype(np.float32)
    c[::3, :5] = 1.0                    # exact ties in survival
    c[5, 2] = 0.0                       # a zero stops survival
    c[7] = 0.5                          # dyadic survival values
    cases.append((c, sps, 0))
    cases.append((c, sps, 1))
    cases.append((np.ones((B, G), np.float32), sps, 0))
    cases.append((np.full((64, 64), 0.99, np.float32), 1000.0 / (10 + np.arange(64 * 65 + 1)), 0))
    cases.append((rng.uniform(size=(1, 4)).astype(np.float32), np.full(6, 3.0), 0))
    flat = np.full(4096 + 64 + 1, 5.0)
    cases.append((rng.uniform(0.5, 1, size=(64, 64)).astype(np.float32), flat, 0))
    # candidate counts that are not powers of two: the merge's last blocks are ragged
    for Br, Gr in ((5, 3), (100, 7), (37, 16), (129, 16)):
        cr = rng.uniform(0.3, 1, size=(Br, Gr)).astype(np.float32)
        cr[::4, : min(3, Gr)] = 1.0     # ties of a across requests in different blocks
        sr = 1000.0 / (12.0 + 0.05 * np.arange(Br * (Gr + 1) + 1))
        cases.append((cr, sr, 0))
        cases.append((cr, sr, 1))
    # every c = 1/2: a_{b,j} = 2^-(j+1) for every request, so the walk stops inside a group
    # of equal a spread over all requests (admitted in request order)
    half = np.full((16, 8), 0.5, np.float32)
    cases.append((half, 1000.0 / (10 + np.arange(16 * 9 + 1)), 0))
    cases.append((half, 1000.0 / (10 + 0.3 * np.arange(16 * 9 + 1)), 0))
    # confidences above 1 (outside the sigmoid's range): runs sorted by insertion first
    up = rng.choice([0.5, 1.0, 2.0], size=(9, 5)).astype(np.float32)
    cases.append((up, 1000.0 / (10 + np.arange(9 * 6 + 1)), 0))
    cases.append((up, np.full(9 * 6 + 1, 2.0), 1))
    for c, sps_, mode in cases:
        ell_o, th_o, n_o = oracle.schedule(c, sps_, mode)
        ell_g, th_g, n_g = ds.dspark_schedule(dev(c), dev(np.asarray(sps_, np.float64)), mode)
        assert np.array_equal(host(ell_g), ell_o)
        assert host(th_g)[0] == th_o and host(n_g)[0] == n_o


def test_schedule_topk_bit_exact():
    """Top-K admission against the oracle, bit for bit, at the serve128 shape and edges;
    at the greedy schedule's own admitted count it reproduces that schedule."""
    rng = np.random.default_rng(6)
    B, G = 128, 16
    sps = workload.sps_table(workload.CONFIGS["serve128"])
    c = rng.uniform(0, 1, size=(B, G)).astype(np.float32)
    c[::3, :5] = 1.0                    # exact ties in survival
    c[5, 2] = 0.0
    cases = [(c, sps, K) for K in (0, 1, 63, 64, 65, 114, 1000, 2047, 2048, 5000)]
    cases.append((np.full((64, 64), 0.99, np.float32), 1000.0 / (10 + np.arange(64 * 65 + 1)),
                  4095))
    cases.append((rng.uniform(size=(1, 4)).astype(np.float32), np.full(6, 3.0), 2))
    cases.append((rng.uniform(size=(3, 5)).astype(np.float32), np.full(19, 2.0), 7))
    # prefixes that end inside a group of equal a spread over many requests
    half = np.full((16, 8), 0.5, np.float32)
    cases += [(half, np.full(16 * 9 + 1, 2.0), K) for K in (1, 7, 15, 16, 17, 40, 100, 127)]
    up = rng.choice([0.5, 1.0, 2.0], size=(9, 5)).astype(np.float32)   # unsorted runs
    cases += [(up, np.full(9 * 6 + 1, 2.0), K) for K in (3, 10, 21, 44)]
    for c_, sps_, K in cases:
        ell_o, th_o, n_o = oracle.schedule_topk(c_, sps_, K)
        ell_g, th_g, n_g = ds.dspark_schedule_topk(dev(c_), dev(np.asarray(sps_, np.float64)), K)
        assert np.array_equal(host(ell_g), ell_o), (c_.shape, K)
        assert host(th_g)[0] == th_o and host(n_g)[0] == n_o, (c_.shape, K)
    ell_g, th_g, n_g = ds.dspark_schedule(dev(c), dev(sps), 0)
    ell_k, th_k, n_k = ds.dspark_schedule_topk(dev(c), dev(sps), int(host(n_g)[0]) - B)
    assert np.array_equal(host(ell_g), host(ell_k)) and host(th_g)[0] == host(th_k)[0]


@pytest.mark.parametrize("n,G,n_t,n_bins,seed", [
    (50000, 6, 64, 15, 1),
    (3001, 3, 7, 10, 2),          # a ragged last chunk, a short grid
    (65536, 16, 256, 15, 3),      # the serve128 draft length, a fine grid
    (1000, 2, 1, 1, 4),           # one temperature, one bin
    (20000, 4, 5, 256, 5),        # the most bins
    (777, 8, 3, 2, 6),            # a short ragged set, two bins
    (5000, 12, 9, 1, 7),          # one bin: ECE = |sum p - sum y| / n
])
def test_sts_calibration_matches_oracle(n, G, n_t, n_bins, seed):
    """Chosen temperatures exactly (the seeds keep every runner-up ECE at least 1e-9 away)
    and ECE within 1e-9 (the GPU sums p in 2^-40 units)."""
    cal = workload.calibration_inputs(n, G, seed=seed)
    grid = np.geomspace(0.4, 5.0, n_t)
    t_o, ece_o, gap_o = oracle.sts_calibrate(cal.logit, cal.n_accept, grid, n_bins)
    assert np.all(gap_o >= 1e-9), gap_o
    t_g, ece_g = ds.dspark_sts_calibrate(dev(cal.logit), dev(cal.n_accept), dev(grid), n_bins)
    assert np.array_equal(host(t_g), t_o)
    assert_abs(host(ece_g), ece_o, "sts ece", 1e-9)


@pytest.mark.parametrize("hb,wb,vb", [(h, w, v) for h in (0, 1) for w in (0, 1)
                                      for v in (0, 1)])
def test_confidence_every_dtype_combination(hb, wb, vb):
    """The confidence head with h, W1 and w each fp32 or bf16 (eight kernel instantiations),
    d = 1000 (two 512-entry rounds of 16-byte loads and an element tail) and r = 96."""
    rng = np.random.default_rng(11)
    B, G, V, r, d = 6, 5, 700, 96, 1000
    h = rng.standard_normal((B, G, d)).astype(np.float32)
    W1 = (0.1 * rng.standard_normal((V, r))).astype(np.float32)
    w = (0.05 * rng.standard_normal(d + r)).astype(np.float32)
    h, W1, w = (workload.to_bf16_bits(x) if flag else x for x, flag in ((h, hb), (W1, wb), (w, vb)))
    anchor = rng.integers(0, V, size=B).astype(np.int32)
    tokens = rng.integers(0, V, size=(B, G)).astype(np.int32)
    c_o = oracle.confidence(h, W1, w, anchor, tokens)
    c_g = ds.dspark_confidence(dev(h), dev(W1), dev(w), dev(anchor), dev(tokens))
    assert_rel(host(c_g), c_o, f"confidence h{hb} W1{wb} w{vb}")


@pytest.mark.parametrize("name", ["tiny", "bf16_rows_b16", "mfma_b64_v_odd", "mfma_b128"])
def test_token_ids_out_of_range_are_clamped(name):
    """Anchor and forced ids below 0 or at/above V (a caller's error) are used as the
    clamped ids 0 and V - 1 wherever they index a table: the draft and the confidence head
    equal the oracle's on the clamped ids."""
    cfg = SMALL[name]
    inp = workload.generate(cfg, 5)
    D = DeviceInputs(inp)
    V = cfg.V
    raw_anchor = inp.anchor.copy()
    raw_anchor[0], raw_anchor[-1] = -5, V + 10
    rng = np.random.default_rng(5)
    raw_forced = rng.integers(0, V, size=(cfg.B, cfg.gamma)).astype(np.int32)
    raw_forced[0, 0], raw_forced[-1, -1] = -1, V
    raw_forced[cfg.B // 2, 0] = 2**31 - 1
    anchor_c, forced_c = np.clip(raw_anchor, 0, V - 1), np.clip(raw_forced, 0, V - 1)
    inp_c = dataclasses.replace(inp, anchor=anchor_c)
    od = par_draft(inp_c, forced=forced_c)
    tg, lg, sg = ds.dspark_draft_markov(D.U, D.W1, D.W2t, dev(raw_anchor), cfg.temperature,
                                        inp.seed, forced=dev(raw_forced))
    tg_h, lg_h, sg_h = host(tg), host(lg), host(sg)
    mism = compare_tokens(tg_h, od["tokens"], od["gap"], "draft tokens (clamped ids)")
    assert_abs(sg_h, od["lse"], "draft lse (clamped ids)", 1e-4)
    assert_rel(np.exp(lg_h.astype(np.float64)), np.exp(od["logp"]), "p_d(x_k) (clamped ids)",
               mask=~mism)
    c_o = oracle.confidence(inp.h, inp.W1, inp.w, anchor_c, forced_c)
    c_g = ds.dspark_confidence(D.h, D.W1, D.w, dev(raw_anchor), dev(raw_forced))
    assert_rel(host(c_g), c_o, "confidence (clamped ids)")


def test_calls_on_concurrent_streams_match_sequential_calls():
    """Draft and verification of three batches (the 16-column matrix-core draft, the
    resident draft's cooperative launch, the row kernels) enqueued together on three
    streams, each with its own workspaces, three times over: every output equals the same
    calls made one after another on one stream, bit for bit."""
    names = ["mfma_b128", "bf16_rows_b16", "tiny"]
    runs = []
    for name in names:
        cfg = SMALL[name]
        inp = workload.generate(cfg, 4)
        D = DeviceInputs(inp)
        B, G, V, r = cfg.B, cfg.gamma, cfg.V, cfg.r
        tok, lp, ls = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature,
                                             inp.seed)
        T = dev(workload.synthesize_target(inp, host(tok)))
        ell = dev(np.full(B, G, np.int32))
        ws_d = torch.empty(ds.workspace_bytes(ds.OP_DRAFT, B, G, V, r), dtype=torch.uint8,
                           device="cuda")
        ws_v = torch.empty(ds.workspace_bytes(ds.OP_VERIFY, B, G, V, r), dtype=torch.uint8,
                           device="cuda")
        outs = (torch.empty_like(tok), torch.empty_like(lp), torch.empty_like(ls),
                torch.empty(B, dtype=torch.int32, device="cuda"),
                torch.empty((B, G + 1), dtype=torch.int32, device="cuda"),
                torch.empty((B, G), dtype=torch.float32, device="cuda"))
        runs.append((cfg, inp, D, T, ell, ws_d, ws_v, outs))

    def enqueue(run, stream):
        cfg, inp, D, T, ell, ws_d, ws_v, o = run
        ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, cfg.temperature, inp.seed,
                               out=o[:3], ws=ws_d, stream=stream)
        ds.dspark_verify(D.U, D.W1, D.W2t, D.anchor, o[0], o[1], o[2], T, ell,
                         cfg.temperature, inp.seed, out=o[3:], ws=ws_v, stream=stream)

    for run in runs:
        enqueue(run, None)
    torch.cuda.synchronize()
    ref = [[t.clone() for t in run[-1]] for run in runs]
    streams = [torch.cuda.Stream() for _ in runs]
    for rep in range(3):
        for run in runs:
            for t in run[-1]:
                t.fill_(-7)
        torch.cuda.synchronize()
        for run, st in zip(runs, streams):
            enqueue(run, st)
        torch.cuda.synchronize()
        for name, run, want in zip(names, runs, ref):
            for a, b in zip(run[-1], want):
                assert torch.equal(a, b), f"{name}: concurrent call {rep} differs"


def test_calibrated_confidence_matches_oracle():
    cfg = SMALL["bf16_rows_b16"]
    inp = workload.generate(cfg, 1)
    D = DeviceInputs(inp)
    tokens = np.random.default_rng(3).integers(0, cfg.V, size=(cfg.B, cfg.gamma)).astype(np.int32)
    temps = np.geomspace(0.6, 2.4, cfg.gamma)
    c_o = oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tokens, temps)
    c_g = ds.dspark_confidence_calibrated(D.h, D.W1, D.w, D.anchor, dev(tokens), dev(temps))
    assert_rel(host(c_g), c_o, "calibrated confidence")


# ------------------------------------------------------------------------------------
# full-size workloads, every request
# ------------------------------------------------------------------------------------
@pytest.mark.timeout(1200)
@pytest.mark.parametrize("name", ["qwen1", "serve128", "v4dspark5", "bigvocab"])
def test_full_size_all_requests(name):
    cfg = workload.CONFIGS[name]
    _flush(f"full-size {name}: generating inputs")
    inp = workload.generate(cfg, 0)
    D = DeviceInputs(inp)
    temp = cfg.temperature

    # the benchmark's configuration: a free-running draft over the whole batch
    tf, lf, sf = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, temp, inp.seed)
    tf_h = host(tf)
    _flush(f"full-size {name}: oracle draft of all {cfg.B} requests")
    od = par_draft(inp)
    tok_o = od["tokens"]
    for b in range(cfg.B):
        diff = np.nonzero(tf_h[b] != tok_o[b])[0]
        if diff.size:
            assert od["gap"][b, diff[0]] < 1e-4, f"row {b} pos {diff[0] + 1}"

    # teacher-forced on the oracle's tokens: every position compared
    forced = dev(tok_o)
    tg, lg, sg = ds.dspark_draft_markov(D.U, D.W1, D.W2t, D.anchor, temp, inp.seed,
                                        forced=forced)
    tg_h, lg_h, sg_h = host(tg), host(lg), host(sg)
    mism = compare_tokens(tg_h, tok_o, od["gap"], f"{name} draft tokens")
    assert_abs(sg_h, od["lse"], f"{name} lse", 1e-4)
    assert_rel(np.exp(lg_h.astype(np.float64)), np.exp(od["logp"]), f"{name} p_d(x)",
               mask=~mism)

    c_g = host(ds.dspark_confidence(D.h, D.W1, D.w, D.anchor, forced))
    c_o = oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tok_o)
    assert_rel(c_g, c_o, f"{name} confidence")

    # the scheduler at full batch on the round's own GPU confidences (the same fp32 values
    # on both sides), and on seeded confidences that admit many more tokens
    ell_o, th_o, n_o = oracle.schedule(c_g, inp.sps, cfg.sched_mode)
    ell_g, th_g, n_g = ds.dspark_schedule(dev(c_g), D.sps, cfg.sched_mode)
    assert np.array_equal(host(ell_g), ell_o)
    assert host(th_g)[0] == th_o and host(n_g)[0] == n_o
    rng = np.random.default_rng(cfg.index)
    c_syn = (1.0 / (1.0 + np.exp(-rng.normal(0.0, 5.0, size=(cfg.B, cfg.gamma))))
             ).astype(np.float32)
    ell_s, th_s, n_s = oracle.schedule(c_syn, inp.sps, cfg.sched_mode)
    ell_sg, th_sg, n_sg = ds.dspark_schedule(dev(c_syn), D.sps, cfg.sched_mode)
    assert np.array_equal(host(ell_sg), ell_s)
    assert host(th_sg)[0] == th_s and host(n_sg)[0] == n_s

    _flush(f"full-size {name}: target synthesis")
    T = workload.synthesize_target(inp, tok_o)
    Td = dev(T)
    budgets = [("scheduled", ell_o)]
    if not np.all(ell_o == cfg.gamma):
        budgets.append(("full block", np.full(cfg.B, cfg.gamma, np.int32)))
    for what, ell in budgets:
        n_v, out_v, pt_v = ds.dspark_verify(D.U, D.W1, D.W2t, D.anchor, forced, lg, sg, Td,
                                            dev(ell), temp, inp.seed)
        _flush(f"full-size {name}: oracle verify, {what} budget (sum ell {int(ell.sum())})")
        check_verify(inp, tok_o, T, ell, host(n_v), host(out_v), host(pt_v))

    if cfg.tv:
        _flush(f"full-size {name}: TV of all {cfg.B * cfg.gamma} positions")
        a_g = host(ds.dspark_accept_rate_tv(D.U, D.W1, D.W2t, D.anchor, forced, sg, Td, temp))
        a_o, _ = par_accept_tv(inp, tok_o, T)
        assert_rel(a_g, a_o, f"{name} TV accept rate")
    torch.cuda.synchronize()


def test_stream_read_probe_times_a_read():
    """The measurement aid reads its regions and reports a physically possible duration."""
    buf = torch.empty(4 * (16 << 20), dtype=torch.uint8, device="cuda")
    ms = ds.dspark_stream_read_probe(buf, 16 << 20, reps=5)
    gbs = (16 << 20) / (ms * 1e-3) / 1e9
    assert 0.0 < ms and 10.0 < gbs < 20000.0, (ms, gbs)


def test_zz_near_tie_rate():
    """Over every sampled token compared in this session: the GPU's token differs from the
    oracle's only at flagged near-ties (asserted where each is compared), and the flagged
    near-ties (oracle top-2 gap below 1e-4) are at most 0.01% of the samples; the same for
    accept decisions inside the 1e-5 margin.  The counts appear in the terminal summary."""
    _flush(f"tally {TALLY}")
    if TALLY["samples"] < 10000:
        pytest.skip(f"only {TALLY['samples']} samples compared in this session: too few to "
                    "resolve a 0.01% rate (the whole GPU suite compares more than 10^4)")
    assert TALLY["flagged"] <= 1e-4 * TALLY["samples"]
    assert TALLY["excused"] <= TALLY["flagged"]
    assert TALLY["accept_flagged"] <= 1e-4 * TALLY["accept_tests"]
    assert TALLY["accept_excused"] <= TALLY["accept_flagged"]
