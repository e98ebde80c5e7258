"""GPU parity of the closed loop of rounds (draft -> confidence -> schedule -> stand-in
target -> verify -> next anchor) against the oracle, round by round.

Every round is checked on the state the GPU loop itself reached (its anchor and drafted
block), with the tolerances of the single-round tests: drafted tokens equal to the oracle's
free-running draft up to the first position whose oracle top-2 gap is below 1e-4;
confidences to 1e-4 relative; the schedule bit-exact on the GPU's fp32 confidences; the
verification outputs against the oracle's verification on the oracle's fp64 stand-in
target (decisions excused only inside the stated rounding margins).
"""
import dataclasses

import numpy as np
import pytest
import torch

import draft_verify_sampling_step_amd as ds
import oracle
import workload
from gpu_round import DeviceInputs, assert_rel, check_verify, host

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def _run_loop(inp, D, rounds, sigma, tseed, seed=None):
    cfg = inp.cfg
    return ds.dspark_closed_loop(D.U, D.W1, D.W2t, D.h, D.w, D.anchor, D.sps, rounds,
                                 cfg.temperature, inp.seed if seed is None else seed,
                                 cfg.sched_mode, sigma, tseed)


LOOPS = {
    "tiny": (workload.CONFIGS["tiny"], 6, 0.5),
    # V % 4 != 0 (the stand-in target's entry-by-entry path), full-block verification
    "odd_v_full": (workload.custom(name="loopodd", B=5, gamma=3, V=1001, r=16, d=32,
                                   sched_mode=1), 4, 0.8),
    # bf16 weights with r = 256: the matrix-core draft and residual paths
    "bf16_b40": (workload.custom(name="loopbf16", B=40, gamma=8, V=8192, r=256, d=256,
                                 bf16=True, logits="zipf", sigma0=0.3, sigma1=0.05,
                                 table="serve"), 4, 0.7),
    # the production scheduler: top-K admission with K from the greedy schedule of two
    # rounds earlier (greedy in rounds 0 and 1)
    "tiny_topk_delayed": (workload.custom(name="looptopk", B=4, gamma=4, V=1024, r=16, d=64,
                                          sched_mode=ds.SCHED_TOPK_DELAYED), 7, 0.5),
    "bf16_b40_topk_delayed": (workload.custom(name="loopbf16k", B=40, gamma=8, V=8192, r=256,
                                              d=256, bf16=True, logits="zipf", sigma0=0.3,
                                              sigma1=0.05, table="serve",
                                              sched_mode=ds.SCHED_TOPK_DELAYED), 6, 0.7),
}


def _oracle_schedule(cfg, c_rounds, t, sps):
    """The oracle's schedule of round t: greedy or full block, or in the delayed top-K
    mode the first K candidates of round t's order with K = N - B of the greedy schedule
    of round t - 2 (of round t itself in rounds 0 and 1).  Returns (ell, theta, N, K or
    None, own greedy N)."""
    if cfg.sched_mode != ds.SCHED_TOPK_DELAYED:
        return oracle.schedule(c_rounds[t], sps, cfg.sched_mode) + (None, None)
    n_own = oracle.schedule(c_rounds[t], sps, 0)[2]
    n_hist = oracle.schedule(c_rounds[t - 2], sps, 0)[2] if t >= 2 else n_own
    K = n_hist - cfg.B
    return oracle.schedule_topk(c_rounds[t], sps, K) + (K, n_own)


@pytest.mark.parametrize("name", list(LOOPS))
def test_closed_loop_matches_oracle_round_by_round(name):
    cfg, rounds, sigma = LOOPS[name]
    _flush(f"closed loop {name}: B={cfg.B} gamma={cfg.gamma} V={cfg.V} rounds={rounds}")
    inp = workload.generate(cfg, 3)
    D = DeviceInputs(inp)
    tseed = 0xC105ED
    out = _run_loop(inp, D, rounds, sigma, tseed)
    o = {k: (host(v) if v is not None else None) for k, v in out.items()}
    G = cfg.gamma
    assert np.array_equal(o["anchors"][0], inp.anchor)
    taus = []
    delayed = []
    for t in range(rounds):
        anchor_t = o["anchors"][t]
        if t > 0:
            prev_n = o["n_accept"][t - 1]
            expect = o["out_tokens"][t - 1][np.arange(cfg.B), prev_n]
            assert np.array_equal(anchor_t, expect), f"round {t}: anchor"
        seed_t = inp.seed + t
        tok_g = o["tokens"][t]
        # the draft: free-running oracle from the same anchor and seed
        od = oracle.draft(inp.U, inp.W1, inp.W2t, anchor_t, cfg.temperature, seed_t)
        for b in range(cfg.B):
            diff = np.nonzero(tok_g[b] != od["tokens"][b])[0]
            if diff.size:
                assert od["gap"][b, diff[0]] < 1e-4, f"round {t} request {b} pos {diff[0] + 1}"
        # the rest of the round on the GPU's own block
        c_o = oracle.confidence(inp.h, inp.W1, inp.w, anchor_t, tok_g)
        assert_rel(o["c"][t], c_o, f"round {t} confidence")
        ell_o, th_o, n_o, K, n_own = _oracle_schedule(cfg, o["c"], t, inp.sps)
        assert np.array_equal(o["ell"][t], ell_o), f"round {t}: ell"
        assert o["theta"][t] == th_o and o["n_total"][t] == n_o
        if K is not None:
            delayed.append((t, K, n_own - cfg.B))
        T_o = oracle.markov_target(inp.U, anchor_t, tok_g, sigma, tseed)
        inp_t = dataclasses.replace(inp, anchor=anchor_t.astype(np.int32), seed=seed_t)
        check_verify(inp_t, tok_g, T_o, o["ell"][t], o["n_accept"][t], o["out_tokens"][t],
                     o["pt_tok"][t])
        taus.append(float((o["n_accept"][t] + 1).mean()))
    _flush(f"closed loop {name}: tau per round {np.round(taus, 3).tolist()}")
    if cfg.sched_mode == ds.SCHED_TOPK_DELAYED:
        # (round, K admitted, K its own greedy schedule would have admitted)
        _flush(f"closed loop {name}: delayed K per round {delayed}")
        assert any(k != own for t, k, own in delayed if t >= 2), \
            "the delayed K never differed from the round's own: the delay went untested"
    # acceptance falls below one when the target adds a transition term the draft lacks
    assert np.mean(taus) < 1 + G


def test_closed_loop_target_equal_to_draft_accepts_every_scheduled_token():
    """No Markov bias in the draft (W1 = 0) and no transition term in the target
    (sigma = 0): the target law equals the draft law at every position, so every scheduled
    token is accepted and tau = ell + 1, round after round."""
    cfg = workload.CONFIGS["tiny"]
    inp = workload.generate(cfg, 5)
    inp = dataclasses.replace(inp, W1=np.zeros_like(inp.W1))
    D = DeviceInputs(inp)
    out = _run_loop(inp, D, 5, 0.0, 1)
    n = host(out["n_accept"])
    ell = host(out["ell"])
    assert np.array_equal(n, ell)
    assert (ell > 0).any()


def test_closed_loop_is_deterministic():
    cfg = workload.CONFIGS["tiny"]
    inp = workload.generate(cfg, 7)
    D = DeviceInputs(inp)
    a = _run_loop(inp, D, 4, 0.5, 9)
    b = _run_loop(inp, D, 4, 0.5, 9)
    for k in a:
        if a[k] is not None:
            x, y = a[k], b[k]
            if x.is_floating_point():   # bit patterns: the NaN padding compares equal
                x = x.view(torch.int32 if x.element_size() == 4 else torch.int64)
                y = y.view(x.dtype)
            assert torch.equal(x, y), k


@pytest.mark.parametrize("V", [1001, 4096])
def test_stand_in_target_matches_oracle(V):
    """The loop's stand-in target exported on its own (used to time the target side of a
    round apart from the loop): every entry against the oracle's fp64 definition, within the
    fp32 rounding of one add and one multiply."""
    cfg = workload.custom(name="tgt", B=5, gamma=3, V=V, r=16, d=8)
    inp = workload.generate(cfg, 2)
    tokens = np.random.default_rng(V).integers(0, V, size=(cfg.B, cfg.gamma)).astype(np.int32)
    D = DeviceInputs(inp)
    T_g = host(ds.dspark_markov_target(D.U, D.anchor, ds.to_device(tokens), 0.7, 0xC105ED))
    T_o = oracle.markov_target(inp.U, inp.anchor, tokens, 0.7, 0xC105ED)
    err = np.abs(T_g.astype(np.float64) - T_o)
    assert np.all(err <= 4e-7 * (np.abs(T_o) + 1.0)), err.max()
