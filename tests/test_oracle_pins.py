"""Pins of the fp64 oracle to facts fixed outside the oracle itself.

Every check here compares the oracle with something it does not compute: published
known-answer vectors, textbook/library routines in special cases, brute force over all
choices, the sampling law (chi-square against the distribution the method must
reproduce), or identities of the mathematics.  Each is chosen so that a plausible slip in
the oracle (a dropped term, a wrong sign, a wrong index or operand) fails one of them.
"""
import itertools
import os

import numpy as np
import pytest
from scipy import special, stats

import oracle
import workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------------------------
# random numbers
# ------------------------------------------------------------------------------------
def test_philox_known_answers():
    """Philox4x32-10 matches the published known-answer vectors of the SC'11 generator."""
    n = 0
    with open(os.path.join(GOLDEN, "philox4x32_10_kat.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            w = [int(x, 16) for x in line.split()]
            got = oracle.philox4x32(w[0:4], w[4:6])
            assert [int(x) for x in got] == w[6:10], line
            n += 1
    assert n == 3


def test_uniform_lattice_and_range():
    u = oracle.uniforms(123, 0, 1, 0, 0, 1 << 16)
    m = u * 2.0 ** 24
    assert np.all(m == np.round(m)) and np.all(np.round(m) % 2 == 1)
    assert u.min() > 0.0 and u.max() < 1.0
    # exact in fp32
    assert np.all(u.astype(np.float32).astype(np.float64) == u)


def test_uniform_word_mapping_follows_counter_definition():
    """u(seed,b,k,s,v) is word v mod 4 of Philox(counter=(v div 4, k, b, s), key=seed)."""
    seed = 0x0123456789ABCDEF
    for (b, k, s, v) in [(0, 1, 0, 0), (5, 3, 2, 7), (127, 16, 1, 0), (3, 2, 0, 151935)]:
        words = oracle.philox4x32([v // 4, k, b, s], [seed & 0xFFFFFFFF, seed >> 32])
        expect = (2.0 * (int(words[v % 4]) >> 9) + 1.0) * 2.0 ** -24
        assert oracle.uniforms(seed, b, k, s, v, 1)[0] == expect


def test_uniform_chi_square_and_stream_independence():
    u = oracle.uniforms(7, 3, 2, 0, 0, 1 << 20)
    counts, _ = np.histogram(u, bins=256, range=(0, 1))
    assert stats.chisquare(counts).pvalue > 1e-6
    # different (b, k, s) give unrelated sequences
    u2 = oracle.uniforms(7, 4, 2, 0, 0, 1 << 16)
    u3 = oracle.uniforms(7, 3, 2, 2, 0, 1 << 16)
    assert abs(np.corrcoef(u[:1 << 16], u2)[0, 1]) < 0.02
    assert abs(np.corrcoef(u[:1 << 16], u3)[0, 1]) < 0.02


# ------------------------------------------------------------------------------------
# draft
# ------------------------------------------------------------------------------------
def _tiny(seed=0, **kw):
    cfg = workload.custom(**kw)
    return workload.generate(cfg, seed)


def test_draft_rows_normalised_and_consistent():
    inp = _tiny(B=3, gamma=4, V=512, r=8)
    out = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, 1.0, inp.seed, want_probs=True)
    p = out["probs"]
    assert np.allclose(p.sum(-1), 1.0, atol=1e-12, rtol=0)
    tok = out["tokens"]
    picked = np.take_along_axis(p, tok[..., None], axis=-1)[..., 0]
    assert np.allclose(np.log(picked), out["logp"], atol=1e-12)
    assert np.all(out["gap"] > 0)


@pytest.mark.parametrize("temperature", [1.0, 0.7, 2.0])
def test_draft_without_markov_bias_is_softmax(temperature):
    """W2 = 0 removes the Markov bias: p_k = softmax(U_k / T) (library softmax)."""
    inp = _tiny(B=2, gamma=3, V=300, r=4)
    W2t = np.zeros_like(inp.W2t)
    out = oracle.draft(inp.U, inp.W1, W2t, inp.anchor, temperature, inp.seed, want_probs=True)
    ref = special.softmax(inp.U.astype(np.float64) / temperature, axis=-1)
    assert np.allclose(out["probs"], ref, atol=1e-13, rtol=1e-11)


def test_draft_bias_uses_previous_token_row():
    """Rank 1 with W1[v] = s_v: bias_k = s_{x_{k-1}} * W2t[:, 0], x_0 = anchor."""
    rng = np.random.default_rng(5)
    B, G, V = 3, 4, 64
    U = rng.normal(size=(B, G, V)).astype(np.float32)
    s = rng.normal(size=(V, 1)) * 3
    W2t = rng.normal(size=(V, 1))
    anchor = rng.integers(0, V, size=B).astype(np.int32)
    out = oracle.draft(U, s, W2t, anchor, 1.3, 99, want_probs=True)
    tok = out["tokens"]
    for b in range(B):
        prev = [anchor[b]] + list(tok[b, :-1])
        for k in range(G):
            z = (U[b, k].astype(np.float64) + s[prev[k], 0] * W2t[:, 0]) / 1.3
            assert np.allclose(out["probs"][b, k], special.softmax(z), atol=1e-13)


def test_draft_gumbel_max_sampling_law():
    """argmax(z + G) with G = -ln(-ln u) is distributed as softmax(z) (chi-square).

    200k requests share the same logits; each request draws its own uniforms.  Position 2
    checks the law conditioned on position 1's token (Markov bias through W1)."""
    rng = np.random.default_rng(11)
    B, G, V, r = 200000, 2, 8, 2
    U1 = rng.normal(size=(G, V)) * 1.5
    U = np.broadcast_to(U1, (B, G, V)).astype(np.float32)
    W1 = rng.normal(size=(V, r))
    W2t = rng.normal(size=(V, r))
    anchor = np.full(B, 3, np.int32)
    out = oracle.draft(U, W1, W2t, anchor, 1.0, 2024, want_probs=False)
    tok = out["tokens"]
    z1 = U1[0].astype(np.float32).astype(np.float64) + W1[3] @ W2t.T
    p1 = special.softmax(z1)
    c1 = np.bincount(tok[:, 0], minlength=V)
    assert stats.chisquare(c1, p1 * B).pvalue > 1e-4
    for x in range(V):
        sel = tok[:, 0] == x
        if sel.sum() < 2000:
            continue
        z2 = U1[1].astype(np.float32).astype(np.float64) + W1[x] @ W2t.T
        p2 = special.softmax(z2)
        c2 = np.bincount(tok[sel, 1], minlength=V)
        assert stats.chisquare(c2, p2 * sel.sum()).pvalue > 1e-4
    # negative control: the law of the wrong-sign Gumbel is far from p
    assert stats.chisquare(np.bincount(np.argmax(z1[None, :] + np.log(-np.log(
        rng.uniform(size=(B, V)))), 1), minlength=V), p1 * B).pvalue < 1e-10


def test_draft_forced_prefix_reproduces_free_run():
    inp = _tiny(B=4, gamma=5, V=257, r=8)
    free = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, 1.0, inp.seed)
    forced = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, 1.0, inp.seed,
                          forced=free["tokens"])
    for key in ("tokens", "logp", "lse", "gap"):
        assert np.array_equal(free[key], forced[key])


def test_draft_global_request_id_keys_randomness():
    inp = _tiny(B=4, gamma=3, V=200, r=4)
    full = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, 1.0, inp.seed)
    sub = oracle.draft(inp.U[2:], inp.W1, inp.W2t, inp.anchor[2:], 1.0, inp.seed, gid=[2, 3])
    assert np.array_equal(full["tokens"][2:], sub["tokens"])


def _scores_by_library(U, W1, W2t, prev, temperature, seed, b, k):
    """Gumbel scores of one draft position computed apart from the oracle: numpy's matmul
    for the bias, the pinned uniforms of stream 0, G = -ln(-ln u)."""
    z = (np.asarray(U, np.float64) + oracle.widen(W1)[prev] @ oracle.widen(W2t).T) / temperature
    u = oracle.uniforms(seed, b, k, 0, 0, z.shape[0])
    return z - np.log(-np.log(u))


def test_draft_gap_is_the_top_two_score_margin():
    """The oracle's reported gap (what excuses a GPU/oracle token mismatch) equals the
    margin between the two largest Gumbel scores computed apart (sorted fp64 scores), and
    its token is the largest."""
    inp = _tiny(seed=2, B=3, gamma=4, V=300, r=8, temperature=0.8)
    T = 0.8
    out = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, T, inp.seed)
    tok = out["tokens"]
    for b in range(3):
        prev = [int(inp.anchor[b])] + [int(x) for x in tok[b, :-1]]
        for k in range(4):
            sc = _scores_by_library(inp.U[b, k], inp.W1, inp.W2t, prev[k], T, inp.seed, b, k + 1)
            top = np.sort(sc)[::-1]
            assert tok[b, k] == int(np.argmax(sc))
            assert abs(out["gap"][b, k] - (top[0] - top[1])) <= 1e-9


def test_draft_gap_moves_with_the_winning_logit():
    """Raising the winner's base logit by d raises the gap by d/T; lowering it by half the
    gap (times T) halves the gap; lowering it by 1.5 gaps hands the draw to the runner-up,
    whose gap is then the smaller of half the old gap and its own lead over the third.  The
    prefix is teacher-forced so only that position changes."""
    inp = _tiny(seed=4, B=2, gamma=3, V=200, r=8)
    T = 1.25
    base = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, T, inp.seed)
    tok = base["tokens"]
    for b, k in [(0, 0), (1, 2)]:
        g0 = base["gap"][b, k]
        x = tok[b, k]
        prev = int(inp.anchor[b]) if k == 0 else int(tok[b, k - 1])
        sc = _scores_by_library(inp.U[b, k], inp.W1, inp.W2t, prev, T, inp.seed, b, k + 1)
        s1, s2, s3 = np.sort(sc)[::-1][:3]
        runner = int(np.argsort(sc)[::-1][1])
        for shift, moves in [(0.7, False), (-0.5 * g0 * T, False), (-1.5 * g0 * T, True)]:
            U = inp.U.copy()
            U[b, k, x] += np.float32(shift)
            d = (float(U[b, k, x]) - float(inp.U[b, k, x])) / T   # the score change, fp32-rounded
            out = oracle.draft(U, inp.W1, inp.W2t, inp.anchor, T, inp.seed, forced=tok)
            if moves:
                assert out["tokens"][b, k] == runner
                expect = s2 - max(s1 + d, s3)
            else:
                assert out["tokens"][b, k] == x
                expect = s1 + d - s2
            assert abs(out["gap"][b, k] - expect) <= 1e-9, (shift, out["gap"][b, k], expect)


def test_verify_margin_and_decisions_computed_apart():
    """The margin |u p_d(x) - p_t(x)| / p_t(x) the oracle reports for each accept test (what
    excuses a GPU/oracle decision flip) and the decisions themselves, against p_d and p_t
    from scipy's softmax of the draft and target logits and the pinned stream-1 uniforms;
    NaN where no test is made (beyond the first rejection or beyond ell)."""
    inp = _tiny(seed=6, B=6, gamma=4, V=60, r=8, temperature=0.9)
    T = 0.9
    d = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, T, inp.seed)
    tok = d["tokens"]
    Tl = workload.synthesize_target(inp, tok).astype(np.float64)
    ell = np.array([4, 4, 3, 2, 1, 0], np.int32)
    v = oracle.verify(inp.U, inp.W1, inp.W2t, inp.anchor, tok, Tl, ell, T, inp.seed)
    W1, W2t = oracle.widen(inp.W1), oracle.widen(inp.W2t)
    n_tests = 0
    for b in range(6):
        prev = [int(inp.anchor[b])] + [int(x) for x in tok[b, :-1]]
        n = int(v["n_accept"][b])
        made = min(n + 1, int(ell[b]))
        for k in range(4):
            if k >= made:
                assert np.isnan(v["margin"][b, k])
                continue
            x = tok[b, k]
            pd = special.softmax((inp.U[b, k].astype(np.float64) + W1[prev[k]] @ W2t.T) / T)[x]
            pt = special.softmax(Tl[b, k] / T)[x]
            u = oracle.uniforms(inp.seed, b, k + 1, 1, 0, 1)[0]
            assert abs(v["margin"][b, k] - abs(u * pd - pt) / pt) <= 1e-10 * max(1.0, u * pd / pt)
            assert (u * pd < pt) == (k < n)
            n_tests += 1
    assert n_tests >= 8 and (v["n_accept"] < ell).any()


# ------------------------------------------------------------------------------------
# confidence head
# ------------------------------------------------------------------------------------
def test_confidence_special_cases():
    inp = _tiny(B=3, gamma=4, V=100, r=5, d=7)
    tokens = np.random.default_rng(1).integers(0, 100, size=(3, 4)).astype(np.int32)
    d, r = 7, 5
    w = np.zeros(d + r)
    assert np.all(oracle.confidence(inp.h, inp.W1, w, inp.anchor, tokens) == 0.5)
    for j in (0, 3, 6):
        w = np.zeros(d + r); w[j] = 1.0
        c = oracle.confidence(inp.h, inp.W1, w, inp.anchor, tokens)
        assert np.allclose(c, special.expit(inp.h[:, :, j].astype(np.float64)), atol=1e-15)
    W1 = np.asarray(inp.W1, np.float64)
    for i in (0, 4):
        w = np.zeros(d + r); w[d + i] = 2.0
        c = oracle.confidence(inp.h, inp.W1, w, inp.anchor, tokens)
        prev = np.concatenate([inp.anchor[:, None], tokens[:, :-1]], axis=1)
        assert np.allclose(c, special.expit(2.0 * W1[prev, i]), atol=1e-15)


# ------------------------------------------------------------------------------------
# scheduler
# ------------------------------------------------------------------------------------
def _theta(c, sps, ell):
    """Theta(ell) = (B + sum_b sum_{j<=ell_b} prod_{i<=j} c_bi) * SPS(B + sum ell)."""
    B = c.shape[0]
    tau = float(B)
    for b in range(B):
        a = 1.0
        for j in range(ell[b]):
            a *= c[b, j]
            tau += a
    return tau * sps[B + int(sum(ell))]


@pytest.mark.parametrize("seed", range(12))
def test_schedule_matches_brute_force_on_convex_tables(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    G = int(rng.integers(1, 5))
    c = rng.uniform(0.05, 1.0, size=(B, G)).astype(np.float32)
    N = np.arange(B * (G + 1) + 1, dtype=np.float64)
    t = rng.uniform(5, 15) + rng.uniform(0, 2) * N + rng.uniform(0, 0.3) * N * N   # convex
    sps = 1000.0 / t
    ell, theta, n_total = oracle.schedule(c, sps, 0)
    c64 = c.astype(np.float64)
    best = max(_theta(c64, sps, e) for e in itertools.product(range(G + 1), repeat=B))
    assert abs(theta - best) <= 1e-12 * best
    assert abs(_theta(c64, sps, ell) - theta) <= 1e-12 * best
    assert n_total == B + int(ell.sum())


def test_schedule_closed_form_half_confidences():
    """c = 1/2 gives a_j = 2^-j; with t(N) = 10 + N the stop point has a closed form."""
    B, G = 2, 6
    c = np.full((B, G), 0.5, np.float32)
    sps = 1000.0 / (10.0 + np.arange(B * (G + 1) + 1))
    ell, theta, n_total = oracle.schedule(c, sps, 0)
    # admitting a token is worth it iff a > tau * dt / t = tau / (10 + N)
    tau, N, expect = 2.0, 2, [0, 0]
    order = [(0.5 ** j, b, j) for j in range(1, G + 1) for b in range(B)]
    order.sort(key=lambda x: (-x[0], x[1], x[2]))
    for a, b, j in order:
        if (tau + a) / (10 + N + 1) <= tau / (10 + N):
            break
        tau, N = tau + a, N + 1
        expect[b] = j
    assert list(ell) == expect and n_total == N
    assert theta == pytest.approx(1000.0 * tau / (10 + N), rel=1e-15)


def test_schedule_flat_and_steep_tables():
    rng = np.random.default_rng(3)
    B, G = 5, 4
    c = rng.uniform(0.01, 0.99, size=(B, G)).astype(np.float32)
    flat = np.full(B * (G + 1) + 1, 7.0)
    ell, _, n = oracle.schedule(c, flat, 0)
    assert np.all(ell == G) and n == B * (G + 1)
    steep = 1000.0 / (1.0 + 1e6 * np.arange(B * (G + 1) + 1))
    ell, theta, n = oracle.schedule(c, steep, 0)
    assert np.all(ell == 0) and n == B and theta == B * steep[B]
    ell, _, n = oracle.schedule(c, steep, 1)
    assert np.all(ell == G) and n == B * (G + 1)


def test_schedule_tie_order_request_then_position():
    """Equal survival: the lower request index is admitted first, then the lower j."""
    c = np.array([[0.5], [0.5]], np.float32)
    sps = np.array([0.0, 0.0, 1.0, 1.0, 0.8])
    ell, theta, n = oracle.schedule(c, sps, 0)
    assert list(ell) == [1, 0] and theta == 2.5 and n == 3
    c = np.array([[1.0, 1.0, 0.5]], np.float32)
    sps = np.array([0, 1.0, 1.0, 1.0, 0.5])
    ell, theta, n = oracle.schedule(c, sps, 0)
    assert list(ell) == [2] and theta == 3.0


def test_schedule_confidence_above_one_reports_the_largest_admitted_position():
    """Outside the sigmoid's range (c > 1) a request's survival can grow, so its admitted
    positions need not come in j order; ell_b is then the largest admitted j (greedy and
    top-K alike).  c = (1/2, 2): a = (1/2, 1), so position 2 is taken before position 1."""
    c = np.array([[0.5, 2.0]], np.float32)
    flat = np.full(4, 2.0)            # every admission raises Theta: both are taken
    ell, theta, n = oracle.schedule(c, flat, 0)
    assert list(ell) == [2] and n == 3 and theta == (1.0 + 1.0 + 0.5) * 2.0
    ell, theta, n = oracle.schedule_topk(c, flat, 1)   # only the first in order
    assert list(ell) == [2] and n == 2 and theta == 2.0 * 2.0
    ell, _, n = oracle.schedule_topk(c, flat, 2)
    assert list(ell) == [2] and n == 3


def _tau(c, ell):
    """tau(ell) = B + sum_b sum_{j<=ell_b} prod_{i<=j} c_bi (expected output tokens)."""
    B = c.shape[0]
    tau = float(B)
    for b in range(B):
        a = 1.0
        for j in range(ell[b]):
            a *= c[b, j]
            tau += a
    return tau


@pytest.mark.parametrize("seed", range(10))
def test_schedule_topk_is_the_best_admission_of_its_size(seed):
    """For a fixed number K of admitted tokens (fixed N = B + K), the admitted set with
    the most expected output tokens is the top-K by survival [XTL §6/§7]: brute force
    over every ell with sum(ell) = K reaches the same tau, at the same ell when unique."""
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 4))
    G = int(rng.integers(1, 5))
    c = rng.uniform(0.05, 1.0, size=(B, G)).astype(np.float32)
    c64 = c.astype(np.float64)
    sps = 1000.0 / (10.0 + np.arange(B * (G + 1) + 1))
    for K in range(B * G + 1):
        ell, theta, n_total = oracle.schedule_topk(c, sps, K)
        assert n_total == B + K and int(ell.sum()) == K
        cands = [e for e in itertools.product(range(G + 1), repeat=B) if sum(e) == K]
        taus = np.array([_tau(c64, e) for e in cands])
        best = taus.max()
        assert abs(_tau(c64, ell) - best) <= 1e-12 * best
        assert abs(theta - best * sps[B + K]) <= 1e-12 * theta
        if (taus >= best * (1 - 1e-12)).sum() == 1:
            assert tuple(ell) == cands[int(taus.argmax())]


@pytest.mark.parametrize("seed", range(6))
def test_schedule_topk_at_the_greedy_count_is_the_greedy_schedule(seed):
    """The greedy schedule admits the first n_total - B candidates of the same order, so
    top-K with that K must reproduce its ell, Theta and N bit for bit."""
    rng = np.random.default_rng(200 + seed)
    B, G = int(rng.integers(2, 40)), int(rng.integers(1, 17))
    c = rng.uniform(0.0, 1.0, size=(B, G)).astype(np.float32)
    c[rng.random((B, G)) < 0.1] = 1.0     # exact ties in survival
    N = np.arange(B * (G + 1) + 1, dtype=np.float64)
    sps = 1000.0 / (12.0 + 0.02 * N + 1e-5 * N * N)
    ell_g, theta_g, n_g = oracle.schedule(c, sps, 0)
    ell_k, theta_k, n_k = oracle.schedule_topk(c, sps, n_g - B)
    assert np.array_equal(ell_g, ell_k) and theta_g == theta_k and n_g == n_k


def test_schedule_topk_edges_and_monotonicity():
    rng = np.random.default_rng(7)
    B, G = 6, 5
    c = rng.uniform(0.1, 0.95, size=(B, G)).astype(np.float32)
    sps = 1000.0 / (10.0 + np.arange(B * (G + 1) + 1))
    ell, theta, n = oracle.schedule_topk(c, sps, 0)
    assert np.all(ell == 0) and n == B and theta == B * sps[B]
    full = oracle.schedule(c, sps, 1)
    for K in (B * G, B * G + 7):
        ell, theta, n = oracle.schedule_topk(c, sps, K)
        assert np.all(ell == G) and n == B * (G + 1) and theta == full[1]
    assert np.all(oracle.schedule_topk(c, sps, -3)[0] == 0)
    prev = np.zeros(B, np.int32)
    for K in range(B * G + 1):
        ell = oracle.schedule_topk(c, sps, K)[0]
        assert np.all(ell >= prev) and int((ell - prev).sum()) == (1 if K else 0)
        prev = ell


# ------------------------------------------------------------------------------------
# sequential temperature scaling of the confidence head
# ------------------------------------------------------------------------------------
def test_sts_recovers_known_temperatures():
    """Labels drawn so that sigmoid(logit / t*_k) is the true conditional acceptance: the
    left-to-right search must find t*_k (within the grid's spacing and the sampling noise)
    and leave the cumulative products calibrated, where the raw head (t = 1) is not."""
    cal = workload.calibration_inputs(200000, 6, seed=1)
    grid = np.geomspace(0.5, 4.0, 64)          # neighbouring values 3.4% apart
    t, ece, gap = oracle.sts_calibrate(cal.logit, cal.n_accept, grid, 15)
    step = np.log(grid[1] / grid[0])
    assert np.all(np.abs(np.log(t / cal.t_true)) <= 2.5 * step), (t, cal.t_true)
    assert np.all(ece < 0.006)
    _, ece_raw, _ = oracle.sts_calibrate(cal.logit, cal.n_accept, np.array([1.0]), 15)
    assert np.all(ece_raw > 3 * ece)


def test_sts_calibrated_head_keeps_temperature_one():
    cal = workload.calibration_inputs(200000, 4, seed=2, t_true=np.ones(4))
    grid = np.geomspace(0.5, 2.0, 41)
    t, _, _ = oracle.sts_calibrate(cal.logit, cal.n_accept, grid, 15)
    assert np.all(np.abs(np.log(t)) <= 2.5 * np.log(grid[1] / grid[0]))


def test_calibrated_confidence_is_the_scaled_logit():
    """sigmoid(logit / t) from the calibrated head equals the plain head's c pushed back
    through the logit: c' = sigmoid(log(c / (1 - c)) / t)."""
    inp = workload.generate(workload.CONFIGS["tiny"], 2)
    tokens = np.random.default_rng(1).integers(0, 1024, size=(4, 4)).astype(np.int32)
    temps = np.array([0.5, 1.0, 1.7, 3.0])
    c = oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tokens)
    ct = oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tokens, temps)
    assert np.allclose(ct, special.expit(special.logit(c) / temps), rtol=1e-12, atol=0)
    assert np.array_equal(oracle.confidence(inp.h, inp.W1, inp.w, inp.anchor, tokens,
                                            np.ones(4)), c)


def test_sts_ece_by_hand():
    """Four samples, one position, t = 1: c = sigmoid(logit) put p at 0.1, 0.15 (bin 1 of
    10), 0.5 (bin 5) and 0.9 (bin 9); labels 0, 1, 1, 1.
    ECE = (2/4)|0.125 - 0.5| + (1/4)|0.5 - 1| + (1/4)|0.9 - 1| = 0.1875 + 0.125 + 0.025."""
    p = np.array([0.1, 0.15, 0.5, 0.9])
    logit = np.log(p / (1 - p))[:, None]
    t, ece, gap = oracle.sts_calibrate(logit, np.array([0, 1, 1, 1]), np.array([1.0]), 10)
    assert t[0] == 1.0 and np.isinf(gap[0])
    assert ece[0] == pytest.approx(0.3375, abs=1e-15)


def test_sts_one_value_grid_and_first_on_ties():
    """A one-value grid returns that value at every position, with the ECE of the plain
    products; a grid listing the same value twice chooses the first (a zero gap)."""
    cal = workload.calibration_inputs(5000, 3, seed=3)
    t, ece, _ = oracle.sts_calibrate(cal.logit, cal.n_accept, np.array([1.7]), 12)
    assert np.all(t == 1.7)
    t2, ece2, gap2 = oracle.sts_calibrate(cal.logit, cal.n_accept, np.array([1.7, 1.7]), 12)
    assert np.array_equal(t2, t) and np.array_equal(ece2, ece) and np.all(gap2 == 0.0)


# ------------------------------------------------------------------------------------
# verification
# ------------------------------------------------------------------------------------
def test_verify_identical_target_accepts_everything():
    inp = _tiny(B=4, gamma=4, V=256, r=8)
    W2t = np.zeros_like(inp.W2t)
    d = oracle.draft(inp.U, inp.W1, W2t, inp.anchor, 0.8, inp.seed)
    T = np.concatenate([inp.U, inp.U_extra[:, None, :]], axis=1)
    ell = np.array([4, 2, 0, 3], np.int32)
    v = oracle.verify(inp.U, inp.W1, W2t, inp.anchor, d["tokens"], T, ell, 0.8, inp.seed)
    assert np.array_equal(v["n_accept"], ell)
    assert np.all(v["kind"] == 0)
    for b in range(4):
        assert np.array_equal(v["out_tokens"][b, :ell[b]], d["tokens"][b, :ell[b]])
        assert np.all(v["out_tokens"][b, ell[b] + 1:] == -1)


def test_verify_one_hot_target_rejects_and_corrects():
    inp = _tiny(B=3, gamma=3, V=128, r=4)
    d = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, 1.0, inp.seed)
    T = np.full((3, 4, 128), -1e4, np.float32)
    vstar = (d["tokens"][:, 0] + 5) % 128
    T[np.arange(3), 0, vstar] = 0.0
    v = oracle.verify(inp.U, inp.W1, inp.W2t, inp.anchor, d["tokens"], T,
                      np.full(3, 3, np.int32), 1.0, inp.seed)
    assert np.all(v["n_accept"] == 0)
    assert np.array_equal(v["out_tokens"][:, 0], vstar)
    assert np.all(v["out_tokens"][:, 1:] == -1) and np.all(v["kind"] == 1)


def _markov_tables(rng, G, V, conc):
    """log p_t,k(. | prev) for k = 1..G+1, shape [G+1][V(prev)][V]."""
    p = rng.dirichlet(np.full(V, conc), size=(G + 1, V))
    return np.log(p)


def _complete_and_histogram(rng, out_tokens, logpt, anchor, G, V):
    """Complete each emitted prefix with the target chain; histogram full strings."""
    B = out_tokens.shape[0]
    seq = out_tokens.astype(np.int64).copy()
    pt = np.exp(logpt)
    for k in range(G + 1):
        need = seq[:, k] < 0
        if not need.any():
            continue
        prev = anchor[need] if k == 0 else seq[need, k - 1]
        cdf = np.cumsum(pt[k][prev], axis=1)
        u = rng.uniform(size=need.sum())[:, None]
        seq[need, k] = np.minimum((u > cdf).sum(1), V - 1)
    code = np.zeros(B, np.int64)
    for k in range(G + 1):
        code = code * V + seq[:, k]
    return np.bincount(code, minlength=V ** (G + 1))


def _target_law(logpt, a0, G, V):
    prob = np.zeros(V ** (G + 1))
    for i, ys in enumerate(itertools.product(range(V), repeat=G + 1)):
        lp, prev = 0.0, a0
        for k, y in enumerate(ys):
            lp += logpt[k][prev][y]
            prev = y
        prob[i] = np.exp(lp)
    return prob


def _lossless_round(rng, B, G, V, r, ell_rule, seed):
    """Draft with a Markov head, build Markov target rows, verify with ell from ell_rule."""
    U1 = rng.normal(size=(G, V)) * 1.2
    U = np.broadcast_to(U1, (B, G, V)).astype(np.float32)
    W1 = rng.normal(size=(V, r))
    W2t = rng.normal(size=(V, r))
    anchor = np.full(B, 1, np.int32)
    logpt = _markov_tables(rng, G, V, 1.0)
    d = oracle.draft(U, W1, W2t, anchor, 1.0, seed)
    tok = d["tokens"]
    prev = np.concatenate([anchor[:, None], tok], axis=1)             # x_0..x_G
    T = np.stack([logpt[k][prev[:, k]] for k in range(G + 1)], axis=1).astype(np.float64)
    ell = ell_rule(tok, d, T).astype(np.int32)
    v = oracle.verify(U, W1, W2t, anchor, tok, T, ell, 1.0, seed)
    hist = _complete_and_histogram(rng, v["out_tokens"], logpt, anchor, G, V)
    law = _target_law(logpt, 1, G, V)
    return hist, law, v


def _chi2_p(hist, law):
    n = hist.sum()
    keep = law * n > 5
    obs = np.append(hist[keep], hist[~keep].sum())
    exp = np.append(law[keep], law[~keep].sum()) * n
    return stats.chisquare(obs, exp).pvalue


@pytest.mark.parametrize("rule", ["full", "fixed_mix", "scheduler", "topk_delayed"])
def test_verify_is_lossless_monte_carlo(rule):
    """The emitted tokens, completed with the target chain, follow the target law."""
    rng = np.random.default_rng({"full": 1, "fixed_mix": 2, "scheduler": 3,
                                 "topk_delayed": 4}[rule])
    B, G, V, r = 200000, 3, 4, 2

    def ell_rule(tok, d, T):
        if rule == "full":
            return np.full(B, G)
        if rule == "fixed_mix":
            return np.arange(B) % (G + 1)
        # confidence head + greedy scheduler: admission of x_k uses c_1..c_k only,
        # and c_k depends on x_{k-1}, never on x_k (non-anticipating)
        h = rng.normal(size=(B, G, 3))
        w = rng.normal(size=3 + r)
        c = oracle.confidence(h, np.eye(V, r) * 3.0, w, np.full(B, 1), tok).astype(np.float32)
        N = np.arange(B * (G + 1) + 1, dtype=np.float64)
        sps = 1000.0 / (10.0 + 3.0 * N / B + 1.0 * (N / B) ** 2)
        if rule == "scheduler":
            return oracle.schedule(c, sps, 0)[0]
        # dynamic top-K [XTL §7]: K from an earlier, independent batch's schedule (the
        # history), the admitted set from the current confidences
        c_old = rng.uniform(0.0, 1.0, size=(B, G)).astype(np.float32)
        K = oracle.schedule(c_old, sps, 0)[2] - B
        return oracle.schedule_topk(c, sps, K)[0]

    hist, law, v = _lossless_round(rng, B, G, V, r, ell_rule, seed=77 + len(rule))
    assert _chi2_p(hist, law) > 1e-4
    if rule != "fixed_mix":
        assert (v["kind"] == 1).any()


def test_verify_losslessness_check_has_power():
    """Negative control: truncating on the drafted token itself (anticipating) is biased."""
    rng = np.random.default_rng(9)
    B, G, V, r = 200000, 3, 4, 2

    def anticipating(tok, d, T):
        # stop right before the first token the target likes less than the draft
        pt = np.exp(np.take_along_axis(T[:, :G], tok[..., None], axis=2)[..., 0])
        bad = pt < np.exp(d["logp"])
        first = np.where(bad.any(1), bad.argmax(1), G)
        return first

    hist, law, _ = _lossless_round(rng, B, G, V, r, anticipating, seed=5)
    assert _chi2_p(hist, law) < 1e-12


# ---- exact enumeration of the verification law ([XTL] §1 and §6: lossless rejection
# sampling).  Every draft block is enumerated with the oracle's own draft distributions,
# and every branch of the step with its exact probability: x_k accepted with
# min(1, p_t/p_d), a rejection resampled from max(0, p_t - p_d) normalised, and the bonus
# from p_t.  Each emitted prefix is completed with the target chain.  The law of the
# completed strings must be the target chain's law.
def _enum_tables(seed, V, G, r):
    """Draft rows p_d,k(. | prev) from the oracle (one request per prev, the prefix forced
    to prev) and Markov target rows p_t,k(. | prev), k = 1..G+1."""
    rng = np.random.default_rng(seed)
    U1 = rng.normal(size=(G, V)) * 1.2
    W1 = rng.normal(size=(V, r)) * 0.8
    W2t = rng.normal(size=(V, r)) * 0.8
    U = np.broadcast_to(U1, (V, G, V)).copy()
    prevs = np.arange(V, dtype=np.int32)
    d = oracle.draft(U, W1, W2t, prevs, 1.0, 1, forced=np.repeat(prevs[:, None], G, axis=1),
                     want_probs=True)
    pd = np.transpose(d["probs"], (1, 0, 2))                   # [G][prev][V]
    logpt = _markov_tables(rng, G, V, 0.7)                     # [G+1][prev][V]
    return U1, W1, W2t, pd, logpt


def _completions(pt, G, V):
    """C[m][prev]: law of the tokens at positions m..G given the token before them."""
    C = [None] * (G + 2)
    C[G + 1] = np.ones((V, 1))
    for m in range(G, -1, -1):
        C[m] = np.stack([np.concatenate([pt[m][pv][y] * C[m + 1][y] for y in range(V)])
                         for pv in range(V)])
    return C


def _emitted_law(pd, pt, C, a0, x, ell, G, V):
    """Law over the (G+1)-strings of one verification of the block x with budget ell."""
    law = np.zeros(V ** (G + 1))
    prevs = (a0,) + tuple(x)

    def add(prefix, w):
        code = 0
        for y in prefix:
            code = code * V + y
        n = V ** (G + 1 - len(prefix))
        law[code * n:(code + 1) * n] += w * C[len(prefix)][prefix[-1]]

    acc = 1.0
    for k in range(ell):
        q_t, q_d = pt[k][prevs[k]], pd[k][prevs[k]]
        a = min(1.0, q_t[x[k]] / q_d[x[k]])
        rho = np.maximum(0.0, q_t - q_d)
        if a < 1.0:
            for y in np.nonzero(rho > 0)[0]:
                add(tuple(x[:k]) + (int(y),), acc * (1.0 - a) * rho[y] / rho.sum())
        acc *= a
    for y in range(V):
        add(tuple(x[:ell]) + (y,), acc * pt[ell][prevs[ell]][y])
    return law


def _block_prob(pd, a0, x):
    p, prev = 1.0, a0
    for k, y in enumerate(x):
        p *= pd[k][prev][y]
        prev = y
    return p


def _enumerate(pd, pt, a0, G, V, ell_of):
    C = _completions(pt, G, V)
    law = np.zeros(V ** (G + 1))
    for x in itertools.product(range(V), repeat=G):
        law += _block_prob(pd, a0, x) * _emitted_law(pd, pt, C, a0, x, ell_of(x), G, V)
    return law


@pytest.mark.parametrize("rule", ["full", "ell0", "ell1", "ell2", "scheduler"])
def test_verify_is_lossless_by_exact_enumeration(rule):
    """V = 8, gamma = 3: all 512 draft blocks and every branch; the law of the completed
    strings equals the target chain's to 1e-12."""
    V, G, r, a0 = 8, 3, 3, 2
    U1, W1, W2t, pd, logpt = _enum_tables(11, V, G, r)
    pt = np.exp(logpt)
    if rule == "full":
        ell_of = lambda x: G
    elif rule.startswith("ell"):
        ell_of = lambda x, e=int(rule[3:]): e
    else:
        # confidence head + greedy scheduler, one request: c_k depends on x_{k-1} only
        rng = np.random.default_rng(5)
        h = rng.normal(size=(1, G, 4))
        w = rng.normal(size=4 + r)
        W1c = rng.normal(size=(V, r)) * 2.0
        N = np.arange(G + 2, dtype=np.float64)
        sps = 1000.0 / (10.0 + 3.0 * N + N ** 2)
        table = {}
        for x in itertools.product(range(V), repeat=G):
            c = oracle.confidence(h, W1c, w, np.array([a0]), np.array([x], np.int32))
            table[x] = int(oracle.schedule(c.astype(np.float32), sps, 0)[0][0])
        assert len(set(table.values())) > 1          # the budget does vary with the block
        ell_of = table.__getitem__
    law = _enumerate(pd, pt, a0, G, V, ell_of)
    target = _target_law(logpt, a0, G, V)
    assert abs(law.sum() - 1.0) < 1e-12
    assert np.max(np.abs(law - target)) < 1e-12


def test_verify_lossless_enumeration_two_coupled_requests():
    """B = 2, V = 4, gamma = 2 with the greedy scheduler choosing both budgets from both
    blocks: the joint law of the two completed strings is the product of the target laws."""
    V, G, r = 4, 2, 2
    U1, W1, W2t, pd, logpt = _enum_tables(12, V, G, r)
    pt = np.exp(logpt)
    a = (1, 3)
    C = _completions(pt, G, V)
    rng = np.random.default_rng(17)
    h = rng.normal(size=(2, G, 3)) * 0.3
    w = rng.normal(size=3 + r)
    W1c = rng.normal(size=(V, r)) * 2.0
    N = np.arange(2 * (G + 1) + 1, dtype=np.float64)
    sps = 1000.0 / (30.0 + N + 0.5 * N ** 2)
    joint = np.zeros((V ** (G + 1), V ** (G + 1)))
    budgets = set()
    for x1 in itertools.product(range(V), repeat=G):
        for x2 in itertools.product(range(V), repeat=G):
            toks = np.array([x1, x2], np.int32)
            c = oracle.confidence(h, W1c, w, np.array(a), toks).astype(np.float32)
            ell = oracle.schedule(c, sps, 0)[0]
            budgets.add(tuple(int(e) for e in ell))
            l1 = _emitted_law(pd, pt, C, a[0], x1, int(ell[0]), G, V)
            l2 = _emitted_law(pd, pt, C, a[1], x2, int(ell[1]), G, V)
            joint += _block_prob(pd, a[0], x1) * _block_prob(pd, a[1], x2) * np.outer(l1, l2)
    assert len(budgets) >= 4          # each request's budget depends on both blocks
    target = np.outer(_target_law(logpt, a[0], G, V), _target_law(logpt, a[1], G, V))
    assert np.max(np.abs(joint - target)) < 1e-12


def _emitted_prefixes(pd, pt, a0, x, ell, V):
    """Law over the variable-length token strings one verification of block x with budget
    ell emits (x_1..x_n and the residual or bonus token), as {string: probability}."""
    out = {}
    prevs = (a0,) + tuple(x)
    acc = 1.0
    for k in range(ell):
        q_t, q_d = pt[k][prevs[k]], pd[k][prevs[k]]
        a = min(1.0, q_t[x[k]] / q_d[x[k]])
        rho = np.maximum(0.0, q_t - q_d)
        if a < 1.0:
            for y in np.nonzero(rho > 0)[0]:
                key = tuple(x[:k]) + (int(y),)
                out[key] = out.get(key, 0.0) + acc * (1.0 - a) * rho[y] / rho.sum()
        acc *= a
    for y in range(V):
        key = tuple(x[:ell]) + (y,)
        out[key] = out.get(key, 0.0) + acc * pt[ell][prevs[ell]][y]
    return out


class _ChainedRounds:
    """Two requests (B = 2), V = 4, gamma = 2, Markov draft and target tables, a confidence
    head with its own hidden states per round, and the greedy scheduler's step-time table."""
    V, G, B, r = 4, 2, 2, 2

    def __init__(self, seed):
        V, G, r = self.V, self.G, self.r
        _, _, _, self.pd, logpt = _enum_tables(seed, V, G, r)
        self.logpt = logpt
        self.pt = np.exp(logpt)
        self.C = _completions(self.pt, G, V)
        rng = np.random.default_rng(seed + 100)
        self.h = rng.normal(size=(3, self.B, G, 3)) * 0.3      # hidden states of rounds 0-2
        self.w = rng.normal(size=3 + r)
        self.W1c = rng.normal(size=(V, r)) * 4.0
        N = np.arange(self.B * (G + 1) + 1, dtype=np.float64)
        self.sps = 1000.0 / (10.0 + N + 0.3 * N ** 2)
        self.blocks = list(itertools.product(range(V), repeat=G))

    def conf(self, rnd, anchors, x1, x2):
        toks = np.array([x1, x2], np.int32)
        return oracle.confidence(self.h[rnd], self.W1c, self.w, np.array(anchors),
                                 toks).astype(np.float32)

    def block_pairs(self, anchors):
        for x1 in self.blocks:
            p1 = _block_prob(self.pd, anchors[0], x1)
            for x2 in self.blocks:
                yield x1, x2, p1 * _block_prob(self.pd, anchors[1], x2)

    def target_pair(self, anchors):
        return np.outer(_target_law(self.logpt, anchors[0], self.G, self.V),
                        _target_law(self.logpt, anchors[1], self.G, self.V))

    def greedy_round(self, rnd, anchors):
        """Greedy round: ({(last token 1, last token 2, N - B): probability}, completed
        joint law of the two requests' emitted strings)."""
        states, joint = {}, np.zeros((self.V ** (self.G + 1),) * 2)
        for x1, x2, w in self.block_pairs(anchors):
            ell, _, N = oracle.schedule(self.conf(rnd, anchors, x1, x2), self.sps, 0)
            e1 = _emitted_prefixes(self.pd, self.pt, anchors[0], x1, int(ell[0]), self.V)
            e2 = _emitted_prefixes(self.pd, self.pt, anchors[1], x2, int(ell[1]), self.V)
            for o1, q1 in e1.items():
                for o2, q2 in e2.items():
                    key = (o1[-1], o2[-1], N - self.B)
                    states[key] = states.get(key, 0.0) + w * q1 * q2
            joint += w * np.outer(
                _emitted_law(self.pd, self.pt, self.C, anchors[0], x1, int(ell[0]), self.G, self.V),
                _emitted_law(self.pd, self.pt, self.C, anchors[1], x2, int(ell[1]), self.G, self.V))
        return states, joint

    def topk_round(self, rnd, anchors, k_of):
        """Top-K round, K = k_of(x1, x2): completed joint law of the emitted strings, and
        whether K ever differed from the round's own greedy count."""
        joint = np.zeros((self.V ** (self.G + 1),) * 2)
        differs = False
        for x1, x2, w in self.block_pairs(anchors):
            c = self.conf(rnd, anchors, x1, x2)
            K = k_of(x1, x2)
            ell = oracle.schedule_topk(c, self.sps, K)[0]
            differs |= K != oracle.schedule(c, self.sps, 0)[2] - self.B
            joint += w * np.outer(
                _emitted_law(self.pd, self.pt, self.C, anchors[0], x1, int(ell[0]), self.G, self.V),
                _emitted_law(self.pd, self.pt, self.C, anchors[1], x2, int(ell[1]), self.G, self.V))
        return joint, differs


def test_verify_lossless_enumeration_delayed_topk_chained_rounds():
    """The production scheduler ([XTL] §7): round t admits the first K candidates of its own
    order with K = N - B of the greedy schedule of round t - 2.  Three chained rounds, each
    anchored on the last tokens the round before emitted, from every anchor pair at the
    start: rounds 0 and 1 greedy, round 2 top-K with K from round 0.  Every (anchor pair,
    K) state round 2 can start from is enumerated (all draft blocks, every accept / residual
    / bonus branch): its completed output law is exactly the product of the target laws from
    its anchors, so the chain is lossless whatever history K carries.  Rounds 0 and 1 are
    checked the same way."""
    ch = _ChainedRounds(21)
    after0 = {}                      # (anchor pair after round 0, K of round 0) -> probability
    for a0 in itertools.product(range(ch.V), repeat=2):
        st0, j0 = ch.greedy_round(0, a0)
        assert np.max(np.abs(j0 - ch.target_pair(a0))) < 1e-12
        for (l1, l2, K0), p in st0.items():
            after0[(l1, l2, K0)] = after0.get((l1, l2, K0), 0.0) + p / ch.V ** 2
    round1 = {}
    states2 = {}                     # (anchor pair after round 1, K of round 0) -> probability
    for (l1, l2, K0), p0 in after0.items():
        if p0 <= 0.0:
            continue
        if (l1, l2) not in round1:
            st1, j1 = ch.greedy_round(1, (l1, l2))
            assert np.max(np.abs(j1 - ch.target_pair((l1, l2)))) < 1e-12
            round1[(l1, l2)] = st1
        for (m1, m2, _), p1 in round1[(l1, l2)].items():
            if p1 > 0.0:
                states2[(m1, m2, K0)] = states2.get((m1, m2, K0), 0.0) + p0 * p1
    assert abs(sum(states2.values()) - 1.0) < 1e-12
    assert len({K for _, _, K in states2}) >= 3         # the carried K does vary
    worst, any_differs = 0.0, False
    for (m1, m2, K0) in sorted(states2):
        j2, differs = ch.topk_round(2, (m1, m2), lambda x1, x2, K=K0: K)
        any_differs |= differs
        worst = max(worst, np.max(np.abs(j2 - ch.target_pair((m1, m2)))))
    assert worst < 1e-12
    assert any_differs          # the delayed K is not simply the round's own greedy count


def test_delayed_topk_enumeration_detects_a_budget_from_the_current_block():
    """Negative control: K taken from round 2's own drafted tokens (the number of them the
    target likes at least as much as the draft -- it looks at x_k itself) changes the law."""
    ch = _ChainedRounds(21)
    pd, pt = ch.pd, ch.pt

    def anticipating(anchors):
        def k_of(x1, x2):
            n = 0
            for a, x in ((anchors[0], x1), (anchors[1], x2)):
                prevs = (a,) + tuple(x)
                n += sum(pt[k][prevs[k]][x[k]] >= pd[k][prevs[k]][x[k]] for k in range(ch.G))
            return n
        return k_of

    worst = 0.0
    for anchors in [(1, 3), (0, 2), (2, 2)]:
        j2, _ = ch.topk_round(2, anchors, anticipating(anchors))
        worst = max(worst, 0.5 * np.abs(j2 - ch.target_pair(anchors)).sum())
    assert worst > 1e-3, worst


def test_verify_enumeration_detects_an_anticipating_budget():
    """Negative control: a budget that stops before the first drafted token the target
    likes less than the draft (it looks at x_k itself) changes the law."""
    V, G, r, a0 = 8, 3, 3, 2
    U1, W1, W2t, pd, logpt = _enum_tables(11, V, G, r)
    pt = np.exp(logpt)

    def anticipating(x):
        prevs = (a0,) + tuple(x)
        for k in range(G):
            if pt[k][prevs[k]][x[k]] < pd[k][prevs[k]][x[k]]:
                return k
        return G

    law = _enumerate(pd, pt, a0, G, V, anticipating)
    # total variation 0.027 here, against below 1e-12 per string for every rule above
    assert 0.5 * np.abs(law - _target_law(logpt, a0, G, V)).sum() > 1e-2


def test_oracle_verify_takes_the_enumerated_branches():
    """The oracle's verification follows the branches enumerated above: on every one of the
    512 blocks, x_k is accepted exactly when u * p_d(x_k) < p_t(x_k) for its uniform u, a
    correction token has positive residual mass, and a bonus token has positive p_t."""
    V, G, r, a0 = 8, 3, 3, 2
    U1, W1, W2t, pd, logpt = _enum_tables(11, V, G, r)
    pt = np.exp(logpt)
    blocks = np.array(list(itertools.product(range(V), repeat=G)), np.int32)
    B = len(blocks)
    anchor = np.full(B, a0, np.int32)
    prevs = np.concatenate([anchor[:, None], blocks], axis=1)
    T = np.stack([logpt[k][prevs[:, k]] for k in range(G + 1)], axis=1)
    U = np.broadcast_to(U1, (B, G, V)).copy()
    seed = 4242
    v = oracle.verify(U, W1, W2t, anchor, blocks, T, np.full(B, G, np.int32), 1.0, seed)
    kinds = set()
    for b in range(B):
        n = int(v["n_accept"][b])
        out = v["out_tokens"][b]
        assert np.array_equal(out[:n], blocks[b][:n])
        for k in range(min(n + 1, G)):
            u = oracle.uniforms(seed, b, k + 1, 1, 0, 1)[0]
            q_t, q_d = pt[k][prevs[b, k]], pd[k][prevs[b, k]]
            accepted = u * q_d[blocks[b][k]] < q_t[blocks[b][k]]
            assert accepted == (k < n), (b, k)
        y = int(out[n])
        if n < G:
            rho = np.maximum(0.0, pt[n][prevs[b, n]] - pd[n][prevs[b, n]])
            assert rho[y] > 0
            kinds.add("residual")
        else:
            assert pt[G][prevs[b, G]][y] > 0
            kinds.add("bonus")
        assert np.all(out[n + 1:] == -1)
    assert kinds == {"residual", "bonus"}


def test_verify_acceptance_frequency_equals_tv_rate():
    """P(accept x_1) = sum_v min(p_d, p_t) = alpha (Monte Carlo, 5-sigma)."""
    rng = np.random.default_rng(4)
    B, G, V, r = 100000, 1, 16, 3
    U = np.broadcast_to(rng.normal(size=(G, V)), (B, G, V)).astype(np.float32)
    W1 = rng.normal(size=(V, r)) * 0.5
    W2t = rng.normal(size=(V, r)) * 0.5
    anchor = np.full(B, 2, np.int32)
    T1 = rng.normal(size=(G + 1, V)) * 1.5
    T = np.broadcast_to(T1, (B, G + 1, V)).astype(np.float64)
    d = oracle.draft(U, W1, W2t, anchor, 1.0, 31)
    v = oracle.verify(U, W1, W2t, anchor, d["tokens"], T, np.ones(B, np.int32), 1.0, 31)
    alpha, l1 = oracle.accept_tv(U[:1], W1, W2t, anchor[:1], d["tokens"][:1], T[:1], 1.0)
    freq = v["n_accept"].mean()
    a = alpha[0, 0]
    assert abs(freq - a) < 5 * np.sqrt(a * (1 - a) / B)


# ------------------------------------------------------------------------------------
# analytic accept rate
# ------------------------------------------------------------------------------------
def test_tv_identity_and_bounds():
    inp = _tiny(B=3, gamma=4, V=300, r=6)
    d = oracle.draft(inp.U, inp.W1, inp.W2t, inp.anchor, 1.0, inp.seed, want_probs=True)
    T = workload.synthesize_target(inp, d["tokens"])
    alpha, l1 = oracle.accept_tv(inp.U, inp.W1, inp.W2t, inp.anchor, d["tokens"], T, 1.0)
    assert np.allclose(alpha, l1, atol=1e-13)
    assert np.all((alpha > 0) & (alpha < 1))
    # alpha = sum_x p_d(x) min(1, p_t(x)/p_d(x)): the exact acceptance probability
    pt = special.softmax(T[:, :4].astype(np.float64), axis=-1)
    pd = d["probs"]
    assert np.allclose(alpha, (pd * np.minimum(1.0, pt / pd)).sum(-1), atol=1e-13)


def test_tv_is_one_for_identical_and_zero_for_disjoint():
    inp = _tiny(B=2, gamma=2, V=64, r=4)
    W2t = np.zeros_like(inp.W2t)
    tok = np.zeros((2, 2), np.int32)
    T = np.concatenate([inp.U, inp.U_extra[:, None]], axis=1) / 0.5
    alpha, _ = oracle.accept_tv(inp.U, inp.W1, W2t, inp.anchor, tok, T * 0.5, 1.0)
    assert np.allclose(alpha, 1.0, atol=1e-13)
    U = np.full((2, 2, 64), -1e4, np.float32); U[:, :, :32] = 0
    T = np.full((2, 3, 64), -1e4, np.float32); T[:, :, 32:] = 0
    alpha, _ = oracle.accept_tv(U, inp.W1, W2t, inp.anchor, tok, T, 1.0)
    assert np.all(alpha < 1e-300)


# ------------------------------------------------------------------------------------
# distribution-matching training loss
# ------------------------------------------------------------------------------------
ALPHAS = (0.1, 0.9, 1.0)


def test_draft_loss_by_hand():
    """B=1, gamma=2, V=2 worked by hand.
    Row k=1: p_d = (1/2, 1/2), p_t = (3/4, 1/4), y = 0, confidence logit 0:
      l1 = 1/2, a = 3/4, ce = ln 2, bce = ln 2; signs (-1, +1), S = 0;
      per-unit-weight gradient 0.1 (p_d - e_0) + 0.9 p_d (s - S) = (-1/2, 1/2),
      confidence gradient c - a = -1/4.
    Row k=2: p_d = (3/4, 1/4), p_t = (1/2, 1/2), y = 1, confidence logit ln 3 (c = 3/4):
      l1 = 1/2, a = 3/4, ce = ln 4, bce = ln 4 - (3/4) ln 3; signs (+1, -1), S = 1/2;
      gradient 0.1 (3/4, -3/4) + 0.9 (3/8, -3/8) = (0.4125, -0.4125), confidence 0.
    Weights 1 and e^{-1/2}, normalised by their sum."""
    ln2, ln3, ln4 = np.log(2.0), np.log(3.0), np.log(4.0)
    zd = np.array([[[0.0, 0.0], [ln3, 0.0]]])
    zt = np.array([[[ln3, 0.0], [0.0, 0.0]]])
    labels = np.array([[0, 1]])
    cl = np.array([[0.0, ln3]])
    r = oracle.draft_loss(zd, zt, labels, cl, ALPHAS)
    w2 = np.exp(-0.5)
    W = 1.0 + w2
    t1 = 0.1 * ln2 + 0.9 * 0.5 + ln2
    t2 = 0.1 * ln4 + 0.9 * 0.5 + (ln4 - 0.75 * ln3)
    assert r["loss"] == pytest.approx((t1 + w2 * t2) / W, rel=1e-14)
    np.testing.assert_allclose(r["terms"][0], [[ln2, 0.5, ln2], [ln4, 0.5, ln4 - 0.75 * ln3]],
                               rtol=1e-14)
    np.testing.assert_allclose(r["grad_zd"][0], [[-0.5 / W, 0.5 / W],
                                                 [0.4125 * w2 / W, -0.4125 * w2 / W]],
                               rtol=1e-13)
    np.testing.assert_allclose(r["grad_conf"][0], [-0.25 / W, 0.0], atol=1e-15)


def _loss_case(seed, B=2, G=3, V=7):
    rng = np.random.default_rng(seed)
    zt = rng.normal(size=(B, G, V)) * 2.0
    zd = zt + rng.normal(size=(B, G, V)) * 0.7
    labels = rng.integers(0, V, size=(B, G))
    cl = rng.normal(size=(B, G)) * 1.5
    return zd, zt, labels, cl


@pytest.mark.parametrize("alphas", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.1, 0.9, 0.0)])
def test_draft_loss_gradient_finite_differences(alphas):
    """Central differences of the loss in every draft logit (the confidence term off, so
    that the soft label, held fixed by the gradient, plays no part)."""
    zd, zt, labels, cl = _loss_case(11)
    g = oracle.draft_loss(zd, zt, labels, cl, alphas)["grad_zd"]
    h = 1e-6
    fd = np.zeros_like(zd)
    for idx in np.ndindex(zd.shape):
        zp = zd.copy()
        zm = zd.copy()
        zp[idx] += h
        zm[idx] -= h
        fd[idx] = (oracle.draft_loss(zp, zt, labels, cl, alphas, grads=False)["loss"] -
                   oracle.draft_loss(zm, zt, labels, cl, alphas, grads=False)["loss"]) / (2 * h)
    np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-9)


def test_draft_loss_confidence_gradient_finite_differences():
    zd, zt, labels, cl = _loss_case(12)
    g = oracle.draft_loss(zd, zt, labels, cl, ALPHAS)["grad_conf"]
    h = 1e-6
    for idx in np.ndindex(cl.shape):
        cp = cl.copy()
        cm = cl.copy()
        cp[idx] += h
        cm[idx] -= h
        fd = (oracle.draft_loss(zd, zt, labels, cp, ALPHAS, grads=False)["loss"] -
              oracle.draft_loss(zd, zt, labels, cm, ALPHAS, grads=False)["loss"]) / (2 * h)
        assert g[idx] == pytest.approx(fd, rel=1e-6, abs=1e-10)


def test_draft_loss_soft_label_is_held_fixed():
    """The confidence term trains only the confidence head: the draft-logit gradient does
    not depend on its weight, and is the softmax Jacobian applied to the other terms."""
    zd, zt, labels, cl = _loss_case(13)
    g1 = oracle.draft_loss(zd, zt, labels, cl, (0.1, 0.9, 1.0))["grad_zd"]
    g0 = oracle.draft_loss(zd, zt, labels, cl, (0.1, 0.9, 0.0))["grad_zd"]
    np.testing.assert_array_equal(g1, g0)
    # softmax invariance: every row of the gradient sums to zero
    assert np.abs(g1.sum(axis=2)).max() < 1e-15


def test_draft_loss_cross_entropy_is_the_library_one():
    """With only the cross-entropy term on, the loss is the position-weighted mean of
    -log_softmax at the labels (scipy), and the gradient is softmax minus one-hot."""
    zd, zt, labels, cl = _loss_case(14, B=3, G=4, V=9)
    r = oracle.draft_loss(zd, zt, labels, cl, (1.0, 0.0, 0.0))
    ls = special.log_softmax(zd, axis=2)
    ce = -np.take_along_axis(ls, labels[..., None], axis=2)[..., 0]
    w = np.exp(-np.arange(4) / 4.0)
    assert r["loss"] == pytest.approx((ce * w).sum() / (3 * w.sum()), rel=1e-13)
    np.testing.assert_allclose(r["terms"][..., 0], ce, rtol=1e-13)
    onehot = np.eye(9)[labels]
    np.testing.assert_allclose(r["grad_zd"], (np.exp(ls) - onehot) * w[None, :, None] /
                               (3 * w.sum()), rtol=1e-12, atol=1e-16)


def test_draft_loss_identical_distributions():
    """p_d = p_t (draft logits shifted per row): no L1 term, soft label 1, so the
    confidence term is -log sigmoid(l) (scipy's log_expit) and its gradient c - 1."""
    _, zt, labels, cl = _loss_case(15)
    zd = zt + np.arange(6).reshape(2, 3, 1) * 0.37
    r = oracle.draft_loss(zd, zt, labels, cl, ALPHAS)
    assert np.abs(r["terms"][..., 1]).max() < 1e-14
    np.testing.assert_allclose(r["terms"][..., 2], -special.log_expit(cl), rtol=1e-13)
    w = np.exp(-np.arange(3) / 3.0)
    np.testing.assert_allclose(r["grad_conf"], (special.expit(cl) - 1.0) * w / (2 * w.sum()),
                               rtol=1e-12)
    # identical logits: every difference is exactly zero, its sign taken as 0, so the L1
    # term adds nothing to the gradient
    g_l1 = oracle.draft_loss(zt.copy(), zt, labels, cl, (0.0, 1.0, 0.0))["grad_zd"]
    assert np.abs(g_l1).max() == 0.0


def test_draft_loss_disjoint_distributions():
    """Draft and target put their mass on different tokens: L1 -> 2, soft label -> 0, so
    the confidence term is softplus(l) = -log(1 - sigmoid(l))."""
    V = 6
    zd = np.full((1, 1, V), -60.0)
    zt = np.full((1, 1, V), -60.0)
    zd[0, 0, 1] = 0.0
    zt[0, 0, 4] = 0.0
    cl = np.array([[0.8]])
    r = oracle.draft_loss(zd, zt, np.array([[4]]), cl, ALPHAS)
    assert r["terms"][0, 0, 1] == pytest.approx(2.0, abs=1e-15)
    assert r["terms"][0, 0, 2] == pytest.approx(-special.log_expit(-0.8), rel=1e-12)
    assert r["terms"][0, 0, 0] == pytest.approx(60.0, rel=1e-12)


# ------------------------------------------------------------------------------------
# stand-in target of the closed loop
# ------------------------------------------------------------------------------------
def test_markov_target_rows_and_previous_token():
    """sigma = 0: the target rows are the base rows, the last one repeated for position
    gamma + 1.  sigma > 0: the transition term depends on the previous token alone."""
    B, G, V = 2, 3, 64
    U = np.arange(B * G, dtype=np.float64).reshape(B, G, 1) * np.ones((1, 1, V))
    anchor = np.array([5, 9])
    tokens = np.array([[9, 5, 5], [7, 9, 5]])
    T0 = oracle.markov_target(U, anchor, tokens, 0.0, 1)
    np.testing.assert_array_equal(T0[:, :G], U)
    np.testing.assert_array_equal(T0[:, G], U[:, G - 1])
    T = oracle.markov_target(U, anchor, tokens, 0.8, 1)
    term = T - np.concatenate([U, U[:, G - 1:]], axis=1)
    prev = np.concatenate([anchor[:, None], tokens], axis=1)   # prev of positions 1..G+1
    for tok in (5, 9):
        rows = [term[b, j] for b in range(B) for j in range(G + 1) if prev[b, j] == tok]
        assert len(rows) >= 3
        for r_ in rows[1:]:
            np.testing.assert_allclose(r_, rows[0], rtol=0, atol=1e-14)   # base + term - base
    assert not np.array_equal(term[0, 0], term[0, 1])          # prev 5 vs prev 9
    assert np.abs(term).max() <= 0.8 * np.sqrt(3.0)


def test_markov_target_term_moments():
    """The transition term is uniform on [-sigma sqrt 3, sigma sqrt 3]: mean 0, variance
    sigma^2 (65536 draws: 6-sigma bounds)."""
    V = 65536
    U = np.zeros((1, 1, V))
    T = oracle.markov_target(U, np.array([17]), np.zeros((1, 1), np.int64), 1.3, 99)
    x = T[0, 0]
    assert abs(x.mean()) < 6 * 1.3 / np.sqrt(V)
    assert abs(x.var() / 1.3 ** 2 - 1.0) < 6 * np.sqrt(0.8 / V)
    h, _ = np.histogram(x, bins=16, range=(-1.3 * np.sqrt(3), 1.3 * np.sqrt(3)))
    assert stats.chisquare(h).pvalue > 1e-4
