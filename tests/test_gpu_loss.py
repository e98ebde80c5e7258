"""GPU parity of the distribution-matching training loss (forward and backward) against the
fp64 oracle.

Tolerances (fp32 kernel against the fp64 definition):
  loss                  relative 2e-5 (a sum of rows, each good to ~1e-6);
  ce, l1, bce per row   relative 1e-4 plus an absolute 2e-5 (ce: the fp32 normaliser
                        log sum exp is good to ~1e-6 absolute, which dominates a ce near 0);
  grad_conf             relative 1e-4 plus 1e-6 of the row weight;
  grad_zd               relative 1e-4 plus 1e-5 p_d(j) of the row weight (the fp32
                        probabilities and the row sum S carry ~1e-6 relative error), except
                        where p_d(j) and p_t(j) are equal to within 1e-5 relative: there the
                        sign of their difference (-1, 0 or +1) is a coin toss in fp32, and the
                        gradient of any of the three signs is accepted.
"""
import numpy as np
import pytest
import torch
from scipy import special

import draft_verify_sampling_step_amd as ds
import oracle
import workload

pytestmark = pytest.mark.gpu

ALPHAS = (0.1, 0.9, 1.0)


def _flush(msg):
    print(msg, flush=True)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    return t.detach().cpu().numpy()


def _case(B, G, V, seed, labels_oob=False, neg_inf_band=None):
    cfg = workload.custom(name="loss", B=B, gamma=G, V=V, logits="zipf", sigma0=0.3,
                          sigma1=0.05)
    tr = workload.training_inputs(cfg, seed)
    if labels_oob:
        tr.labels[0, 0] = -3
        tr.labels[-1, -1] = V + 7
    if neg_inf_band is not None:
        lo, hi = neg_inf_band
        tr.zd[..., lo:hi] = -np.inf
        tr.zt[..., lo:hi] = -np.inf
        bad = (tr.labels >= lo) & (tr.labels < hi)
        tr.labels[bad] = 0
    return tr


def _row_weights(B, G):
    w = np.exp(-np.arange(G) / G)
    return np.broadcast_to(w / (B * w.sum()), (B, G))


def check_loss(tr, rows=None, g=None, scale=1.0):
    """Compare GPU outputs g = (loss, terms, grad_zd, grad_conf) (host arrays, full batch)
    with the oracle on the requests `rows` (all when None).  scale: oracle gradients of a
    sub-batch are multiplied by it to match the full batch's normalisation."""
    zd, zt, labels, cl = tr.zd, tr.zt, tr.labels, tr.conf_logit
    B, G, V = zd.shape
    sel = np.arange(B) if rows is None else np.asarray(rows)
    o = oracle.draft_loss(zd[sel], zt[sel], labels[sel], cl[sel], ALPHAS)
    loss_g, terms_g, gz_g, gc_g = g
    if rows is None:
        assert abs(loss_g - o["loss"]) <= 2e-5 * abs(o["loss"]), (loss_g, o["loss"])
    t_o = o["terms"]
    t_g = terms_g[sel].astype(np.float64)
    for i, name in enumerate(("ce", "l1", "bce")):
        err = np.abs(t_g[..., i] - t_o[..., i])
        tol = 1e-4 * np.abs(t_o[..., i]) + 2e-5
        assert np.all(err <= tol), (name, float((err - tol).max()))
    wrow = _row_weights(B, G)[sel]
    gc_o = o["grad_conf"] * scale
    err = np.abs(gc_g[sel].astype(np.float64) - gc_o)
    assert np.all(err <= 1e-4 * np.abs(gc_o) + 1e-6 * wrow), float(err.max())

    gz_o = o["grad_zd"] * scale
    gz = gz_g[sel].astype(np.float64)
    pd = special.softmax(zd[sel].astype(np.float64), axis=2)
    pt = special.softmax(zt[sel].astype(np.float64), axis=2)
    near = np.abs(pd - pt) <= 1e-5 * np.maximum(pd, pt)
    w = wrow[..., None]
    tol = 1e-4 * np.abs(gz_o) + 1e-5 * pd * w * (ALPHAS[0] + ALPHAS[1]) + 1e-30
    ok = np.abs(gz - gz_o) <= tol
    # near-equal probabilities: the L1 term's sign may differ (-1, 0, +1), moving the
    # gradient by a multiple (-2..2) of alpha_l1 p_d(j) w
    step = ALPHAS[1] * pd * w
    ok_near = np.zeros_like(ok)
    for m in (-2, -1, 1, 2):
        ok_near |= np.abs(gz - (gz_o + m * step)) <= tol
    ok = ok | (near & ok_near)
    n_bad = int((~ok).sum())
    assert n_bad == 0, (n_bad, np.argwhere(~ok)[:5].tolist())
    return int(near.sum())


@pytest.mark.parametrize("B,G,V,seed,extra", [
    (2, 3, 5000, 1, {}),                         # two chunks per row, 16-byte path
    (3, 4, 10001, 2, {"labels_oob": True}),      # V % 4 != 0: direct loads; clamped labels
    (1, 1, 1, 3, {}),                            # one-token vocabulary: p_d = p_t = 1
    (2, 2, 4, 4, {}),                            # one quad
    (32, 16, 5000, 5, {}),                       # more rows than streams: rows claimed
    (2, 4, 9000, 6, {"neg_inf_band": (4400, 9000)}),   # a whole chunk at -inf
    (4, 16, 151936, 7, {}),                      # the full vocabulary, 38 chunks per row
    (1, 2, (1 << 22) - 5, 8, {}),                # the largest vocabulary: 512 chunks per
                                                 # row (each poller lane takes 8), V % 4 != 0
])
def test_draft_loss_matches_oracle(B, G, V, seed, extra):
    _flush(f"draft loss B={B} G={G} V={V} seed={seed} {extra}")
    tr = _case(B, G, V, seed, **extra)
    loss, terms, gz, gc = ds.dspark_draft_loss(dev(tr.zd), dev(tr.zt), dev(tr.labels),
                                               dev(tr.conf_logit), ALPHAS)
    g = (float(host(loss)[0]), host(terms), host(gz), host(gc))
    assert np.isfinite(g[0])
    check_loss(tr, g=g)


@pytest.mark.parametrize("alphas", [(1.0, 0.0, 0.0), (0.0, 1.0, 0.0), (0.0, 0.0, 2.5),
                                    (0.3, 0.3, 0.3)])
def test_draft_loss_term_weights(alphas):
    """Each term alone and other weights: the kernel takes the weights as arguments."""
    _flush(f"draft loss alphas={alphas}")
    tr = _case(3, 5, 7000, 9)
    loss, terms, gz, gc = ds.dspark_draft_loss(dev(tr.zd), dev(tr.zt), dev(tr.labels),
                                               dev(tr.conf_logit), alphas)
    o = oracle.draft_loss(tr.zd, tr.zt, tr.labels, tr.conf_logit, alphas)
    assert abs(float(host(loss)[0]) - o["loss"]) <= 2e-5 * abs(o["loss"]) + 1e-12
    w = _row_weights(3, 5)
    gz_o = o["grad_zd"]
    pd = special.softmax(tr.zd.astype(np.float64), axis=2)
    pt = special.softmax(tr.zt.astype(np.float64), axis=2)
    near = np.abs(pd - pt) <= 1e-5 * np.maximum(pd, pt)
    tol = 1e-4 * np.abs(gz_o) + 1e-5 * pd * w[..., None] * (alphas[0] + alphas[1]) + 1e-30
    step = alphas[1] * pd * w[..., None]
    ok = np.abs(host(gz) - gz_o) <= tol
    for m in (-2, -1, 1, 2):
        ok |= near & (np.abs(host(gz) - (gz_o + m * step)) <= tol)
    assert ok.all()
    gc_o = o["grad_conf"]
    assert np.all(np.abs(host(gc) - gc_o) <= 1e-4 * np.abs(gc_o) + 1e-6 * w)


def test_draft_loss_forward_only_and_deterministic():
    tr = _case(8, 16, 20000, 8)
    args = (dev(tr.zd), dev(tr.zt), dev(tr.labels), dev(tr.conf_logit), ALPHAS)
    l1, t1, g1, c1 = ds.dspark_draft_loss(*args)
    l2, t2, g2, c2 = ds.dspark_draft_loss(*args)
    l3, t3, g3, c3 = ds.dspark_draft_loss(*args, grads=False)
    assert g3 is None and c3 is None
    assert torch.equal(l1, l2) and torch.equal(t1, t2) and torch.equal(g1, g2)
    assert torch.equal(c1, c2)
    assert torch.equal(l1, l3) and torch.equal(t1, t3)


@pytest.mark.timeout(600)
def test_draft_loss_full_size_sampled():
    """B=128, gamma=16, V=151936 (the serving batch's training counterpart) in the launch
    configuration the benchmark times; three requests checked against the oracle."""
    cfg = workload.CONFIGS["serve128"]
    _flush("draft loss full size: generating inputs")
    tr = workload.training_inputs(cfg, 0)
    loss, terms, gz, gc = ds.dspark_draft_loss(dev(tr.zd), dev(tr.zt), dev(tr.labels),
                                               dev(tr.conf_logit), ALPHAS)
    torch.cuda.synchronize()
    rows = [0, cfg.B // 2, cfg.B - 1]
    _flush(f"draft loss full size: oracle on requests {rows}")
    g = (float(host(loss)[0]), host(terms), host(gz), host(gc))
    assert np.isfinite(g[0])
    # the oracle's call on 3 requests normalises by 3 sum w instead of B sum w
    check_loss(tr, rows=rows, g=g, scale=len(rows) / cfg.B)
    # the loss is the weighted mean of the rows: check it against the GPU's own terms
    w = _row_weights(cfg.B, cfg.gamma)
    t = g[1].astype(np.float64)
    recon = float((w * (ALPHAS[0] * t[..., 0] + ALPHAS[1] * t[..., 1] +
                        ALPHAS[2] * t[..., 2])).sum())
    assert abs(recon - g[0]) <= 1e-5 * abs(g[0])
