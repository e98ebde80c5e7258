"""The bounded waits of the cooperative kernels -- the resident draft (up to 16 requests: one
launch for all positions, a hand-off across the chip between positions) and the training
loss (a stream of workgroups per row, an exchange per row).

dspark_test_wait_limit forces the failure path from the host: every wait gives up after a
few polls because the completion it looks for is made unreachable.  The call must then
report its failure in its outputs (draft: every token -1, logp and lse NaN; loss: NaN)
while every kernel ends; with normal operation restored, the next call must be exactly the
call before the failure (the fault word is cleared per call, nothing else is left behind).
"""
import numpy as np
import pytest
import torch

import draft_verify_sampling_step_amd as ds
import workload

pytestmark = pytest.mark.gpu


def _flush(msg):
    print(msg, flush=True)


def host(t):
    return t.detach().cpu().numpy()


@pytest.mark.parametrize("B", [1, 4])
def test_resident_draft_reports_a_wait_that_gave_up(B):
    # bf16, rank 256, V % 4 == 0 and V <= 163840: the resident draft (one workgroup per
    # compute unit); B = 1 hands the winners over through per-workgroup slots, B = 4
    # through the two-level arrival counter
    cfg = workload.custom(name="waits", B=B, gamma=4, V=8192, r=256, d=64, bf16=True,
                          wsigma=0.3)
    inp = workload.generate(cfg, 2)
    U, W1, W2t, anchor = (ds.to_device(x) for x in (inp.U, inp.W1, inp.W2t, inp.anchor))
    _flush(f"resident draft, B={B}: normal call")
    t0, l0, s0 = (host(x) for x in ds.dspark_draft_markov(U, W1, W2t, anchor, 1.0, inp.seed))
    assert (t0 >= 0).all() and np.isfinite(l0).all() and np.isfinite(s0).all()
    try:
        ds.dspark_test_wait_limit(8)
        _flush(f"resident draft, B={B}: every wait gives up after 8 polls")
        t1, l1, s1 = (host(x) for x in ds.dspark_draft_markov(U, W1, W2t, anchor, 1.0,
                                                              inp.seed))
    finally:
        ds.dspark_test_wait_limit(-1)
    torch.cuda.synchronize()
    assert (t1 == -1).all()
    assert np.isnan(l1).all() and np.isnan(s1).all()
    _flush(f"resident draft, B={B}: normal operation restored")
    t2, l2, s2 = (host(x) for x in ds.dspark_draft_markov(U, W1, W2t, anchor, 1.0, inp.seed))
    assert np.array_equal(t2, t0) and np.array_equal(l2, l0) and np.array_equal(s2, s0)


def test_training_loss_reports_a_wait_that_gave_up():
    cfg = workload.custom(name="loss", B=2, gamma=3, V=20000, logits="zipf", sigma0=0.3,
                          sigma1=0.05)
    tr = workload.training_inputs(cfg, 4)
    zd, zt, lab, cf = (torch.from_numpy(np.ascontiguousarray(a)).cuda()
                       for a in (tr.zd, tr.zt, tr.labels, tr.conf_logit))
    _flush("training loss: normal call")
    loss0, _, g0, _ = ds.dspark_draft_loss(zd, zt, lab, cf)
    loss0, g0 = host(loss0), host(g0)
    assert np.isfinite(loss0).all()
    try:
        ds.dspark_test_wait_limit(8)
        _flush("training loss: every wait gives up after 8 polls")
        loss1 = host(ds.dspark_draft_loss(zd, zt, lab, cf)[0])
    finally:
        ds.dspark_test_wait_limit(-1)
    assert np.isnan(loss1).all()
    _flush("training loss: normal operation restored")
    loss2, _, g2, _ = ds.dspark_draft_loss(zd, zt, lab, cf)
    assert np.array_equal(host(loss2), loss0) and np.array_equal(host(g2), g0)
