#!/usr/bin/env python3
"""Throughput of one DSpark draft/verify round on one MI355X.

A step is one pass of the whole hot path over one batch: Markov-head draft (gamma positions)
-> confidence head -> greedy prefix scheduler -> rejection-sampling verification (+ the TV
accept rate for workloads that ask for it).  Inputs are resident in HBM before timing; the
target logits (the stand-in for the target model's forward) are synthesised once, untimed,
from the round's drafted tokens -- every step re-drafts the identical tokens (same seed).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload serve128]

Prints one JSON line.  `value` = drafted+verified positions per second = B * gamma / step,
the step timed as one HIP-graph replay of the eager step (its outputs checked against the
eager step's in the same run; `ms_per_step_eager` is the eager time).
`roofline` covers the dominant kernel, one draft position: its algorithmic bytes (W2t once
and the B base-logit rows of the position) over its mean launch duration, measured with
HIP events on the launch stream in a timed pass of its own (one pair around the gamma
consecutive launches of each call, the span over gamma, dispatch gaps included); beside it,
`read_probe` is a plain streaming read of the same bytes per launch, the achievable rate.
`cpu_baseline` times the fp64 oracle on a bounded sample of requests on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
METRIC = "draft+verify positions/s at B=128,gamma=16,V=151936; % of HBM peak BW"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="serve128")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target length of the oracle CPU-baseline sample")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device-to-device copy three times (the "
                         "reference for scaling hardware byte counters), then the benchmark")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the round is "
              "sharded by request across GPUs by design, but no multi-GPU path is built.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_verify_sampling_step_amd as ds
    import workload

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n // 4, dtype=torch.float32, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        torch.cuda.empty_cache()
        log(f"copy calibration: 3 device copies of {n} bytes")

    if not os.path.exists(ds.LIB_PATH):   # fail loudly before any work
        raise RuntimeError(f"{ds.LIB_PATH} is missing: build it first (__graft_entry__.build())")
    cfg = workload.CONFIGS[args.workload]
    B, G, V, r, d = cfg.B, cfg.gamma, cfg.V, cfg.r, cfg.d
    temp = cfg.temperature

    t0 = time.time()
    log(f"generating {cfg.name} inputs")
    inp = workload.generate(cfg, args.seed)
    # the oracle baseline runs first, on the host only: its worker processes are forked
    # before this process makes any GPU call
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the oracle on the host")
        cpu = cpu_baseline(inp, args.cpu_seconds)

    ds.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    U = ds.to_device(inp.U)
    W1 = ds.to_device(inp.W1)
    W2t = ds.to_device(inp.W2t)
    h = ds.to_device(inp.h)
    w = ds.to_device(inp.w)
    anchor = ds.to_device(inp.anchor)
    sps = ds.to_device(inp.sps)
    stream = torch.cuda.current_stream()

    # outputs and workspaces allocated once
    tokens = torch.empty((B, G), dtype=torch.int32, device=dev)
    logp = torch.empty((B, G), dtype=torch.float32, device=dev)
    lse = torch.empty((B, G), dtype=torch.float32, device=dev)
    conf = torch.empty((B, G), dtype=torch.float32, device=dev)
    ell = torch.empty(B, dtype=torch.int32, device=dev)
    theta = torch.empty(1, dtype=torch.float64, device=dev)
    ntot = torch.empty(1, dtype=torch.int32, device=dev)
    nacc = torch.empty(B, dtype=torch.int32, device=dev)
    outtok = torch.empty((B, G + 1), dtype=torch.int32, device=dev)
    alpha = torch.empty((B, G), dtype=torch.float32, device=dev)
    ws_d = torch.empty(ds.workspace_bytes(ds.OP_DRAFT, B, G, V, r), dtype=torch.uint8, device=dev)
    ws_v = torch.empty(ds.workspace_bytes(ds.OP_VERIFY, B, G, V, r), dtype=torch.uint8, device=dev)
    ws_t = torch.empty(max(256, ds.workspace_bytes(ds.OP_TV, B, G, V, r)), dtype=torch.uint8,
                       device=dev)

    # untimed: draft once, synthesise the target logits for those tokens
    ds.dspark_draft_markov(U, W1, W2t, anchor, temp, inp.seed, out=(tokens, logp, lse), ws=ws_d)
    torch.cuda.synchronize()
    log("synthesising target logits")
    T = ds.to_device(workload.synthesize_target(inp, tokens.cpu().numpy()))
    log(f"inputs ready in {time.time() - t0:.1f}s")

    ev_d0 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_d1 = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]

    def step(i=None):
        if i is not None:
            ev_d0[i].record(stream)
        ds.dspark_draft_markov(U, W1, W2t, anchor, temp, inp.seed, out=(tokens, logp, lse),
                               ws=ws_d)
        if i is not None:
            ev_d1[i].record(stream)
        ds.dspark_confidence(h, W1, w, anchor, tokens, out=conf)
        ds.dspark_schedule(conf, sps, cfg.sched_mode, out=(ell, theta, ntot))
        ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, inp.seed,
                         out=(nacc, outtok, None), ws=ws_v)
        if cfg.tv:
            ds.dspark_accept_rate_tv(U, W1, W2t, anchor, tokens, lse, T, temp, out=alpha,
                                     ws=ws_t)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    wall0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = e0.elapsed_time(e1) / args.steps
    draft_ms = float(np.mean([a.elapsed_time(b) for a, b in zip(ev_d0, ev_d1)]))
    log(f"timed {args.steps} steps: {ms_step:.3f} ms/step (wall {wall * 1e3 / args.steps:.3f}), "
        f"draft {draft_ms:.3f} ms")

    # the same step captured once in a HIP graph (every call launches on the current stream
    # and none uses a memset), replayed; each replay is checked against the eager outputs,
    # with eager work between replays, before its time is used
    outs = (tokens, logp, lse, conf, ell, theta, ntot, nacc, outtok) + ((alpha,) if cfg.tv else ())
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in outs]
    graph_ok, graph_note = False, ""
    try:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph_ok = True
        for _ in range(4):
            for t in outs:
                t.fill_(-7)
            graph.replay()
            torch.cuda.synchronize()
            graph_ok = graph_ok and all(torch.equal(a, b) for a, b in zip(ref, outs))
            step()
            torch.cuda.synchronize()
        if not graph_ok:
            graph_note = "a replay differed from the eager step"
    except RuntimeError as exc:          # capture refused: report the eager time only
        graph_note = f"capture failed: {exc}"
        graph_ok = False
    ms_step_eager = ms_step
    ms_step_mean = ms_step
    if graph_ok:
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        gev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        gev[0].record(stream)
        for i in range(args.steps):
            graph.replay()
            gev[i + 1].record(stream)
        torch.cuda.synchronize()
        per_step = [gev[i].elapsed_time(gev[i + 1]) for i in range(args.steps)]
        ms_step_mean = gev[0].elapsed_time(gev[-1]) / args.steps
        ms_step = float(np.median(per_step))
        log(f"graph replay: median {ms_step:.3f} ms/step, mean {ms_step_mean:.3f} "
            f"(eager {ms_step_eager:.3f})")
        del graph
    else:
        log(f"graph replay not used: {graph_note}")

    # the dominant kernel, one draft position (fused bias MFMA + softmax + Gumbel race):
    # HIP events around the consecutive launches of each call on the launch stream (the
    # span over the launch count, dispatch gaps included), in a pass of its own so
    # that the events do not perturb the step timing above
    ds.dspark_profile_start(args.steps * G + 16)
    for _ in range(args.steps):
        ds.dspark_draft_markov(U, W1, W2t, anchor, temp, inp.seed, out=(tokens, logp, lse),
                               ws=ws_d)
    kern_ms, kern_n, kern_pos = ds.dspark_profile_stop()
    log(f"draft sampling kernel: {kern_ms * 1e3:.2f} us mean over {kern_n} launches of "
        f"{kern_pos:g} positions each")

    # the achievable read rate at the same bytes per launch: a plain streaming-read kernel
    # over four rotating regions (so that consecutive launches miss the caches)
    probe_bytes = (V * r * 2 + B * V * 4) // 16 * 16
    probe_buf = torch.empty(4 * probe_bytes, dtype=torch.uint8, device=dev)
    probe_ms = ds.dspark_stream_read_probe(probe_buf, probe_bytes, reps=40)
    del probe_buf
    probe_gbs = probe_bytes / (probe_ms * 1e-3) / 1e9
    log(f"plain streaming read of {probe_bytes} bytes: {probe_ms * 1e3:.2f} us "
        f"({probe_gbs:.0f} GB/s)")

    # verification alone (rows pass, decisions, residual pass, final), same inputs as a step
    vf0 = torch.cuda.Event(enable_timing=True)
    vf1 = torch.cuda.Event(enable_timing=True)
    vf0.record(stream)
    for _ in range(args.steps):
        ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, inp.seed,
                         out=(nacc, outtok, None), ws=ws_v)
    vf1.record(stream)
    torch.cuda.synchronize()
    verify_ms = vf0.elapsed_time(vf1) / args.steps
    verify_ms_eager = verify_ms
    # the same call as a graph replay (host launch overhead excluded), checked against the
    # eager outputs first
    if graph_ok:
        vref = (nacc.clone(), outtok.clone())
        vside = torch.cuda.Stream()
        vside.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(vside):
            ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, inp.seed,
                             out=(nacc, outtok, None), ws=ws_v)
        torch.cuda.current_stream().wait_stream(vside)
        torch.cuda.synchronize()
        vgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(vgraph):
            ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, inp.seed,
                             out=(nacc, outtok, None), ws=ws_v)
        nacc.fill_(-7)
        outtok.fill_(-7)
        vgraph.replay()
        torch.cuda.synchronize()
        if torch.equal(vref[0], nacc) and torch.equal(vref[1], outtok):
            vf0.record(stream)
            for _ in range(args.steps):
                vgraph.replay()
            vf1.record(stream)
            torch.cuda.synchronize()
            verify_ms = vf0.elapsed_time(vf1) / args.steps
        del vgraph

    # verification at the full block (ell = gamma for every request: the budget's upper
    # bound, every target row read), as a checked graph replay like the call above
    ell_full = torch.full((B,), G, dtype=torch.int32, device=dev)
    vfull_ms, vfull_rej = timed_verify(ds, args, stream, graph_ok, U, W1, W2t, anchor, tokens,
                                       logp, lse, T, ell_full, temp, inp.seed, nacc, outtok,
                                       ws_v)
    vfull_bytes = B * (G + 1) * V * 4 + ((V * r * 2 + vfull_rej * 2 * V * 4) if vfull_rej else 0)

    # the target side of a closed-loop round on its own: the stand-in target's logits for
    # this round's block (sigma 0.5, as in the loop below), then verification on them at
    # this round's schedule -- timed apart from the loop, for the latency model
    T_loop = torch.empty((B, G + 1, V), dtype=torch.float32, device=dev)
    ds.dspark_markov_target(U, anchor, tokens, 0.5, 1, out=T_loop)
    tt0 = torch.cuda.Event(enable_timing=True)
    tt1 = torch.cuda.Event(enable_timing=True)
    tt0.record(stream)
    for _ in range(args.steps):
        ds.dspark_markov_target(U, anchor, tokens, 0.5, 1, out=T_loop)
    tt1.record(stream)
    torch.cuda.synchronize()
    target_ms = tt0.elapsed_time(tt1) / args.steps
    vloop_ms, _ = timed_verify(ds, args, stream, False, U, W1, W2t, anchor, tokens, logp, lse,
                               T_loop, ell, temp, inp.seed, nacc, outtok, ws_v)
    del T_loop
    torch.cuda.empty_cache()

    # the draft side of a round alone (draft, confidence, schedule)
    ds0 = torch.cuda.Event(enable_timing=True)
    ds1 = torch.cuda.Event(enable_timing=True)
    ds0.record(stream)
    for _ in range(args.steps):
        ds.dspark_draft_markov(U, W1, W2t, anchor, temp, inp.seed, out=(tokens, logp, lse),
                               ws=ws_d)
        ds.dspark_confidence(h, W1, w, anchor, tokens, out=conf)
        ds.dspark_schedule(conf, sps, cfg.sched_mode, out=(ell, theta, ntot))
    ds1.record(stream)
    torch.cuda.synchronize()
    draft_side_ms = ds0.elapsed_time(ds1) / args.steps

    # closed loop: LOOP_R rounds chained on the device (next anchor = last emitted token)
    # with the synthetic Markov stand-in target (transition term sigma = 0.5); the loop's
    # latency per token is the round time over tau, the tokens a request gains per round
    LOOP_R = 8
    ds.dspark_closed_loop(U, W1, W2t, h, w, anchor, sps, 2, temp, inp.seed, cfg.sched_mode,
                          0.5, 1, pt_tok=False)
    lp0 = torch.cuda.Event(enable_timing=True)
    lp1 = torch.cuda.Event(enable_timing=True)
    lp0.record(stream)
    loop_out = ds.dspark_closed_loop(U, W1, W2t, h, w, anchor, sps, LOOP_R, temp, inp.seed,
                                     cfg.sched_mode, 0.5, 1, pt_tok=False)
    lp1.record(stream)
    torch.cuda.synchronize()
    loop_round_ms = lp0.elapsed_time(lp1) / LOOP_R
    loop_tau = (loop_out["n_accept"].double() + 1.0).mean(dim=1).cpu().numpy()
    del loop_out
    torch.cuda.empty_cache()

    # the production form of the scheduler (top-K admission, K from history): timed alone at
    # this round's admitted count; one workgroup, latency-bound, so reported in us only
    k_admit = int(ntot.cpu()[0]) - B
    topk_out = (torch.empty(B, dtype=torch.int32, device=dev),
                torch.empty(1, dtype=torch.float64, device=dev),
                torch.empty(1, dtype=torch.int32, device=dev))
    ds.dspark_schedule_topk(conf, sps, k_admit, out=topk_out)
    tk0 = torch.cuda.Event(enable_timing=True)
    tk1 = torch.cuda.Event(enable_timing=True)
    tk0.record(stream)
    for _ in range(args.steps):
        ds.dspark_schedule_topk(conf, sps, k_admit, out=topk_out)
    tk1.record(stream)
    torch.cuda.synchronize()
    topk_us = tk0.elapsed_time(tk1) * 1e3 / args.steps

    # sequential temperature scaling of the confidence head on a held-out set of this draft
    # length (synthetic, 131072 blocks, 256-value grid, 15 bins): fp64 sigmoid evaluations
    # dominate, n * grid * gamma of them
    cal = workload.calibration_inputs(131072, G, seed=args.seed)
    cal_logit, cal_acc = ds.to_device(cal.logit), ds.to_device(cal.n_accept)
    cal_grid = torch.tensor(np.geomspace(0.4, 5.0, 256), dtype=torch.float64, device=dev)
    ds.dspark_sts_calibrate(cal_logit, cal_acc, cal_grid, 15)
    sc0 = torch.cuda.Event(enable_timing=True)
    sc1 = torch.cuda.Event(enable_timing=True)
    sc0.record(stream)
    for _ in range(3):
        ds.dspark_sts_calibrate(cal_logit, cal_acc, cal_grid, 15)
    sc1.record(stream)
    torch.cuda.synchronize()
    sts_ms = sc0.elapsed_time(sc1) / 3

    # training side: the distribution-matching loss, forward and backward, over a batch of
    # this shape (B blocks of gamma positions, draft and target logits over V); HBM-bound at
    # 12 bytes per logit (read draft and target, write the gradient)
    log("training loss: generating a batch")
    tr = workload.training_inputs(cfg, args.seed)
    zd_t, zt_t = ds.to_device(tr.zd), ds.to_device(tr.zt)
    lab_t, cl_t = ds.to_device(tr.labels), ds.to_device(tr.conf_logit)
    del tr
    loss_out = (torch.empty(1, dtype=torch.float64, device=dev),
                torch.empty(B, G, 3, dtype=torch.float32, device=dev),
                torch.empty_like(zd_t), torch.empty(B, G, dtype=torch.float32, device=dev))
    for _ in range(2):
        ds.dspark_draft_loss(zd_t, zt_t, lab_t, cl_t, out=loss_out)
    lo0 = torch.cuda.Event(enable_timing=True)
    lo1 = torch.cuda.Event(enable_timing=True)
    lo0.record(stream)
    for _ in range(5):
        ds.dspark_draft_loss(zd_t, zt_t, lab_t, cl_t, out=loss_out)
    lo1.record(stream)
    torch.cuda.synchronize()
    loss_ms = lo0.elapsed_time(lo1) / 5
    loss_val = float(loss_out[0].cpu()[0])
    loss_bytes = B * G * V * 12
    del zd_t, zt_t, loss_out
    torch.cuda.empty_cache()

    # algorithmic bytes (what the method must move), from this round's realised ell, n
    ell_h = ell.cpu().numpy().astype(np.int64)
    n_h = nacc.cpu().numpy().astype(np.int64)
    w2t_bytes = V * r * 2
    draft_bytes = G * (w2t_bytes + B * V * 4)
    conf_bytes = B * G * (d + r) * 2
    n_rej = int((n_h < ell_h).sum())
    verify_bytes = int((ell_h + 1).sum()) * V * 4 + (w2t_bytes + n_rej * 2 * V * 4 if n_rej else 0)
    tv_bytes = (G * w2t_bytes + 3 * B * G * V * 4) if cfg.tv else 0
    step_bytes = draft_bytes + conf_bytes + verify_bytes + tv_bytes
    positions = B * G
    value = positions / (ms_step * 1e-3)
    pos_bytes = w2t_bytes + B * V * 4          # one position: W2t once, B base-logit rows
    launch_bytes = int(round(pos_bytes * kern_pos))
    achieved = launch_bytes / (kern_ms * 1e-3) / 1e9
    strict_bytes = int(round((w2t_bytes / G + B * V * 4) * kern_pos))
    strict_achieved = strict_bytes / (kern_ms * 1e-3) / 1e9
    ksrc = kernel_sources(B, V, r)
    traffic = measured_traffic(cfg.name, ksrc)
    mfma_util = measured_mfma_util(cfg.name, ksrc)

    rec = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "positions/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "ms_per_step_mean": round(ms_step_mean, 4),
        "ms_per_step_eager": round(ms_step_eager, 4),
        "launch": "HIP graph replay of the step (checked against the eager step)" if graph_ok
                  else f"eager ({graph_note})",
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16+f32",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: B={B} gamma={G} V={V} r={r} d={d} bf16 weights, fp32 "
                        f"logits, temperature {temp}, "
                        f"{'greedy scheduler' if cfg.sched_mode == 0 else 'full-block verify'}",
            "global_batch": B, "gamma": G, "vocab": V, "rank": r, "hidden": d,
            "parallelism": "single GPU",
        },
        "roofline": {
            "kernel": draft_kernel_name(B, V, r) + ": fused bias + softmax + Gumbel race "
                      "over W2t and the B base-logit rows, "
                      + ("one draft position per launch" if kern_pos == 1 else
                         f"{kern_pos:g} draft positions per launch"),
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "bytes_per_launch": launch_bytes,
            "positions_per_launch": kern_pos,
            "ms_per_launch": round(kern_ms, 5),
            "launches": kern_n,
            "read_probe": {
                "kind": "plain 16-byte streaming read of the same bytes per launch, four "
                        "rotating regions",
                "achieved": round(probe_gbs, 1),
                "ms_per_launch": round(probe_ms, 5),
                "bytes_per_launch": probe_bytes,
            },
            "frac_of_read_probe": round(achieved / probe_gbs, 4),
            "strict": {
                "kind": "W2t counted once per round (gamma positions) instead of once per "
                        "position, so that on-die reuse of W2t across positions cannot "
                        "inflate the fraction",
                "bytes_per_launch": strict_bytes,
                "achieved": round(strict_achieved, 1),
                "frac": round(strict_achieved / HBM_PEAK_GBS, 4),
            },
            "mfma_util": mfma_util,
        },
        "draft_call_ms": round(draft_ms, 4),
        "verify_call_ms": round(verify_ms, 4),
        "verify_call_ms_eager": round(verify_ms_eager, 4),
        "verify_hbm_frac": round(verify_bytes / (verify_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "verify_full_block_ms": round(vfull_ms, 4),
        "verify_full_block_hbm_frac": round(vfull_bytes / (vfull_ms * 1e-3) / 1e9 /
                                            HBM_PEAK_GBS, 4),
        "verify_full_block_rejections": vfull_rej,
        "step_hbm_frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "step_bytes": step_bytes,
        "schedule_topk_us": round(topk_us, 2),
        "sts_calibrate_ms": round(sts_ms, 4),
        "sts_sigmoids_per_s": round(131072 * 256 * G / (sts_ms * 1e-3), 1),
        "loop_rounds": LOOP_R,
        "loop_round_ms": round(loop_round_ms, 4),
        "loop_draft_side_ms": round(draft_side_ms, 4),
        "loop_target_side_ms": round(target_ms + vloop_ms, 4),
        "loop_target_side_parts_ms": {"stand_in_target": round(target_ms, 4),
                                      "verify": round(vloop_ms, 4)},
        "loop_tau_per_round": [round(float(x), 3) for x in loop_tau],
        "loop_tau": round(float(loop_tau.mean()), 4),
        "loop_ms_per_token": round(loop_round_ms / float(loop_tau.mean()), 4),
        "loop_eq1_ms_per_token": round((draft_side_ms + target_ms + vloop_ms) /
                                       float(loop_tau.mean()), 4),
        "loop_tokens_per_s": round(B * float(loop_tau.mean()) / (loop_round_ms * 1e-3), 1),
        "loss_call_ms": round(loss_ms, 4),
        "loss_hbm_frac": round(loss_bytes / (loss_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "loss_value": round(loss_val, 6),
        "accepted_mean": round(float(n_h.mean()), 3),
        "verify_tokens": int((ell_h + 1).sum()),
    }

    if cpu is not None:
        single, parallel = cpu
        rec["cpu_baseline"] = single
        if parallel is not None:
            rec["cpu_baseline_all_cores"] = parallel
    print(json.dumps(rec), flush=True)

    # release what this run holds on the device before the interpreter exits: every stream
    # drained, device tensors and events dropped, the allocator's cache and the binding's
    # workspaces returned
    torch.cuda.synchronize()
    del U, W1, W2t, h, w, anchor, sps, T, tokens, logp, lse, conf, ell, theta, ntot, nacc
    del outtok, alpha, ws_d, ws_v, ws_t, ev_d0, ev_d1, e0, e1
    import gc
    gc.collect()
    ds.release_cached_workspaces()


# the dominant kernel's source files, hashed in this order (the counter summary names it)
def kernel_sources(B: int, V: int, r: int):
    """The sources of the draft kernel this shape runs, whose sha256 binds the committed
    counter summaries to it."""
    if draft_kernel_name(B, V, r).startswith("k_draft_resident"):
        return ("resident.hip", "mfma_common.h")
    return ("mfma16.hip", "mfma_common.h")


def measured_traffic(workload_name: str, sources):
    """HBM bytes per launch of the draft position kernel from the committed counter
    summary (FETCH_SIZE + WRITE_SIZE, scaled by the copy-kernel calibration), or None when
    there is none for this workload or the kernel source has changed since it was taken."""
    import hashlib
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    path = os.path.join(here, "profiles", f"draft_position_{workload_name}_pmc.md")
    csrc = os.path.join(here, "draft_verify_sampling_step_amd", "csrc")
    srcs = [os.path.join(csrc, f) for f in sources]
    if not (os.path.exists(path) and all(os.path.exists(f) for f in srcs)):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel source sha256:\s*([0-9a-f]{64})", text)
    m_b = re.search(r"traffic bytes per launch:\s*([0-9]+)", text)
    if not (m_sha and m_b):
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    if h.hexdigest() != m_sha.group(1):
        return None
    return int(m_b.group(1))


def _sha_bound_figure(path: str, pattern: str, sources):
    """A figure from a committed counter summary, or None when the summary is missing or the
    draft kernel's source has changed since it was taken (its sha256 is recorded in it)."""
    import hashlib
    import re
    here = os.path.dirname(os.path.abspath(__file__))
    csrc = os.path.join(here, "draft_verify_sampling_step_amd", "csrc")
    srcs = [os.path.join(csrc, f) for f in sources]
    if not (os.path.exists(path) and all(os.path.exists(f) for f in srcs)):
        return None
    text = open(path).read()
    m_sha = re.search(r"kernel source sha256:\s*([0-9a-f]{64})", text)
    m_v = re.search(pattern, text)
    if not (m_sha and m_v):
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(f, "rb").read())
    return m_v.group(1) if h.hexdigest() == m_sha.group(1) else None


def measured_mfma_util(workload_name: str, sources):
    """Matrix-core busy fraction of the draft position kernel (SQ counters, from the
    committed summary bound to the kernel source), or None."""
    here = os.path.dirname(os.path.abspath(__file__))
    v = _sha_bound_figure(os.path.join(here, "profiles", f"draft_position_{workload_name}_mfma.md"),
                          r"matrix-core busy fraction:\s*([0-9.]+)", sources)
    return None if v is None else float(v)


def timed_verify(ds, args, stream, use_graph, U, W1, W2t, anchor, tokens, logp, lse, T, ell,
                 temp, seed, nacc, outtok, ws_v):
    """Mean time of dspark_verify on these inputs (a graph replay checked against the eager
    call when use_graph, else eager) and the number of rejected requests."""
    import torch
    ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, seed,
                     out=(nacc, outtok, None), ws=ws_v)
    torch.cuda.synchronize()
    rej = int((nacc < ell.clamp(0, tokens.shape[1])).sum().item())
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    if use_graph:
        vref = (nacc.clone(), outtok.clone())
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, seed,
                             out=(nacc, outtok, None), ws=ws_v)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, seed,
                             out=(nacc, outtok, None), ws=ws_v)
        nacc.fill_(-7)
        outtok.fill_(-7)
        g.replay()
        torch.cuda.synchronize()
        if torch.equal(vref[0], nacc) and torch.equal(vref[1], outtok):
            e0.record(stream)
            for _ in range(args.steps):
                g.replay()
            e1.record(stream)
            torch.cuda.synchronize()
            del g
            return e0.elapsed_time(e1) / args.steps, rej
        del g
    e0.record(stream)
    for _ in range(args.steps):
        ds.dspark_verify(U, W1, W2t, anchor, tokens, logp, lse, T, ell, temp, seed,
                         out=(nacc, outtok, None), ws=ws_v)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / args.steps, rej


def draft_kernel_name(B: int, V: int, r: int) -> str:
    """The draft position kernel the library dispatches for this shape (bf16 weights)."""
    if r == 256 and B <= 16 and V % 4 == 0 and V <= 256 * 40 * 16:
        return "k_draft_resident (W2t held in accumulation registers and LDS for all gamma " \
            "positions, one cooperative launch per draft call)"
    if r == 256 and B == 1 and V % 4 == 0:
        return "k_draft_gemv (streaming kernel for one request, one vocabulary range per " \
            "workgroup)"
    if r == 256 and 32 < B <= 256 and V % 4 == 0:
        nw = 4 if B <= 64 else (8 if B <= 128 else 16)
        return f"k_draft16<{nw}, false>" + \
            " (16x16x32 bf16 MFMA, 16-column waves)"
    if r == 256:
        return "k_mfma_bias<NCB, draft> (32x32x16 bf16 MFMA, 32-column waves)"
    return "k_draft_row (row kernel, one request per workgroup row)"


def cpu_baseline(inp, budget_s: float):
    """The fp64 oracle, single-threaded, on the first S requests of the same workload
    (full vocabulary, all positions): draft, confidence, schedule over those S, verify.
    Target logits for the sample are synthesised from the oracle's own tokens, untimed."""
    import oracle
    import workload

    cfg = inp.cfg
    G = cfg.gamma
    temp = cfg.temperature

    def run(rows):
        t_draft = time.perf_counter()
        od = oracle.draft(inp.U[rows], inp.W1, inp.W2t, inp.anchor[rows], temp, inp.seed,
                          gid=rows)
        c = oracle.confidence(inp.h[rows], inp.W1, inp.w, inp.anchor[rows], od["tokens"])
        sps = 1000.0 / workload.step_time_ms(cfg.table, np.arange(len(rows) * (G + 1) + 1))
        ell, _, _ = oracle.schedule(c.astype(np.float32), sps, cfg.sched_mode)
        t_mid = time.perf_counter()
        T = workload.synthesize_target(inp, _tokens_full(cfg, rows, od["tokens"]), rows=rows)
        t_ver = time.perf_counter()
        oracle.verify(inp.U[rows], inp.W1, inp.W2t, inp.anchor[rows], od["tokens"], T, ell,
                      temp, inp.seed, gid=rows)
        if cfg.tv:
            oracle.accept_tv(inp.U[rows], inp.W1, inp.W2t, inp.anchor[rows], od["tokens"], T,
                             temp)
        t_end = time.perf_counter()
        return (t_mid - t_draft) + (t_end - t_ver)

    t1 = run(np.array([0]))
    S = int(max(1, min(cfg.B, budget_s // max(t1, 1e-3))))
    rows = np.arange(S)
    secs = run(rows) if S > 1 else t1
    what = (f"draft+confidence+schedule+verify{'+TV' if cfg.tv else ''} in fp64 "
            f"(all {G} positions, full V={cfg.V})")
    single = {
        "value": round(S * G / secs, 3),
        "unit": "positions/s",
        "cores": 1,
        "kind": "oracle",
        "sample": f"requests 0..{S - 1} of {cfg.name}: {what}, {secs:.1f} s on 1 thread",
    }
    # the same oracle over disjoint request shards in worker processes, one per host core
    # (at most 16): each shard runs the per-request path above on its own requests
    try:
        ncores = len(os.sched_getaffinity(0))
    except AttributeError:
        ncores = os.cpu_count() or 1
    ncores = max(1, min(16, ncores))
    parallel = None
    if ncores > 1 and S < cfg.B:
        import multiprocessing as mp
        SP = int(min(cfg.B, S * ncores))
        shards = [a for a in np.array_split(np.arange(SP), ncores) if len(a)]
        global _PAR_RUN
        _PAR_RUN = run
        ctx = mp.get_context("fork")
        t0 = time.perf_counter()
        with ctx.Pool(len(shards)) as pool:
            pool.map(_par_shard, shards)
        wall = time.perf_counter() - t0
        parallel = {
            "value": round(SP * G / wall, 3),
            "unit": "positions/s",
            "cores": len(shards),
            "kind": "oracle",
            "sample": f"requests 0..{SP - 1} of {cfg.name} in {len(shards)} shards: {what}, "
                      f"{wall:.1f} s wall on {len(shards)} processes",
        }
    return single, parallel


_PAR_RUN = None


def _par_shard(rows):
    return _PAR_RUN(rows)


def _tokens_full(cfg, rows, toks):
    full = np.zeros((cfg.B, cfg.gamma), np.int32)
    full[rows] = toks
    return full


if __name__ == "__main__":
    main()
