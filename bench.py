"""Benchmark of the TokenGate gate-layer hot path on one MI355X.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]

One step = the whole prefill path of one gate layer on one batch of synthetic
input, back to back on one HIP stream with no host synchronisation:
    tg_gate_score -> tg_select_topk -> tg_compact -> tg_gated_attn_fwd
(tg_gate_score called as its two halves, tg_gate_pack_w1 + tg_gate_score_packed,
so that each kernel has its own events) on the long-context workload (batch 1, N = 32768 context tokens, 128 scaffold
tokens, K = 2048 kept documents -> M = 2176, hidden 2048, scorer 2048->512->1,
16/8 heads, head dim 128, bf16, RoPE at the original positions).  Selection
ranks a drawn score vector with high-score spans over ~5% of the documents.

Inputs are resident in HBM before timing starts.  Three copies of every input
rotate across steps (3 x 134 MB of hidden states > the 256 MB Infinity Cache),
so each step reads its hidden states from HBM.  The value is whole-job
throughput: context tokens per second over the timed steps' wall clock.  Inside
the timed region only the dominant kernel is bracketed by HIP events (recorded on
its launch stream), which give its live duration for the roofline; the
per-kernel breakdown comes from an untimed pass with an event between every two
launches (each event adds a little to the step, so that pass is not `value`).

Also measured in the same run (not part of `value`): the attention with the
pruning-ratio temperature (the deep dive's operative rule, section 3.2 Eq. 7/8)
on the same inputs; the operative scoring path on the same workload (section 2
Eq. 1 and sections 3.1-3.2 Eqs. 3-8: the scorer on the raw residual with the
RMSNorm in front, the sequence RMS normalisation, selection, compaction, the
softmax-over-S gate and the attention with the per-head gain and the
temperature); the training-path attention (forward + backward at batch 4,
2048 kept tokens) with and without that temperature, and the CPU oracle on
the same workload, timed on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # MI355X HBM3E, bytes/s
PEAK_BF16 = 2.5e15         # MI355X dense bf16 matrix FLOP/s
NCOPY = 3


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def algorithmic_work(w, M):
    """Algorithmic FLOPs and bytes per launch of each kernel (what the method must compute / move)."""
    B, N, d, dff, Hq, Hkv, D = w.B, w.N, w.d, w.d_ff, w.Hq, w.Hkv, w.D
    esz = 2
    return {
        "gate_pack_w1": dict(flops=0.0, bytes=2.0 * dff * d * esz),
        "gate_score": dict(flops=2.0 * B * N * d * dff + 2.0 * B * N * dff,
                           bytes=B * N * d * esz + dff * d * esz + dff * esz + B * N * (1 + 4 + 4)),
        "select_topk": dict(flops=0.0, bytes=B * N * (4 + 1) + B * M * 4),
        "compact": dict(flops=0.0, bytes=2.0 * B * M * d * esz + B * M * (4 + 4 + 4 + 4 + 4)),
        "attn_fwd": dict(flops=4.0 * B * Hq * D * M * (M + 1) / 2,
                         bytes=B * M * (2 * Hq + 2 * Hkv) * D * esz + B * M * (4 + 4) + B * Hq * M * 4),
    }


def run_gpu(args):
    import torch

    import learned_token_pruning_gatescore_amd as tg
    from learned_token_pruning_gatescore_amd import workloads as wl

    dev = torch.device("cuda:0")
    tg.load()
    w = wl.WORKLOADS["qwen3_32k"]
    K = w.Ks[0]
    M = w.M(K)
    log(f"workload {w.name}: B={w.B} N={w.N} n_forced={w.n_forced} K={K} M={M}")
    gi = wl.gate_inputs(w)
    sel = wl.clustered_scores(w)
    at = wl.attn_inputs(w, M)
    T = lambda x: wl.to_torch(x, w.dtype, dev)
    w1, w2 = T(gi["w1"]), T(gi["w2"])
    forced = torch.from_numpy(gi["forced"]).to(dev)
    sel_t = torch.from_numpy(sel).to(dev)
    gamma = torch.from_numpy(at["gamma"]).to(dev)
    h0, q0, k0, v0 = T(gi["hidden"]), T(at["q"]), T(at["k"]), T(at["v"])
    copies = [(h0, q0, k0, v0)] + [(h0.clone(), q0.clone(), k0.clone(), v0.clone()) for _ in range(NCOPY - 1)]
    stream = torch.cuda.current_stream()

    bufs = {}
    scores = torch.empty((w.B, w.N), device=dev)
    gates = torch.empty((w.B, w.N), device=dev)
    kept = torch.empty((w.B, M), dtype=torch.int32, device=dev)
    hk = torch.empty((w.B, M, w.d), dtype=h0.dtype, device=dev)
    pk = torch.empty((w.B, M), dtype=torch.int32, device=dev)
    gk = torch.empty((w.B, M), device=dev)
    o = torch.empty_like(q0)
    lse = torch.empty((w.B, w.Hq, M), device=dev)
    ws = tg.attn_workspace(w.B, M, w.Hq, w.Hkv, w.D, False, dev)
    gws = tg.gate_workspace(w.d, w.d_ff, h0.dtype, dev)
    sws = tg.select_workspace(w.B, w.N, dev)
    # tg_gate_score = tg_gate_pack_w1 + tg_gate_score_packed; the two halves are
    # called (and timed) separately here, the work is the same
    names = ["gate_pack_w1", "gate_score", "select_topk", "compact", "attn_fwd"]
    NEV = len(names) + 1

    launches = [
        ("gate_pack_w1", lambda h, q, k, v: tg.tg_gate_pack_w1(w1, gws)),
        ("gate_score", lambda h, q, k, v: tg.tg_gate_score_packed(h, gws, w.d_ff, w2, forced, scores, gates)),
        ("select_topk", lambda h, q, k, v: tg.tg_select_topk(sel_t, forced, K, w.n_forced, kept, ws=sws)),
        ("compact", lambda h, q, k, v: tg.tg_compact(h, None, gates, kept, hk, pk, gk)),
        ("attn_fwd", lambda h, q, k, v: tg.tg_gated_attn_fwd(q, k, v, gk, gamma, pk, wl.ROPE_THETA, w.tau, o, lse,
                                                               ws)),
    ]
    assert [n for n, _ in launches] == names

    def step(i, marks=None):
        """One pass of the path; marks[j] (if given) is recorded before launch j, marks[len] after the last."""
        h, q, k, v = copies[i % NCOPY]
        for j, (_, f) in enumerate(launches):
            if marks is not None and marks[j] is not None:
                marks[j].record(stream)
            f(h, q, k, v)
        if marks is not None and marks[-1] is not None:
            marks[-1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # per-kernel breakdown: an untimed pass with an event between every two launches
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(NEV)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    per = {n: [] for n in names}
    for e in evs:
        for j, n in enumerate(names):
            per[n].append(e[j].elapsed_time(e[j + 1]) * 1e-3)
    step_dev = [e[0].elapsed_time(e[NEV - 1]) * 1e-3 for e in evs]
    log(f"instrumented pass: device path mean {np.mean(step_dev) * 1e6:.1f} us")
    dom = max(names, key=lambda n: np.mean(per[n]))
    jd = names.index(dom)

    # timed region: only the dominant kernel is bracketed by events (two per step, on its launch stream)
    dev_ev = []
    for i in range(args.steps):
        m = [None] * NEV
        m[jd], m[jd + 1] = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        dev_ev.append(m)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i, dev_ev[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    dom_live = [m[jd].elapsed_time(m[jd + 1]) * 1e-3 for m in dev_ev]
    log(f"timed {args.steps} steps: wall {wall * 1e3:.3f} ms ({wall / args.steps * 1e6:.1f} us/step), "
        f"{dom} {np.mean(dom_live) * 1e6:.1f} us")

    # the operative rule (per-row, per-head temperature) on the same inputs
    sigma = torch.from_numpy(at["sigma"]).to(dev)

    def attn_temp(i):
        h, q, k, v = copies[i % NCOPY]
        tg.tg_gated_attn_fwd(q, k, v, gk, gamma, pk, wl.ROPE_THETA, w.tau, o, lse, ws, sigma=sigma)

    temp_us = time_loop(attn_temp, args.steps, stream) * 1e6
    operative = run_operative(args, tg, wl, w, dev, stream, gi, sel, at, K, M)
    operative["per_head"] = run_operative_heads(args, tg, wl, w, dev, stream, gi, at, K, M)
    operative["clone_scorer"] = run_clone(args, tg, wl, w, dev, gi)

    work = algorithmic_work(w, M)
    kern = {}
    for n in names:
        t = float(np.mean(per[n]))
        wk = work[n]
        ent = dict(us=t * 1e6, us_min=float(np.min(per[n])) * 1e6, alg_bytes=wk["bytes"], alg_flops=wk["flops"],
                   hbm_GBps=wk["bytes"] / t / 1e9, hbm_frac=wk["bytes"] / t / PEAK_HBM)
        if wk["flops"]:
            ent.update(mfma_TFLOPs=wk["flops"] / t / 1e12, mfma_frac=wk["flops"] / t / PEAK_BF16)
        kern[n] = ent
    gate_stage = sum(kern[n]["us"] for n in names[:4]) * 1e-6
    gate_bytes = sum(work[n]["bytes"] for n in names[:4])
    summary = dict(
        gate_stage_us=gate_stage * 1e6, gate_stage_hbm_frac=gate_bytes / gate_stage / PEAK_HBM,
        gate_stage_bound_frac=(max(work["gate_score"]["flops"] / PEAK_BF16, work["gate_score"]["bytes"] / PEAK_HBM)
                               + (work["gate_pack_w1"]["bytes"] + work["select_topk"]["bytes"]
                                  + work["compact"]["bytes"]) / PEAK_HBM) / gate_stage,
        attn_fwd_mfma_frac=kern["attn_fwd"]["mfma_frac"],
        attn_fwd_temperature_us=temp_us,
        attn_fwd_temperature_mfma_frac=work["attn_fwd"]["flops"] / (temp_us * 1e-6) / PEAK_BF16)
    # roofline of the dominant kernel, from its durations inside the timed region
    t_dom = float(np.mean(dom_live))
    if work[dom]["flops"]:
        achieved = work[dom]["flops"] / t_dom
        roof = dict(kernel=dom, bound="mfma", achieved=achieved / 1e12, peak=PEAK_BF16 / 1e12, unit="TFLOP/s",
                    frac=achieved / PEAK_BF16, traffic=None, us=t_dom * 1e6)
    else:
        achieved = work[dom]["bytes"] / t_dom
        roof = dict(kernel=dom, bound="hbm", achieved=achieved / 1e9, peak=PEAK_HBM / 1e9, unit="GB/s",
                    frac=achieved / PEAK_HBM, traffic=None, us=t_dom * 1e6)
    traffic = load_traffic(dom)
    if traffic is not None:
        roof["traffic"] = traffic

    elapsed = wall
    res = dict(elapsed=elapsed, step_dev=float(np.mean(step_dev)), kernels=kern, summary=summary, roofline=roof,
               workload=w, K=K, M=M, operative=operative)
    if args.copy_calib_mb:
        nb = args.copy_calib_mb << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {nb} bytes read + {nb} bytes written")
    if args.train_steps:
        res["training_path"] = run_train(args, tg, wl, dev)
    res["plain_attention_reference"] = run_plain_reference(
        dev, M, kern["attn_fwd"]["us"], res["training_path"]["fwd_us"] if "training_path" in res else None)
    # gpu-side data needed by the CPU baseline (the same inputs)
    res["host_inputs"] = dict(gi=gi, sel=sel, at=at)
    return res


def time_loop(fn, n, stream):
    """Mean device time of fn(i) over n calls, from HIP events on `stream` (after 3 warm-up calls)."""
    import torch

    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        fn(i)
        b.record(stream)
    torch.cuda.synchronize()
    return float(np.mean([a.elapsed_time(b) for a, b in evs])) * 1e-3


def run_operative(args, tg, wl, w, dev, stream, gi, sel, at, K, M):
    """The operative scoring path on the long-context workload, one HIP stream, per-stage events.

    Raw residual rows (three rotating copies, as in the main loop) -> tg_gate_score_ln (RMSNorm
    weight folded into W1 by its pack pass, then the scorer) -> tg_score_normalize -> tg_select_topk
    -> tg_compact (of the normalised scores) -> tg_gate_softmax -> tg_gated_attn_fwd with the
    per-head gain and the Eq. 7/8 temperature.  Selection ranks the drawn clustered score vector
    after the same normalisation (as the main path ranks the drawn vector).
    """
    import torch

    ri = wl.residual_inputs(w)
    T = lambda x: wl.to_torch(x, w.dtype, dev)
    hs = [T(ri["hidden"])]
    hs += [hs[0].clone() for _ in range(NCOPY - 1)]
    lw, w1, w2 = T(ri["ln_w"]), T(gi["w1"]), T(gi["w2"])
    forced = torch.from_numpy(gi["forced"]).to(dev)
    sel_t = torch.from_numpy(sel).to(dev)
    q, k, v = T(at["q"]), T(at["k"]), T(at["v"])
    gain = torch.from_numpy(np.log1p(np.exp(at["gamma"])).astype(np.float32)).to(dev)
    sigma = torch.from_numpy(at["sigma"]).to(dev)
    raw = torch.empty((w.B, w.N), device=dev)
    bsel = torch.empty((w.B, w.N), device=dev)
    kept = torch.empty((w.B, M), dtype=torch.int32, device=dev)
    hk = torch.empty((w.B, M, w.d), dtype=hs[0].dtype, device=dev)
    pk = torch.empty((w.B, M), dtype=torch.int32, device=dev)
    bk = torch.empty((w.B, M), device=dev)
    g = torch.empty((w.B, M), device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, M), device=dev)
    ws = tg.attn_workspace(w.B, M, w.Hq, w.Hkv, w.D, False, dev)
    gws = tg.gate_workspace(w.d, w.d_ff, hs[0].dtype, dev)
    sws = tg.select_workspace(w.B, w.N, dev)
    names = ["gate_score_ln", "score_normalize", "select_topk", "compact", "gate_softmax", "attn_fwd_temperature"]

    def step(i, ev=None):
        rec = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        rec(0)
        tg.tg_gate_score_ln(hs[i % NCOPY], lw, 1e-6, w1, w2, forced, raw, None, gws)
        rec(1)
        tg.tg_score_normalize(sel_t, forced, 1e-6, bsel)
        rec(2)
        tg.tg_select_topk(bsel, forced, K, w.n_forced, kept, ws=sws)
        rec(3)
        tg.tg_compact(hs[i % NCOPY], None, bsel, kept, hk, pk, bk)
        rec(4)
        tg.tg_gate_softmax(bk, kept, g)
        rec(5)
        tg.tg_gated_attn_fwd(q, k, v, g, gain, pk, wl.ROPE_THETA, w.tau, o, lse, ws, sigma=sigma)
        rec(6)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i, e in enumerate(evs):
        step(i, e)
    torch.cuda.synchronize()
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3 for j, n in enumerate(names)}
    tot = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs])) * 1e-3
    return dict(stages_us=per, device_path_us=tot * 1e6, tokens_per_s=w.B * w.N / tot,
                note="gate_score_ln includes its W1 pack pass (RMSNorm weight folded in)")


def run_operative_heads(args, tg, wl, w, dev, stream, gi, at, K, M):
    """The per-head variant (DeepDive section 3.4): the scorer with one output per query head (RMSNorm in
    front), per-head normalisation, uniform head aggregation, selection on the aggregate, compaction,
    per-head gather and softmax gate, attention with per-head gates, gain and temperature."""
    import torch

    H = w.Hq
    ri = wl.residual_inputs(w)
    T = lambda x: wl.to_torch(x, w.dtype, dev)
    hs = [T(ri["hidden"])]
    hs += [hs[0].clone() for _ in range(NCOPY - 1)]
    lw, w1 = T(ri["ln_w"]), T(gi["w1"])
    rs = np.random.default_rng(w.seed + 4000)
    w2h = T(wl.bf16_bits((rs.standard_normal((H, w.d_ff)) / np.sqrt(w.d_ff)).astype(np.float32)))
    forced = torch.from_numpy(gi["forced"]).to(dev)
    q, k, v = T(at["q"]), T(at["k"]), T(at["v"])
    gain = torch.from_numpy(np.log1p(np.exp(at["gamma"])).astype(np.float32)).to(dev)
    sigma = torch.from_numpy(at["sigma"]).to(dev)
    raw = torch.empty((w.B, H, w.N), device=dev)
    b = torch.empty((w.B, H, w.N), device=dev)
    agg = torch.empty((w.B, w.N), device=dev)
    kept = torch.empty((w.B, M), dtype=torch.int32, device=dev)
    hk = torch.empty((w.B, M, w.d), dtype=hs[0].dtype, device=dev)
    pk = torch.empty((w.B, M), dtype=torch.int32, device=dev)
    bk = torch.empty((w.B, H, M), device=dev)
    g = torch.empty((w.B, H, M), device=dev)
    o = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, M), device=dev)
    ws = tg.attn_workspace(w.B, M, w.Hq, w.Hkv, w.D, False, dev)
    gws = tg.gate_workspace(w.d, w.d_ff, hs[0].dtype, dev)
    sws = tg.select_workspace(w.B, w.N, dev)
    names = ["gate_score_heads", "score_normalize_heads", "aggregate_heads", "select_topk", "compact",
             "gather_heads", "gate_softmax_heads", "attn_fwd_headgates"]

    def step(i, ev=None):
        rec = (lambda j: ev[j].record(stream)) if ev is not None else (lambda j: None)
        rec(0)
        tg.tg_gate_score_heads(hs[i % NCOPY], w1, w2h, raw, gws, ln_w=lw, ln_eps=1e-6)
        rec(1)
        tg.tg_score_normalize_heads(raw, forced, 1e-6, b)
        rec(2)
        tg.tg_aggregate_heads(b, agg)
        rec(3)
        tg.tg_select_topk(agg, forced, K, w.n_forced, kept, ws=sws)
        rec(4)
        tg.tg_compact(hs[i % NCOPY], None, None, kept, hk, pk, None)
        rec(5)
        tg.tg_gather_heads(b, kept, bk)
        rec(6)
        tg.tg_gate_softmax_heads(bk, kept, g)
        rec(7)
        tg.tg_gated_attn_fwd_headgates(q, k, v, g, gain, pk, wl.ROPE_THETA, w.tau, o, lse, ws, sigma=sigma)
        rec(8)

    for i in range(3):
        step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(names) + 1)] for _ in range(args.steps)]
    for i, e in enumerate(evs):
        step(i, e)
    torch.cuda.synchronize()
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3 for j, n in enumerate(names)}
    tot = float(np.mean([e[0].elapsed_time(e[-1]) for e in evs])) * 1e-3
    return dict(heads=H, stages_us=per, device_path_us=tot * 1e6, tokens_per_s=w.B * w.N / tot,
                note="gate_score_heads includes its W1 pack pass (RMSNorm weight folded in)")


def run_clone(args, tg, wl, w, dev, gi):
    """The scorer cloned from the gate layer's MLP (SwiGLU at the Qwen3-1.7B width + a 16-row head
    projection) over the same hidden states: time per call, including its weight packing and the
    down/head fold (not part of `value`)."""
    import torch

    d_i, H = wl.QWEN3_1P7B_MLP, 16
    ci = wl.clone_inputs(w, d_i, H)
    T = lambda x: wl.to_torch(x, w.dtype, dev)
    h = T(gi["hidden"])
    wg, wu, wd, wh = (T(ci[k]) for k in ("w_gate", "w_up", "w_down", "w_head"))
    scores = torch.empty((w.B, H, w.N), device=dev)
    ws = torch.empty(tg.tg_gate_score_clone_workspace_size(w.d, d_i, H), dtype=torch.uint8, device=dev)
    call = lambda: tg.tg_gate_score_clone(h, wg, wu, wd, wh, scores, ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    n = max(3, min(args.steps, 10))
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    ev[0].record()
    for i in range(n):
        call()
        ev[i + 1].record()
    torch.cuda.synchronize()
    t = float(np.mean([ev[i].elapsed_time(ev[i + 1]) for i in range(n)])) * 1e-3
    tok = w.B * w.N
    flops = 2.0 * tok * w.d * 2 * d_i + 2.0 * tok * d_i * H
    return dict(d_i=d_i, heads=H, us=t * 1e6, alg_flops=flops, mfma_TFLOPs=flops / t / 1e12,
                mfma_frac=flops / t / PEAK_BF16, tokens_per_s=tok / t,
                note="one tg_gate_score_clone call: gate/up packing, the down x head fold, the gated "
                     "products and the head sums")


def run_train(args, tg, wl, dev):
    """Training-path attention: forward + backward at batch 4, 2048 kept tokens (not part of `value`)."""
    import torch

    w = wl.WORKLOADS["train_b4"]
    M = w.M_fixed
    a = wl.attn_inputs(w, M, with_grad=True)
    T = lambda x: wl.to_torch(x, w.dtype, dev)
    q, k, v, dout = T(a["q"]), T(a["k"]), T(a["v"]), T(a["dout"])
    g = torch.from_numpy(a["g"]).to(dev)
    gamma = torch.from_numpy(a["gamma"]).to(dev)
    pos = torch.from_numpy(a["pos"]).to(dev)
    o = torch.empty_like(q)
    o_lo = torch.empty_like(q)
    lse = torch.empty((w.B, w.Hq, M), device=dev)
    dq = torch.empty(q.shape, device=dev)
    dk = torch.empty(k.shape, device=dev)
    dv = torch.empty(v.shape, device=dev)
    dg = torch.empty(g.shape, device=dev)
    dgam = torch.empty(gamma.shape, device=dev)
    sigma = torch.from_numpy(a["sigma"]).to(dev)
    dsig = torch.empty(gamma.shape, device=dev)
    ws = tg.attn_workspace(w.B, M, w.Hq, w.Hkv, w.D, True, dev)
    stream = torch.cuda.current_stream()

    def step(ev=None, temp=False, use_o=False):
        sg = dict(sigma=sigma) if temp else {}
        if ev:
            ev[0].record(stream)
        tg.tg_gated_attn_fwd(q, k, v, g, gamma, pos, wl.ROPE_THETA, w.tau, o, lse, ws, o_lo=o_lo if use_o else None,
                             **sg)
        if ev:
            ev[1].record(stream)
        if temp:
            sg["dsigma"] = dsig
        if use_o:
            sg.update(o=o, o_lo=o_lo)
        tg.tg_gated_attn_bwd(q, k, v, g, gamma, pos, wl.ROPE_THETA, w.tau, lse, dout, dq, dk, dv, dg, dgam, ws, **sg)
        if ev:
            ev[2].record(stream)

    ff = 4.0 * w.B * w.Hq * w.D * M * (M + 1) / 2
    out = dict(workload=w.name, B=w.B, M=M)
    out["two_budgets_packed"] = run_train_varlen(args, tg, wl, dev, w, False)
    out["two_budgets_packed_d_from_o"] = run_train_varlen(args, tg, wl, dev, w, True)
    out["per_sample_budgets_packed"] = run_train_varlen(args, tg, wl, dev, w, False, per_sample=True)
    # without o: the backward forms D_i by its own pass over the keys; with o: the forward also
    # writes o_lo and the backward takes D_i = dO . (o + o_lo)
    for use_o in (False, True):
        for temp in (False, True):
            for _ in range(3):
                step(temp=temp, use_o=use_o)
            torch.cuda.synchronize()
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.train_steps)]
            for e in evs:
                step(e, temp=temp, use_o=use_o)
            torch.cuda.synchronize()
            fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
            bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
            r = dict(fwd_us=fwd * 1e6, bwd_us=bwd * 1e6, fwd_mfma_frac=ff / fwd / PEAK_BF16,
                     bwd_mfma_frac=2.5 * ff / bwd / PEAK_BF16, tokens_per_s=w.B * M / (fwd + bwd))
            key = ("d_from_o" if use_o else "") + ("_temperature" if use_o and temp else "temperature" if temp else "")
            if key:
                out[key] = r
            else:
                out.update(r)
    return out


def run_train_varlen(args, tg, wl, dev, w, use_o, per_sample=False):
    """Both training budgets in one packed call (DeepDive section 3.3): each of the B rows at its
    full budget (M = 2048 kept) and at half of it (1024), packed by budget, forward + backward with
    the Eq. 7/8 temperature (not part of `value`); use_o: the backward's row terms from o + o_lo.
    per_sample: the budget drawn per sample, as the pages train (log-uniform): 2B rows, each row's
    kept count drawn log-uniform in [512, 2048] and the same row again at half of it, so every
    sequence of the packing has its own length."""
    import torch

    lens = [w.M_fixed] * w.B + [w.M_fixed // 2] * w.B
    if per_sample:
        kr = np.exp(np.random.default_rng(w.seed + 3100).uniform(np.log(512), np.log(2048), 2 * w.B))
        full = [int(x) for x in np.round(kr)]
        lens = full + [m // 2 for m in full]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T_ = int(cu[-1])
    rs = np.random.default_rng(w.seed + 3000)
    T = lambda x: wl.to_torch(x, w.dtype, dev)
    q = T(wl.bf16_bits(rs.standard_normal((T_, w.Hq, w.D), dtype=np.float32)))
    k = T(wl.bf16_bits(rs.standard_normal((T_, w.Hkv, w.D), dtype=np.float32)))
    v = T(wl.bf16_bits(rs.standard_normal((T_, w.Hkv, w.D), dtype=np.float32)))
    dout = T(wl.bf16_bits(rs.standard_normal((T_, w.Hq, w.D), dtype=np.float32)))
    g = torch.from_numpy((1.0 / (1.0 + np.exp(-rs.standard_normal(T_)))).astype(np.float32)).to(dev)
    gamma = torch.from_numpy(rs.uniform(0.5, 1.5, w.Hq).astype(np.float32)).to(dev)
    pos = torch.from_numpy(np.concatenate([np.sort(rs.choice(w.N, n, replace=False)) for n in lens])
                           .astype(np.int32)).to(dev)
    sigma = torch.from_numpy((0.54 + 0.5 * rs.standard_normal(w.Hq)).astype(np.float32)).to(dev)
    o = torch.empty_like(q)
    o_lo = torch.empty_like(q) if use_o else None
    lse = torch.empty(w.Hq * T_, device=dev)
    dq, dk, dv = (torch.empty(x.shape, device=dev) for x in (q, k, v))
    dg = torch.empty(T_, device=dev)
    dgam, dsig = torch.empty(w.Hq, device=dev), torch.empty(w.Hq, device=dev)
    ws = tg.attn_varlen_workspace(cu, w.Hq, w.Hkv, w.D, True, dev)
    stream = torch.cuda.current_stream()

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        tg.tg_gated_attn_fwd_varlen(q, k, v, g, gamma, pos, wl.ROPE_THETA, w.tau, cu, o, lse, ws, sigma=sigma,
                                    o_lo=o_lo)
        if ev:
            ev[1].record(stream)
        tg.tg_gated_attn_bwd_varlen(q, k, v, g, gamma, pos, wl.ROPE_THETA, w.tau, lse, dout, cu, dq, dk, dv, dg, dgam,
                                    ws, sigma=sigma, dsigma=dsig, o=o if use_o else None, o_lo=o_lo)
        if ev:
            ev[2].record(stream)

    for _ in range(3):
        step()
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.train_steps)]
    for e in evs:
        step(e)
    torch.cuda.synchronize()
    fwd = float(np.mean([e[0].elapsed_time(e[1]) for e in evs])) * 1e-3
    bwd = float(np.mean([e[1].elapsed_time(e[2]) for e in evs])) * 1e-3
    ff = sum(4.0 * w.Hq * w.D * n * (n + 1) / 2 for n in lens)
    return dict(lens=(f"{len(lens)} lengths (2 x {2 * w.B} rows, budgets drawn log-uniform per row)" if per_sample
                      else f"{w.B} x {w.M_fixed} + {w.B} x {w.M_fixed // 2}"), tokens=T_, fwd_us=fwd * 1e6,
                bwd_us=bwd * 1e6, fwd_mfma_frac=ff / fwd / PEAK_BF16, bwd_mfma_frac=2.5 * ff / bwd / PEAK_BF16,
                tokens_per_s=T_ / (fwd + bwd))


def run_plain_reference(dev, M, gated_c3_us, gated_train_us):
    """Context for DeepDive section 3.2's statement that the gate-biased attention call costs about what a
    plain fused call costs: PyTorch's fused attention (flash backend only, so no fallback path runs) doing
    plain causal softmax attention -- no gate bias, no RoPE, no temperature, K and V repeated to all 16
    query heads -- at the 32K-context shape (B=1, M kept rows) and at the training shape (B=4, M=2048),
    next to tg_gated_attn_fwd's per-call time (prep + forward) at the same shapes. Not part of `value`."""
    import torch
    from torch.nn.attention import SDPBackend, sdpa_kernel

    out = dict(impl="torch.nn.functional.scaled_dot_product_attention, flash backend only (plain causal: "
                    "no gate bias, no RoPE, no temperature; K/V repeated to the 16 query heads), bf16")
    for name, B, Mx, ours in (("long_context", 1, M, gated_c3_us), ("training", 4, 2048, gated_train_us)):
        try:
            q = torch.randn(B, 16, Mx, 128, device=dev, dtype=torch.bfloat16)
            k = torch.randn(B, 8, Mx, 128, device=dev, dtype=torch.bfloat16).repeat_interleave(2, dim=1).contiguous()
            v = torch.randn(B, 8, Mx, 128, device=dev, dtype=torch.bfloat16).repeat_interleave(2, dim=1).contiguous()
            with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
                f = lambda: torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
                for _ in range(5):
                    f()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                n = 30
                e0.record()
                for _ in range(n):
                    f()
                e1.record()
                torch.cuda.synchronize()
            plain = e0.elapsed_time(e1) / n * 1e3
            out[name] = dict(B=B, M=Mx, plain_us=plain, gated_us=ours,
                             gated_over_plain=None if ours is None else ours / plain)
        except Exception as e:  # backend not available in this PyTorch: report, do not fall back
            out[name] = dict(B=B, M=Mx, error=repr(e)[:200])
    return out


def load_traffic(kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter summary
    (profiles/traffic.json), or None when there is none or the kernel's source has
    changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        ent = json.load(open(path)).get(kernel)
        if ent is None:
            return None
        src = os.path.join(ROOT, "learned_token_pruning_gatescore_amd", "csrc", ent["source"])
        if hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != ent["source_sha256"]:
            return None
        return ent["hbm_bytes_per_launch"]
    except (ValueError, OSError, KeyError):
        return None


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), with the logical CPUs this process may use."""
    name = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    name = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{name} ({len(os.sched_getaffinity(0))} logical CPUs available)"


def run_cpu_baseline(host, w, K, M):
    """The oracle as it stands, on this host's cores, over the same workload (all tokens, all rows)."""
    import oracle
    from learned_token_pruning_gatescore_amd import workloads as wl

    oracle.build(force=False)
    gi, sel, at = host["gi"], host["sel"], host["at"]
    t = {}
    t0 = time.perf_counter()
    hf = wl.as_float(gi["hidden"], w.dtype).reshape(w.B * w.N, w.d)
    s, g = oracle.gate_score(hf, wl.as_float(gi["w1"], w.dtype), wl.as_float(gi["w2"], w.dtype),
                             gi["forced"].reshape(-1))
    t["gate_score"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    kept, _ = oracle.select_topk(sel, gi["forced"], K)
    t["select_topk"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    hk, pk, gk = oracle.compact(gi["hidden"], None, g.astype(np.float32).reshape(w.B, w.N), kept)
    t["compact"] = time.perf_counter() - t0
    t0 = time.perf_counter()
    f = lambda x: wl.as_float(x, w.dtype)
    oracle.attn_fwd(f(at["q"]), f(at["k"]), f(at["v"]), gk, at["gamma"], pos=pk, theta=wl.ROPE_THETA, tau=w.tau,
                    round_bf16=True)
    t["attn_fwd"] = time.perf_counter() - t0
    total = sum(t.values())
    return dict(value=w.B * w.N / total, unit="tokens/s", cores=oracle.num_threads(), cpu=cpu_model(), kind="oracle",
                sample=f"full workload once: {w.B * w.N} tokens scored, selected and compacted, attention over all "
                       f"{M} kept rows x {w.Hq} heads; fp64 plain loops",
                seconds=t, total_s=total)


def run_sweep(args):
    """The same path (pack, score, select, compact, attention forward) at the other workload sizes:
    8K context (K = 1024) and 128K context (K = 256, 1024, 4096, 16384); one JSON line each (not `value`)."""
    import torch

    import learned_token_pruning_gatescore_amd as tg
    from learned_token_pruning_gatescore_amd import workloads as wl

    dev = torch.device("cuda:0")
    tg.load()
    for name in ("qwen3_8k", "sweep_128k"):
        w = wl.WORKLOADS[name]
        gi = wl.gate_inputs(w)
        sel = torch.from_numpy(wl.clustered_scores(w)).to(dev)
        T = lambda x: wl.to_torch(x, w.dtype, dev)
        h, w1, w2 = T(gi["hidden"]), T(gi["w1"]), T(gi["w2"])
        forced = torch.from_numpy(gi["forced"]).to(dev)
        scores = torch.empty((w.B, w.N), device=dev)
        gates = torch.empty_like(scores)
        gws = tg.gate_workspace(w.d, w.d_ff, h.dtype, dev)
        sws = tg.select_workspace(w.B, w.N, dev)
        for K in w.Ks:
            M = w.M(K)
            at = wl.attn_inputs(w, M)
            q, k, v = T(at["q"]), T(at["k"]), T(at["v"])
            gamma = torch.from_numpy(at["gamma"]).to(dev)
            kept = torch.empty((w.B, M), dtype=torch.int32, device=dev)
            hk = torch.empty((w.B, M, w.d), dtype=h.dtype, device=dev)
            pk = torch.empty((w.B, M), dtype=torch.int32, device=dev)
            gk = torch.empty((w.B, M), device=dev)
            o = torch.empty_like(q)
            lse = torch.empty((w.B, w.Hq, M), device=dev)
            ws = tg.attn_workspace(w.B, M, w.Hq, w.Hkv, w.D, False, dev)
            launches = [("gate_pack_w1", lambda: tg.tg_gate_pack_w1(w1, gws)),
                        ("gate_score", lambda: tg.tg_gate_score_packed(h, gws, w.d_ff, w2, forced, scores, gates)),
                        ("select_topk", lambda: tg.tg_select_topk(sel, forced, K, w.n_forced, kept, ws=sws)),
                        ("compact", lambda: tg.tg_compact(h, None, gates, kept, hk, pk, gk)),
                        ("attn_fwd", lambda: tg.tg_gated_attn_fwd(q, k, v, gk, gamma, pk, wl.ROPE_THETA, w.tau, o,
                                                                  lse, ws))]
            step = lambda: [f() for _, f in launches]
            for _ in range(args.warmup):
                step()
            n = max(args.steps // 5, 4)
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(launches) + 1)] for _ in range(n)]
            for e in evs:
                for j, (_, f) in enumerate(launches):
                    e[j].record()
                    f()
                e[-1].record()
            torch.cuda.synchronize()
            per = {nm: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs])) * 1e3
                   for j, (nm, _) in enumerate(launches)}
            # step: back-to-back passes between two events on the launch stream (a wall clock over a
            # few passes from a synchronised start also counts the first enqueue and the final sync)
            nw = max(args.steps, 10)
            t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            t0.record()
            for _ in range(nw):
                step()
            t1.record()
            torch.cuda.synchronize()
            wall = t0.elapsed_time(t1) * 1e-3 / nw
            attn_flops = 4.0 * w.B * w.Hq * w.D * M * (M + 1) / 2
            print(json.dumps(dict(sweep=name, N=w.N, K=K, M=M, step_us=wall * 1e6, tokens_per_s=w.B * w.N / wall,
                                  kernels_us_with_events=per,
                                  gate_score_TFLOPs=2.0 * w.B * w.N * w.d * w.d_ff / (per["gate_score"] * 1e-6) / 1e12,
                                  attn_fwd_TFLOPs=attn_flops / (per["attn_fwd"] * 1e-6) / 1e12)), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--train-steps", type=int, default=10, help="training-path fwd+bwd steps (0 = skip)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sweep", action="store_true",
                    help="instead: the same path at 8K and 128K context, one JSON line per (workload, K)")
    ap.add_argument("--copy-calib-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (--gpus {args.gpus} requested): the library has no multi-GPU path "
              f"(it would shard batch rows, or one row's tokens for scoring and its kv heads for attention, "
              f"one process per GPU).", file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") not in ("", "1"):
        print("bench.py is single-process, single-GPU", file=sys.stderr)
        sys.exit(2)

    if args.sweep:
        run_sweep(args)
        return
    res = run_gpu(args)
    w, K, M = res["workload"], res["K"], res["M"]
    ms = res["elapsed"] / args.steps * 1e3
    value = w.B * w.N * args.steps / res["elapsed"]
    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on the same workload ...")
        cpu = run_cpu_baseline(res["host_inputs"], w, K, M)
        log(f"oracle: {cpu['total_s']:.2f} s on {cpu['cores']} threads")
    roof = dict(res["roofline"])
    line = {
        "metric": "gate-layer prefill tokens/s (N=32K->K=2K, bf16); % of HBM and MFMA peak",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; Qwen3-1.7B-shaped gate layer; drawn clustered selection scores)",
        "config": {"workload": "long-context gate layer: B=1, N=32768 (128 scaffold), K=2048 -> M=2176, "
                               "d=2048, scorer 2048->512->1, 16/8 heads, D=128, RoPE theta 1e6, tau=1",
                   "global_batch": w.B, "seq_len": w.N, "kept": M, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": None if cpu is None else {k: cpu[k] for k in ("value", "unit", "cores", "cpu", "kind",
                                                                       "sample")},
        "device_path_us_instrumented": res["step_dev"] * 1e6,
        "kernels": res["kernels"],
        "summary": res["summary"],
        "operative_path": res["operative"],
    }
    if "training_path" in res:
        line["training_path"] = res["training_path"]
    line["plain_attention_reference"] = res["plain_attention_reference"]
    if cpu is not None:
        line["cpu_baseline_stage_s"] = cpu["seconds"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
