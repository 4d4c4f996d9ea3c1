"""GPU parity of the per-head scoring path against the CPU oracle (DeepDive section 3.4:
per-head scores, uniform head aggregation for selection, per-head bias).

  * tg_gate_score_heads: within 1e-2 (bf16) / 1e-5 (fp32) of the oracle, relative to
    max(|ref|, rms(ref)) per head; with and without the RMSNorm in front.
  * tg_score_normalize_heads, tg_aggregate_heads, tg_gate_softmax_heads: within 1e-5 on the same
    inputs; tg_gather_heads bit-exact.
  * tg_gated_attn_fwd_headgates / _bwd_headgates: o, lse and every gradient within 2e-2 (bf16) /
    1e-4 (fp32).
  * the chain normalise -> aggregate -> select -> gather -> softmax per head, selection bit-exact
    on the aggregated vector.
"""
import numpy as np
import pytest

import oracle
from learned_token_pruning_gatescore_amd import workloads as wl
from tests._gpu import assert_maxabs, assert_scores_close, dev_tensor, device, say, to_np

pytestmark = pytest.mark.gpu


def _wl(B, N, d, d_ff, dtype="bf16", n_forced=5, seed=71):
    return wl.Workload("heads", seed, B=B, N=N, n_forced=min(n_forced, N), d=d, d_ff=d_ff, Ks=(1,), Hq=8, Hkv=4,
                       D=128, tau=1.0, dtype=dtype, rope=True)


def _w2_heads(w, H):
    rng = np.random.default_rng(w.seed + 500)
    x = (rng.standard_normal((H, w.d_ff)) / np.sqrt(w.d_ff)).astype(np.float32)
    return wl.bf16_bits(x) if w.dtype == "bf16" else x


def _heads_scores(w, H, ln, sample=None):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    gi = wl.gate_inputs(w)
    ri = wl.residual_inputs(w)
    src = ri if ln else gi
    h = dev_tensor(src["hidden"], w.dtype, dev)
    w1 = dev_tensor(gi["w1"], w.dtype, dev)
    w2n = _w2_heads(w, H)
    w2 = dev_tensor(w2n, w.dtype, dev)
    lw = dev_tensor(ri["ln_w"], w.dtype, dev) if ln else None
    B, n = w.B, w.N
    out = torch.full((B, H, n), float("nan"), device=dev)
    ws = tg.gate_workspace(w.d, w.d_ff, h.dtype, dev)
    say("gate_score_heads", w.dtype, B, n, w.d, w.d_ff, H, "ln" if ln else "")
    tg.tg_gate_score_heads(h, w1, w2, out, ws, ln_w=lw, ln_eps=1e-6 if ln else None)
    torch.cuda.synchronize()
    hf = wl.as_float(src["hidden"], w.dtype).reshape(B * n, w.d)
    idx = np.arange(B * n) if sample is None else sample
    x = hf[idx]
    if ln:
        x = oracle.rms_norm(x, wl.as_float(ri["ln_w"], w.dtype), 1e-6)
    ref = oracle.gate_score_heads(x, wl.as_float(gi["w1"], w.dtype), wl.as_float(w2n, w.dtype))  # [H, len(idx)]
    got = to_np(out).transpose(1, 0, 2).reshape(H, B * n)[:, idx]
    return got, ref


@pytest.mark.parametrize("B,N,d,d_ff,H,ln", [(2, 1000, 256, 96, 4, False), (2, 300, 128, 640, 16, True),
                                             (1, 513, 96, 100, 1, True), (1, 33001, 128, 200, 8, False),
                                             (1, 1, 32, 1, 3, True)])
def test_score_heads_bf16(B, N, d, d_ff, H, ln):
    got, ref = _heads_scores(_wl(B, N, d, d_ff), H, ln)
    for h in range(H):
        assert_scores_close(got[h], ref[h], 1e-2, f"scores head {h}")


def test_score_heads_f32():
    got, ref = _heads_scores(_wl(1, 200, 64, 48, dtype="f32"), 5, True)
    for h in range(5):
        assert_scores_close(got[h], ref[h], 1e-5, f"scores head {h}")


def test_score_heads_full_size_sampled():
    w = wl.WORKLOADS["qwen3_32k"]
    rng = np.random.default_rng(3)
    sample = np.unique(np.concatenate([[0, 127, 128, w.N - 1], rng.choice(w.N, 200, replace=False)]))
    got, ref = _heads_scores(w, 16, True, sample=sample)
    for h in range(16):
        assert_scores_close(got[h], ref[h], 1e-2, f"scores head {h}")


def test_normalize_aggregate_gather_softmax_heads():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    rng = np.random.default_rng(11)
    B, H, N, K = 2, 6, 3001, 400
    dev = device()
    s = rng.normal(0.2, 1.7, (B, H, N)).astype(np.float32)
    forced = np.zeros((B, N), np.uint8)
    forced[:, :9] = 1
    forced[1, :9] = 0
    forced[1, 1000:1009] = 1  # nine scaffold tokens in each row, at different places
    st = torch.from_numpy(s).to(dev)
    ft = torch.from_numpy(forced).to(dev)
    b = torch.full_like(st, float("nan"))
    say("normalize/aggregate/gather/softmax heads", B, H, N)
    tg.tg_score_normalize_heads(st, ft, 1e-6, b)
    agg = torch.full((B, N), float("nan"), device=dev)
    tg.tg_aggregate_heads(b, agg)
    torch.cuda.synchronize()
    b_np = to_np(b)
    for h in range(H):
        ref = oracle.score_normalize(s[:, h], forced, 1e-6)
        assert np.all(b_np[:, h][forced == 1] == 0.0)
        assert_scores_close(b_np[:, h].reshape(-1), ref.reshape(-1), 1e-5, f"b head {h}")
    assert_scores_close(to_np(agg).reshape(-1), oracle.aggregate_heads(b_np).reshape(-1), 1e-5, "aggregate")
    M = 9 + K
    kept = torch.full((B, M), -7, dtype=torch.int32, device=dev)
    tg.tg_select_topk(agg, ft, K, 9, kept)
    bk = torch.full((B, H, M), float("nan"), device=dev)
    tg.tg_gather_heads(b, kept, bk)
    g = torch.full((B, H, M), float("nan"), device=dev)
    tg.tg_gate_softmax_heads(bk, kept, g)
    torch.cuda.synchronize()
    kept_np = to_np(kept)
    kept_ref, _ = oracle.select_topk(to_np(agg), forced, K, M=M)
    assert np.array_equal(kept_np, kept_ref)
    bk_ref = np.where(kept_np[:, None, :] >= 0,
                      np.take_along_axis(b_np, np.maximum(kept_np, 0)[:, None, :].repeat(H, 1), axis=2), 0.0)
    assert np.array_equal(to_np(bk), bk_ref.astype(np.float32))
    g_np = to_np(g)
    for h in range(H):
        assert_scores_close(g_np[:, h].reshape(-1), oracle.gate_softmax(bk_ref[:, h], kept_np).reshape(-1), 1e-5,
                            f"g head {h}")


def _headgate_case(B, M, Hq, Hkv, D, dtype="bf16", rope=True, temp=False, seed=81, zero_heads=False, far=False,
                   use_o=False):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = wl.Workload("hg", seed, B=B, N=max(4 * M, 64), n_forced=0, d=0, d_ff=0, Ks=(M,), Hq=Hq, Hkv=Hkv, D=D,
                    tau=1.1, dtype=dtype, rope=True, M_fixed=M)
    a = wl.attn_inputs(w, M, with_grad=True)
    rng = np.random.default_rng(seed)
    gh = (1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.5, (B, Hq, M))))).astype(np.float32)
    if zero_heads:
        gh[0, 1, : M // 3] = 0.0  # one head sees no early keys
        gh[0, 0, 0] = 0.0
    if far:
        # gates in [0.5, 0.52] with a gain of 150: biases between -150 and -141.5 (log2 units), so
        # every live logit lies far below zero; head h has g = 0 on its first 32 (h % 3 + 1) keys, so
        # each head's first live key sits in a different tile
        gh = rng.uniform(0.5, 0.52, (B, Hq, M)).astype(np.float32)
        for h in range(Hq):
            gh[:, h, : 32 * (h % 3 + 1)] = 0.0
        a["gamma"] = np.full(Hq, 150.0, np.float32)
    dev = device()
    q, k, v, dout = (dev_tensor(a[n], dtype, dev) for n in ("q", "k", "v", "dout"))
    g = torch.from_numpy(gh).to(dev)
    gamma = torch.from_numpy(a["gamma"]).to(dev)
    pos = torch.from_numpy(a["pos"]).to(dev) if rope else None
    sigma = torch.from_numpy(a["sigma"]).to(dev) if temp else None
    o = torch.full_like(q, float("nan"))
    lse = torch.full((B, Hq, M), float("nan"), device=dev)
    ws = tg.attn_workspace(B, M, Hq, Hkv, D, True, dev)
    say("attn headgates", dtype, B, M, Hq, Hkv, D, "rope" if rope else "", "temp" if temp else "")
    o_lo = torch.full_like(q, float("nan")) if use_o else None
    tg.tg_gated_attn_fwd_headgates(q, k, v, g, gamma, pos, wl.ROPE_THETA, w.tau, o, lse, ws, sigma=sigma, o_lo=o_lo)
    dq, dk, dv = (torch.full(x.shape, float("nan"), device=dev) for x in (q, k, v))
    dg = torch.full(g.shape, float("nan"), device=dev)
    dgam = torch.full(gamma.shape, float("nan"), device=dev)
    dsig = torch.full(gamma.shape, float("nan"), device=dev) if temp else None
    tg.tg_gated_attn_bwd_headgates(q, k, v, g, gamma, pos, wl.ROPE_THETA, w.tau, lse, dout, dq, dk, dv, dg, dgam, ws,
                                   sigma=sigma, dsigma=dsig, o=o if use_o else None, o_lo=o_lo)
    torch.cuda.synchronize()
    f = lambda x: wl.as_float(x, dtype)
    kw = dict(pos=a["pos"] if rope else None, theta=wl.ROPE_THETA, tau=w.tau, round_bf16=(dtype == "bf16"),
              sigma=a["sigma"] if temp else None)
    o_ref, l_ref = oracle.attn_fwd(f(a["q"]), f(a["k"]), f(a["v"]), gh, a["gamma"], **kw)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert_maxabs(to_np(o), o_ref, tol, "o")
    assert_maxabs(to_np(lse), l_ref, tol, "lse")
    ref = oracle.attn_bwd(f(a["q"]), f(a["k"]), f(a["v"]), gh, a["gamma"], f(a["dout"]), **kw)
    got = (dq, dk, dv, dg, dgam) + ((dsig,) if temp else ())
    for name, gt, rf in zip(("dq", "dk", "dv", "dg", "dgamma", "dsigma"), got, ref):
        gt = to_np(gt)
        if far and name == "dg":  # dg_hj = gain_h colsum_h(j) / g_hj: compare the column sums
            sc = gh / a["gamma"][None, :, None]
            gt, rf = gt * sc, rf * sc
        assert_maxabs(gt, rf, tol, name)


@pytest.mark.parametrize("B,M,Hq,Hkv,D,rope,temp", [(2, 100, 4, 2, 128, True, False), (1, 257, 8, 2, 128, True, True),
                                                    (1, 190, 4, 4, 64, False, False), (2, 300, 16, 8, 128, True, True)])
def test_headgates_bf16(B, M, Hq, Hkv, D, rope, temp):
    _headgate_case(B, M, Hq, Hkv, D, rope=rope, temp=temp)


def test_headgates_zero_gates():
    _headgate_case(1, 150, 4, 2, 128, zero_heads=True)


@pytest.mark.parametrize("B,M,Hq,Hkv,temp", [(1, 200, 4, 2, False), (2, 700, 16, 8, True)])
def test_headgates_dead_leading_tiles_far_logits(B, M, Hq, Hkv, temp):
    _headgate_case(B, M, Hq, Hkv, 128, rope=False, temp=temp, far=True)


def test_headgates_f32():
    _headgate_case(1, 60, 4, 2, 32, dtype="f32", temp=True)


@pytest.mark.parametrize("temp", [False, True])
def test_headgates_d_from_o(temp):
    """The backward's row terms from the forward's o + o_lo, with per-head gates (one head without
    its early keys)."""
    _headgate_case(2, 300, 16, 8, 128, temp=temp, zero_heads=True, use_o=True)
