"""GPU parity of the rest of the scoring definition against the CPU oracle.

  * tg_gate_score_ln: the scorer on the raw residual with the RMSNorm (LN2) in front
    (DeepDive section 2 Eq. 1, section 3.1 Eq. 3): scores and gates within 1e-2 (bf16) /
    1e-5 (fp32) of the oracle, relative to max(|ref|, rms(ref)).
  * tg_score_normalize (section 3.1 Eq. 3): within 1e-5 of the oracle on the same input
    scores; zeros on forced positions exactly; selection on the normalised scores bit-exact.
  * tg_gate_softmax / tg_gate_softmax_bwd (section 3.2 Eq. 5): within 1e-5; padding exactly 0.
  * the operative scoring path end to end: raw residual -> LN2 scorer -> normalisation ->
    selection -> compaction of b -> softmax gate -> attention with the per-head gain (Eq. 6),
    against the oracle's same chain, o within 2e-2.
"""
import numpy as np
import pytest

import oracle
from learned_token_pruning_gatescore_amd import workloads as wl
from tests._gpu import assert_maxabs, assert_scores_close, dev_tensor, device, say, to_np

pytestmark = pytest.mark.gpu


def _wl(B, N, d, d_ff, dtype="bf16", n_forced=5, seed=31):
    return wl.Workload("ln", seed, B=B, N=N, n_forced=min(n_forced, N), d=d, d_ff=d_ff, Ks=(1,), Hq=4, Hkv=2, D=128,
                       tau=1.0, dtype=dtype, rope=True)


def _score_ln(w, with_w=True, eps=1e-6, sample=None):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    gi = wl.gate_inputs(w)
    ri = wl.residual_inputs(w)
    h = dev_tensor(ri["hidden"], w.dtype, dev)
    lw = dev_tensor(ri["ln_w"], w.dtype, dev) if with_w else None
    w1, w2 = dev_tensor(gi["w1"], w.dtype, dev), dev_tensor(gi["w2"], w.dtype, dev)
    f = torch.from_numpy(gi["forced"]).to(dev)
    B, n = gi["forced"].shape
    scores = torch.full((B, n), float("nan"), device=dev)
    gates = torch.full((B, n), float("nan"), device=dev)
    ws = tg.gate_workspace(w.d, w.d_ff, h.dtype, dev)
    say("gate_score_ln", w.dtype, B, n, w.d, w.d_ff, "ln_w" if with_w else "no ln_w")
    tg.tg_gate_score_ln(h, lw, eps, w1, w2, f, scores, gates, ws)
    torch.cuda.synchronize()
    hf = wl.as_float(ri["hidden"], w.dtype).reshape(B * n, w.d)
    idx = np.arange(B * n) if sample is None else sample
    s_ref, g_ref = oracle.gate_score_ln(hf[idx], wl.as_float(ri["ln_w"], w.dtype) if with_w else None, eps,
                                        wl.as_float(gi["w1"], w.dtype), wl.as_float(gi["w2"], w.dtype),
                                        gi["forced"].reshape(-1)[idx])
    return to_np(scores).reshape(-1)[idx], to_np(gates).reshape(-1)[idx], s_ref, g_ref


# 64- and 128-token tiles, a ragged last tile, padded inputs (d % 64 == 32) and units
# (d_ff not a multiple of 32), two unit chunks (d_ff > 512)
@pytest.mark.parametrize("B,N,d,d_ff,with_w", [(2, 1000, 256, 96, True), (2, 300, 128, 640, True),
                                               (1, 513, 96, 100, False), (1, 33001, 128, 200, True),
                                               (1, 1, 32, 1, True)])
def test_score_ln_bf16_shapes(B, N, d, d_ff, with_w):
    s, g, sr, gr = _score_ln(_wl(B, N, d, d_ff), with_w=with_w)
    assert_scores_close(s, sr, 1e-2)
    assert_scores_close(g, gr, 1e-2, "gates")


def test_score_ln_f32():
    s, g, sr, gr = _score_ln(_wl(1, 300, 256, 64, dtype="f32"))
    assert_scores_close(s, sr, 1e-5)
    assert_scores_close(g, gr, 1e-5, "gates")


def test_score_ln_full_size_sampled():
    w = wl.WORKLOADS["qwen3_32k"]
    rng = np.random.default_rng(7)
    sample = np.unique(np.concatenate([[0, 127, 128, w.N - 1], rng.choice(w.N, 400, replace=False)]))
    s, g, sr, gr = _score_ln(w, sample=sample)
    assert_scores_close(s, sr, 1e-2)
    assert_scores_close(g, gr, 1e-2, "gates")


def _normalize(s_np, forced_np, eps):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    s = torch.from_numpy(s_np).to(dev)
    f = None if forced_np is None else torch.from_numpy(forced_np).to(dev)
    out = torch.full_like(s, float("nan"))
    say("score_normalize", s_np.shape, eps)
    tg.tg_score_normalize(s, f, eps, out)
    torch.cuda.synchronize()
    return to_np(out)


@pytest.mark.parametrize("B,N,eps", [(3, 32768, 1e-6), (2, 1000, 0.0), (1, 1, 1e-6), (2, 70001, 0.5)])
def test_score_normalize(B, N, eps):
    rng = np.random.default_rng(N)
    s = rng.normal(0.3, 2.0, (B, N)).astype(np.float32)
    forced = (rng.random((B, N)) < 0.05).astype(np.uint8)
    forced[:, :3] = 1
    out = _normalize(s, forced, eps)
    ref = oracle.score_normalize(s, forced, eps)
    assert np.all(out[forced == 1] == 0.0)
    assert_scores_close(out.reshape(-1), ref.reshape(-1), 1e-5)


def test_score_normalize_edge_rows_and_in_place():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    rng = np.random.default_rng(8)
    s = rng.normal(0.0, 1.0, (3, 500)).astype(np.float32)
    forced = np.zeros((3, 500), np.uint8)
    forced[1] = 1  # a row with no prunable position: all zeros
    out = _normalize(s, forced, 1e-6)
    assert np.all(out[1] == 0.0)
    assert_scores_close(out.reshape(-1), oracle.score_normalize(s, forced, 1e-6).reshape(-1), 1e-5)
    # no mask: every position prunable; in place gives the same bits
    dev = device()
    t = torch.from_numpy(s).to(dev)
    o2 = torch.empty_like(t)
    tg.tg_score_normalize(t, None, 1e-6, o2)
    tg.tg_score_normalize(t, None, 1e-6, t)
    torch.cuda.synchronize()
    assert torch.equal(t.view(torch.int32), o2.view(torch.int32))
    assert_scores_close(to_np(o2).reshape(-1), oracle.score_normalize(s, None, 1e-6).reshape(-1), 1e-5)


def test_selection_on_normalized_scores_bit_exact():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = wl.WORKLOADS["qwen3_32k"]
    sel = wl.clustered_scores(w)
    forced = wl.forced_mask(w)
    out = _normalize(sel, forced, 1e-6)
    dev = device()
    K = w.Ks[0]
    M = w.M(K)
    kept = torch.full((w.B, M), -7, dtype=torch.int32, device=dev)
    tg.tg_select_topk(torch.from_numpy(out).to(dev), torch.from_numpy(forced).to(dev), K, w.n_forced, kept)
    torch.cuda.synchronize()
    kept_ref, _ = oracle.select_topk(out, forced, K)  # the same (GPU-normalised) score vector
    assert np.array_equal(to_np(kept), kept_ref)


def _softmax(b_np, kept_np):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    b = torch.from_numpy(b_np).to(dev)
    k = None if kept_np is None else torch.from_numpy(kept_np).to(dev)
    g = torch.full_like(b, float("nan"))
    say("gate_softmax", b_np.shape)
    tg.tg_gate_softmax(b, k, g)
    torch.cuda.synchronize()
    return to_np(g)


@pytest.mark.parametrize("B,M", [(1, 2176), (4, 2048), (2, 1), (1, 70000), (3, 1500)])
def test_gate_softmax(B, M):
    rng = np.random.default_rng(M)
    b = rng.normal(0.0, 1.0, (B, M)).astype(np.float32)
    kept = np.tile(np.arange(M, dtype=np.int32), (B, 1))
    if M > 10:
        kept[0, -7:] = -1  # padding
    g = _softmax(b, kept)
    ref = oracle.gate_softmax(b, kept)
    assert np.all(g[kept < 0] == 0.0)
    assert_scores_close(g.reshape(-1), ref.reshape(-1), 1e-5, "g")
    g2 = _softmax(b, None)
    assert_scores_close(g2.reshape(-1), oracle.gate_softmax(b).reshape(-1), 1e-5, "g")


def test_gate_softmax_all_padding_row():
    b = np.random.default_rng(9).normal(0.0, 1.0, (2, 300)).astype(np.float32)
    kept = np.tile(np.arange(300, dtype=np.int32), (2, 1))
    kept[1] = -1
    g = _softmax(b, kept)
    assert np.all(g[1] == 0.0)
    assert_scores_close(g[0], oracle.gate_softmax(b[0]), 1e-5, "g")


@pytest.mark.parametrize("B,M", [(1, 2176), (4, 2048), (1, 33)])
def test_gate_softmax_bwd(B, M):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    rng = np.random.default_rng(M + 1)
    g = oracle.gate_softmax(rng.normal(0.0, 1.0, (B, M))).astype(np.float32)
    dg = rng.normal(0.0, 1.0, (B, M)).astype(np.float32)
    dev = device()
    db = torch.full((B, M), float("nan"), device=dev)
    say("gate_softmax_bwd", B, M)
    tg.tg_gate_softmax_bwd(torch.from_numpy(g).to(dev), torch.from_numpy(dg).to(dev), db)
    torch.cuda.synchronize()
    assert_scores_close(to_np(db).reshape(-1), oracle.gate_softmax_bwd(g, dg).reshape(-1), 1e-5, "db")


def test_operative_scoring_path_end_to_end():
    """Raw residual -> LN2 scorer -> Eq. 3 normalisation -> selection -> compaction -> Eq. 5 gate ->
    attention with the per-head gain (Eq. 6), against the oracle's chain on the same selection."""
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = _wl(1, 2000, 256, 128, n_forced=16)
    K = 300
    M = w.M(K)
    dev = device()
    gi, ri = wl.gate_inputs(w), wl.residual_inputs(w)
    h = dev_tensor(ri["hidden"], w.dtype, dev)
    lw = dev_tensor(ri["ln_w"], w.dtype, dev)
    w1, w2 = dev_tensor(gi["w1"], w.dtype, dev), dev_tensor(gi["w2"], w.dtype, dev)
    f = torch.from_numpy(gi["forced"]).to(dev)
    raw = torch.empty((1, w.N), device=dev)
    b = torch.empty((1, w.N), device=dev)
    kept = torch.empty((1, M), dtype=torch.int32, device=dev)
    hk = torch.empty((1, M, w.d), dtype=h.dtype, device=dev)
    pk = torch.empty((1, M), dtype=torch.int32, device=dev)
    bk = torch.empty((1, M), device=dev)
    g = torch.empty((1, M), device=dev)
    ws = tg.gate_workspace(w.d, w.d_ff, h.dtype, dev)
    say("operative path", w.N, K, M)
    tg.tg_gate_score_ln(h, lw, 1e-6, w1, w2, f, raw, None, ws)
    tg.tg_score_normalize(raw, f, 1e-6, b)
    tg.tg_select_topk(b, f, K, w.n_forced, kept)
    tg.tg_compact(h, None, b, kept, hk, pk, bk)
    tg.tg_gate_softmax(bk, kept, g)
    at = wl.attn_inputs(w, M)
    q, k, v = (dev_tensor(at[n], w.dtype, dev) for n in ("q", "k", "v"))
    gain = np.log1p(np.exp(at["sigma"])).astype(np.float32)  # softplus of a raw per-head parameter
    o = torch.empty_like(q)
    lse = torch.empty((1, w.Hq, M), device=dev)
    aws = tg.attn_workspace(1, M, w.Hq, w.Hkv, w.D, False, dev)
    tg.tg_gated_attn_fwd(q, k, v, g, torch.from_numpy(gain).to(dev), pk, wl.ROPE_THETA, w.tau, o, lse, aws)
    torch.cuda.synchronize()
    # oracle chain: scores within tolerance, then the same selection on the GPU's b
    hf = wl.as_float(ri["hidden"], w.dtype).reshape(w.N, w.d)
    s_ref, _ = oracle.gate_score_ln(hf, wl.as_float(ri["ln_w"], w.dtype), 1e-6, wl.as_float(gi["w1"], w.dtype),
                                    wl.as_float(gi["w2"], w.dtype), gi["forced"][0])
    assert_scores_close(to_np(raw).reshape(-1), s_ref, 1e-2)
    b_np = to_np(b)
    assert_scores_close(b_np.reshape(-1), oracle.score_normalize(to_np(raw), gi["forced"], 1e-6).reshape(-1), 1e-5)
    kept_ref, _ = oracle.select_topk(b_np, gi["forced"], K)
    assert np.array_equal(to_np(kept), kept_ref)
    g_ref = oracle.gate_softmax(b_np[0, kept_ref[0]])
    assert_scores_close(to_np(g).reshape(-1), g_ref, 1e-5, "g")
    f32 = lambda x: wl.as_float(x, w.dtype)
    o_ref, _ = oracle.attn_fwd(f32(at["q"]), f32(at["k"]), f32(at["v"]), g_ref[None], gain, pos=kept_ref,
                               theta=wl.ROPE_THETA, tau=w.tau, round_bf16=True)
    assert_maxabs(to_np(o), o_ref, 2e-2, "o")
