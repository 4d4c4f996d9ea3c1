"""Pins of the oracle's remaining scoring steps (CPU only).

DeepDive = "TokenGate: Learnable Token Pruning for Fast, Memory-Efficient LLM Prefill".
  * LN2 before the scorer (section 2, Eq. 1; section 3.1, Eq. 3): against PyTorch's
    rms_norm followed by the (separately pinned) scorer, scale invariance, the w = 1 reduction.
  * Sequence RMS normalisation (section 3.1, Eq. 3): a hand-worked example, the closed form
    of the normalised mean square, zeros on the non-prunable set, order preservation, scale
    invariance, an all-forced row.
  * Softmax-over-S gate (section 3.2, Eq. 5) and its backward: SciPy's softmax, padding,
    shift invariance, autograd, central finite differences; Eq. 6's per-head gain reproduced by
    the attention bias through this gate.
  * Per-head scores and uniform head aggregation (section 3.4): each head equals the single-head
    scorer with that row of w2; identical heads aggregate to themselves.  Per-head gates in the
    attention: equal heads reduce to the shared gate; otherwise fp64 SDPA with the per-head
    additive bias, and autograd for the per-head dg.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

import oracle


@pytest.fixture(scope="module")
def o():
    oracle.build(force=False)
    return oracle


def _mlp(seed, T, d, d_ff):
    rng = np.random.default_rng(seed)
    h = rng.normal(0.0, 2.0, (T, d))
    w1 = rng.normal(0.0, 1.0 / math.sqrt(d), (d_ff, d))
    w2 = rng.normal(0.0, 1.0 / math.sqrt(d_ff), d_ff)
    lw = rng.uniform(0.5, 1.5, d)
    return h, w1, w2, lw


def test_ln_scorer_matches_torch_rms_norm(o):
    h, w1, w2, lw = _mlp(1, 37, 48, 20)
    forced = np.zeros(37, np.uint8)
    forced[:5] = 1
    s, g = o.gate_score_ln(h, lw, 1e-6, w1, w2, forced)
    hn = torch.nn.functional.rms_norm(torch.from_numpy(h), (48,), torch.from_numpy(lw), 1e-6).numpy()
    s_ref, g_ref = o.gate_score(hn, w1, w2, forced)
    np.testing.assert_allclose(s, s_ref, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(g, g_ref, rtol=1e-13, atol=1e-14)


def test_rms_norm_matches_torch(o):
    h, _, _, lw = _mlp(11, 19, 48, 8)
    ref = torch.nn.functional.rms_norm(torch.from_numpy(h), (48,), torch.from_numpy(lw), 1e-5).numpy()
    np.testing.assert_allclose(o.rms_norm(h, lw, 1e-5), ref, rtol=1e-13, atol=1e-15)


def test_ln_scorer_scale_invariance_and_unit_weight(o):
    h, w1, w2, _ = _mlp(2, 25, 32, 16)
    s1, _ = o.gate_score_ln(h, None, 0.0, w1, w2)
    s2, _ = o.gate_score_ln(3.7 * h, None, 0.0, w1, w2)
    np.testing.assert_allclose(s1, s2, rtol=1e-12, atol=1e-13)
    # rows already at unit root mean square, w = 1, eps = 0: the normalisation is the identity
    hu = h / np.sqrt(np.mean(h * h, axis=1, keepdims=True))
    s3, _ = o.gate_score_ln(hu, None, 0.0, w1, w2)
    s4, _ = o.gate_score(hu, w1, w2)
    np.testing.assert_allclose(s3, s4, rtol=1e-12, atol=1e-13)


def test_normalize_hand_example(o):
    # P = {1, 2}: mean square (9 + 16) / 2 = 12.5, root 3.5355...; position 0 is forced
    out = o.score_normalize(np.array([[5.0, 3.0, -4.0]]), np.array([[1, 0, 0]], np.uint8), 0.0)
    r = math.sqrt(12.5)
    np.testing.assert_allclose(out, [[0.0, 3.0 / r, -4.0 / r]], rtol=1e-15)


def test_normalize_closed_form_and_invariants(o):
    rng = np.random.default_rng(3)
    B, N = 3, 257
    s = rng.normal(0.4, 2.5, (B, N))
    forced = (rng.random((B, N)) < 0.1).astype(np.uint8)
    eps = 0.3
    out = o.score_normalize(s, forced, eps)
    for b in range(B):
        p = forced[b] == 0
        S = np.mean(s[b, p] ** 2)
        # mean square of the normalised prunable scores = S / (S + eps)
        np.testing.assert_allclose(np.mean(out[b, p] ** 2), S / (S + eps), rtol=1e-13)
        assert np.all(out[b, ~p] == 0.0)
        # order (and sign) of the prunable scores preserved
        assert np.array_equal(np.argsort(out[b, p], kind="stable"), np.argsort(s[b, p], kind="stable"))
        assert np.all(np.sign(out[b, p]) == np.sign(s[b, p]))
    np.testing.assert_allclose(o.score_normalize(7.0 * s, forced, 0.0), o.score_normalize(s, forced, 0.0),
                               rtol=1e-13, atol=1e-15)
    # no forced mask: every position prunable; an all-forced row is all zeros
    full = o.score_normalize(s[:1], None, 0.0)
    np.testing.assert_allclose(np.mean(full ** 2), 1.0, rtol=1e-13)
    assert np.all(o.score_normalize(s[:1], np.ones((1, N), np.uint8), eps) == 0.0)


def test_gate_softmax_matches_scipy_and_padding(o):
    rng = np.random.default_rng(4)
    b = rng.normal(0.0, 1.5, (4, 33))
    g = o.gate_softmax(b)
    np.testing.assert_allclose(g, scipy.special.softmax(b, axis=1), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(g.sum(axis=1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(o.gate_softmax(b + 11.0), g, rtol=1e-12, atol=1e-16)
    kept = np.tile(np.arange(33, dtype=np.int32), (4, 1))
    kept[1, 30:] = -1
    gp = o.gate_softmax(b, kept)
    assert np.all(gp[1, 30:] == 0.0)
    np.testing.assert_allclose(gp[1, :30], scipy.special.softmax(b[1, :30]), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(gp[0], g[0], rtol=1e-15)


def test_gate_softmax_bwd_autograd_and_fd(o):
    rng = np.random.default_rng(5)
    b = rng.normal(0.0, 1.0, (3, 17))
    dg = rng.normal(0.0, 1.0, (3, 17))
    g = o.gate_softmax(b)
    db = o.gate_softmax_bwd(g, dg)
    x = torch.from_numpy(b).requires_grad_()
    (torch.softmax(x, dim=1) * torch.from_numpy(dg)).sum().backward()
    np.testing.assert_allclose(db, x.grad.numpy(), rtol=1e-12, atol=1e-15)
    h = 1e-6
    for (i, j) in [(0, 0), (1, 5), (2, 16)]:
        bp, bm = b.copy(), b.copy()
        bp[i, j] += h
        bm[i, j] -= h
        fd = ((o.gate_softmax(bp) - o.gate_softmax(bm)) * dg).sum() / (2 * h)
        assert abs(fd - db[i, j]) < 1e-8


def test_eq6_gain_through_the_attention_bias(o):
    """Attention with g = softmax_S(b) and gain c equals attention with the additive bias c b_j (Eq. 6)."""
    rng = np.random.default_rng(6)
    B, M, Hq, Hkv, D = 1, 12, 2, 1, 8
    q, k, v = (rng.normal(0.0, 1.0, (B, M, H, D)) for H in (Hq, Hkv, Hkv))
    b = rng.normal(0.0, 1.0, (B, M))
    c = np.array([0.7, 1.9])
    g = o.gate_softmax(b)
    o1, _ = o.attn_fwd(q, k, v, g, c)
    # the same logits with the bias written out: c_h b_j = c_h ln(e^{b_j})
    o2, _ = o.attn_fwd(q, k, v, np.exp(b), c)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    # and against fp64 SDPA with that additive bias
    qt, kt, vt = (torch.from_numpy(x).permute(0, 2, 1, 3) for x in (q, k, v))
    kt, vt = kt.repeat_interleave(Hq // Hkv, 1), vt.repeat_interleave(Hq // Hkv, 1)
    mask = torch.full((M, M), float("-inf"), dtype=torch.float64).triu(1)
    bias = torch.from_numpy(c)[None, :, None, None] * torch.from_numpy(b)[:, None, None, :] + mask
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias).permute(0, 2, 1, 3)
    np.testing.assert_allclose(o1, ref.numpy(), rtol=1e-11, atol=1e-12)


# --- per-head scores, uniform head aggregation, per-head gates (DeepDive section 3.4) ---

def test_score_heads_reduce_to_the_single_head_scorer(o):
    h, w1, _, _ = _mlp(7, 29, 40, 24)
    w2 = np.random.default_rng(8).normal(0.0, 0.2, (5, 24))
    sh = o.gate_score_heads(h, w1, w2)
    assert sh.shape == (5, 29)
    for k in range(5):
        s, _ = o.gate_score(h, w1, w2[k])
        np.testing.assert_allclose(sh[k], s, rtol=1e-13, atol=1e-15)
    # the uniform aggregation of identical heads is that head
    same = np.repeat(sh[:1], 4, axis=0)
    np.testing.assert_allclose(o.aggregate_heads(same), sh[0], rtol=1e-15)
    np.testing.assert_allclose(o.aggregate_heads(sh), sh.mean(axis=0), rtol=1e-14)


def test_per_head_gates_attention(o):
    """Per-head gates: equal heads reduce to the shared gate; otherwise fp64 SDPA with the per-head
    additive bias gamma_h ln g_hj, and autograd for the per-head dg."""
    rng = np.random.default_rng(10)
    B, M, Hq, Hkv, D = 2, 9, 4, 2, 8
    q, k, v = (rng.normal(0.0, 1.0, (B, M, H, D)) for H in (Hq, Hkv, Hkv))
    gamma = rng.uniform(0.5, 1.5, Hq)
    g1 = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, (B, M))))
    o_sh, l_sh = o.attn_fwd(q, k, v, g1, gamma)
    o_ph, l_ph = o.attn_fwd(q, k, v, np.repeat(g1[:, None, :], Hq, axis=1), gamma)
    np.testing.assert_allclose(o_ph, o_sh, rtol=1e-14, atol=1e-15)
    gh = 1.0 / (1.0 + np.exp(-rng.normal(0.0, 1.0, (B, Hq, M))))
    dout = rng.normal(0.0, 1.0, (B, M, Hq, D))
    leaves = [torch.from_numpy(a).requires_grad_() for a in (q, k, v, gh, gamma)]
    qt, kt, vt = (x.permute(0, 2, 1, 3) for x in leaves[:3])
    kt, vt = kt.repeat_interleave(Hq // Hkv, 1), vt.repeat_interleave(Hq // Hkv, 1)
    causal = torch.full((M, M), float("-inf"), dtype=torch.float64).triu(1)
    bias = leaves[4][None, :, None, None] * torch.log(leaves[3])[:, :, None, :] + causal
    ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=bias).permute(0, 2, 1, 3)
    out, _ = o.attn_fwd(q, k, v, gh, gamma)
    np.testing.assert_allclose(out, ref.detach().numpy(), rtol=1e-11, atol=1e-12)
    (ref * torch.from_numpy(dout)).sum().backward()
    got = o.attn_bwd(q, k, v, gh, gamma, dout)
    assert got[3].shape == (B, Hq, M)
    for a, leaf in zip(got, leaves):
        np.testing.assert_allclose(a, leaf.grad.numpy(), rtol=1e-10, atol=1e-11)
