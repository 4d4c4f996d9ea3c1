"""Pins of the oracle's token-gated attention, forward and backward (CPU only).

TokenGate deep dive: section 2 Eq. 2 (causal attention with z = q.k/sqrt(d)),
section 3.2 Eq. 5 (weights multiplied by the key's gate value and
renormalised), Eq. 6 (per-head non-negative gain), and section 3.4 (the
temperature folded into the query-side scale, the gate passed as a per-key
bias).  Summary page, Figure 1(c): each attention weight is multiplied by its
key's gate value.  Form: S_ij = q^.k^/(sqrt(D) tau) + gamma_h ln g_j, j <= i.

The oracle is checked against PyTorch's CPU scaled_dot_product_attention in
float64 with an additive mask, against the multiplicative form of Eq. 5
written with NumPy, against autograd and central finite differences, and
against closed forms and invariances.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F


def _rope_complex(x, pos, theta):
    """Rotary embedding as complex multiplication: pair (x_i, x_{i+D/2}) -> x_i + 1j x_{i+D/2},
    multiplied by exp(1j * p * theta^(-2i/D)).  x: [B, M, H, D] (torch float64)."""
    D = x.shape[-1]
    h = D // 2
    inv = torch.tensor([theta ** (-2.0 * i / D) for i in range(h)], dtype=torch.float64)
    ang = pos.to(torch.float64)[:, :, None, None] * inv  # [B, M, 1, h]
    z = torch.complex(x[..., :h], x[..., h:]) * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([z.real, z.imag], dim=-1)


def _bf16_arith(x):
    """Round float64 values to bf16 arithmetically (frexp, 8 significant bits, half-to-even)."""
    m, e = torch.frexp(x)
    return torch.ldexp(torch.round(m * 256.0) / 256.0, e.to(torch.float64))


def _sdpa_ref(q, k, v, g, gamma, tau, pos=None, theta=1e6, round_=False, st_round=False):
    """Library reference: SDPA (float64, CPU) with an additive float mask gamma_h ln g_j on
    j <= i and -inf above the diagonal; K/V repeated for GQA."""
    B, M, Hq, D = q.shape
    grp = Hq // k.shape[2]
    if pos is not None:
        q = _rope_complex(q, pos, theta)
        k = _rope_complex(k, pos, theta)
        if round_:
            if st_round:
                q = q + (_bf16_arith(q) - q).detach()
                k = k + (_bf16_arith(k) - k).detach()
            else:
                q, k = _bf16_arith(q), _bf16_arith(k)
    qh = q.permute(0, 2, 1, 3)
    kh = k.repeat_interleave(grp, dim=2).permute(0, 2, 1, 3)
    vh = v.repeat_interleave(grp, dim=2).permute(0, 2, 1, 3)
    bias = gamma[None, :, None, None] * torch.log(g)[:, None, None, :]  # [B, Hq, 1, M]
    causal = torch.ones(M, M, dtype=torch.bool).tril()
    mask = torch.where(causal[None, None], bias, torch.tensor(float("-inf"), dtype=torch.float64))
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=1.0 / (math.sqrt(D) * tau))
    return o.permute(0, 2, 1, 3)


def _inputs(seed, B=2, M=13, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, M, Hq, D))
    k = rng.standard_normal((B, M, Hkv, D))
    v = rng.standard_normal((B, M, Hkv, D))
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal((B, M))))
    gamma = rng.uniform(0.5, 1.5, Hq)
    pos = np.sort(rng.choice(1000, (B, M), replace=True), axis=1).astype(np.int32)
    return q, k, v, g, gamma, pos


T = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("shape", [(2, 13, 4, 2, 8), (1, 7, 3, 1, 6), (1, 20, 2, 2, 16)])
def test_fwd_matches_sdpa(oracle_mod, rope, shape):
    B, M, Hq, Hkv, D = shape
    q, k, v, g, gamma, pos = _inputs(11, B, M, Hq, Hkv, D)
    tau = 1.3
    p = pos if rope else None
    o, lse = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=p, theta=500.0, tau=tau)
    ref = _sdpa_ref(T(q), T(k), T(v), T(g), T(gamma), tau, torch.from_numpy(pos) if rope else None, 500.0)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)
    # lse against logsumexp of the same logits
    qq, kk = T(q), T(k)
    if rope:
        qq, kk = _rope_complex(qq, torch.from_numpy(pos), 500.0), _rope_complex(kk, torch.from_numpy(pos), 500.0)
    kk = kk.repeat_interleave(Hq // Hkv, dim=2)
    S = torch.einsum("bihd,bjhd->bhij", qq, kk) / (math.sqrt(D) * tau)
    S = S + T(gamma)[None, :, None, None] * torch.log(T(g))[:, None, None, :]
    S = S.masked_fill(~torch.ones(M, M, dtype=torch.bool).tril(), float("-inf"))
    np.testing.assert_allclose(lse, torch.logsumexp(S, -1).numpy(), rtol=1e-12, atol=1e-12)


def test_fwd_bf16_rounding_point(oracle_mod):
    q, k, v, g, gamma, pos = _inputs(12, 1, 16, 2, 1, 8)
    o, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=pos, theta=1e4, tau=1.0, round_bf16=True)
    ref = _sdpa_ref(T(q), T(k), T(v), T(g), T(gamma), 1.0, torch.from_numpy(pos), 1e4, round_=True)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_fwd_multiplicative_form_eq5(oracle_mod):
    """exp(z_ij / tau) g_j^gamma renormalised over j <= i equals the log-space rule."""
    q, k, v, g, gamma, _ = _inputs(13, 1, 9, 2, 2, 4)
    tau = 0.8
    o, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, tau=tau)
    M, D = 9, 4
    for h in range(2):
        for i in range(M):
            w = np.array([math.exp(np.dot(q[0, i, h], k[0, j, h]) / (math.sqrt(D) * tau)) * g[0, j] ** gamma[h]
                          for j in range(i + 1)])
            ref = (w[:, None] * v[0, : i + 1, h]).sum(0) / w.sum()
            np.testing.assert_allclose(o[0, i, h], ref, rtol=1e-12, atol=1e-13)


def test_fwd_reductions(oracle_mod):
    q, k, v, g, gamma, pos = _inputs(14, 2, 11, 4, 2, 8)
    # gamma = 0 -> plain causal attention (is_causal SDPA), whatever g is
    o0, _ = oracle_mod.attn_fwd(q, k, v, g, np.zeros(4))
    qh = T(q).permute(0, 2, 1, 3)
    kh = T(k).repeat_interleave(2, dim=2).permute(0, 2, 1, 3)
    vh = T(v).repeat_interleave(2, dim=2).permute(0, 2, 1, 3)
    ref = F.scaled_dot_product_attention(qh, kh, vh, is_causal=True).permute(0, 2, 1, 3)
    np.testing.assert_allclose(o0, ref.numpy(), rtol=1e-11, atol=1e-12)
    # g == 1 -> the same unpruned causal attention
    o1, _ = oracle_mod.attn_fwd(q, k, v, np.ones_like(g), gamma)
    np.testing.assert_allclose(o1, ref.numpy(), rtol=1e-11, atol=1e-12)
    # g -> lambda g: identical output (a constant shift of every logit of a row)
    oa, _ = oracle_mod.attn_fwd(q, k, v, g, gamma)
    ob, _ = oracle_mod.attn_fwd(q, k, v, g * 0.37, gamma)
    np.testing.assert_allclose(oa, ob, rtol=1e-11, atol=1e-12)
    # row 0 sees only key 0: O_0 = v_0, lse_0 = S_00
    o, lse = oracle_mod.attn_fwd(q, k, v, g, gamma, tau=1.1)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(o[b, 0, h], v[b, 0, h // 2], rtol=1e-14)
            s00 = np.dot(q[b, 0, h], k[b, 0, h // 2]) / (math.sqrt(8) * 1.1) + gamma[h] * math.log(g[b, 0])
            assert abs(lse[b, h, 0] - s00) < 1e-12
    # M = 1
    o, lse = oracle_mod.attn_fwd(q[:, :1], k[:, :1], v[:, :1], g[:, :1], gamma)
    np.testing.assert_allclose(o[:, 0], np.repeat(v[:, 0], 2, axis=1), rtol=1e-14)


def test_fwd_rope_properties(oracle_mod):
    q, k, v, g, gamma, pos = _inputs(15, 1, 10, 2, 2, 8)
    base, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=None)
    # position 0 everywhere: identity rotation
    o, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=np.zeros_like(pos))
    np.testing.assert_allclose(o, base, rtol=1e-12, atol=1e-13)
    # q^.k^ depends only on position differences: shifting every position leaves O unchanged
    oa, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=pos, theta=100.0)
    ob, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=pos + 12345, theta=100.0)
    np.testing.assert_allclose(oa, ob, rtol=1e-8, atol=1e-9)


def test_fwd_zero_gate_and_rows(oracle_mod):
    q, k, v, g, gamma, _ = _inputs(16, 1, 8, 2, 2, 4)
    g = g.copy()
    g[0, 0] = 0.0  # key 0 gets weight 0; row 0 has no visible key
    o, lse = oracle_mod.attn_fwd(q, k, v, g, gamma)
    assert np.all(o[0, 0] == 0.0) and np.all(np.isneginf(lse[0, :, 0]))
    o2, _ = oracle_mod.attn_fwd(q[:, 1:], k[:, 1:], v[:, 1:], g[:, 1:], gamma)
    np.testing.assert_allclose(o[0, 1:], o2[0], rtol=1e-12, atol=1e-13)
    # a row subset reproduces the full computation on those rows and leaves others NaN
    full, lfull = oracle_mod.attn_fwd(q, k, v, g, gamma)
    part, lpart = oracle_mod.attn_fwd(q, k, v, g, gamma, rows=[3, 7])
    np.testing.assert_array_equal(part[0, [3, 7]], full[0, [3, 7]])
    np.testing.assert_array_equal(lpart[0][:, [3, 7]], lfull[0][:, [3, 7]])
    assert np.isnan(part[0, 2]).all()


@pytest.mark.parametrize("rope", [False, True])
def test_bwd_matches_autograd(oracle_mod, rope):
    B, M, Hq, Hkv, D = 2, 12, 4, 2, 8
    q, k, v, g, gamma, pos = _inputs(21, B, M, Hq, Hkv, D)
    dout = np.random.default_rng(22).standard_normal((B, M, Hq, D))
    tau = 0.9
    p = pos if rope else None
    dq, dk, dv, dg, dgam = oracle_mod.attn_bwd(q, k, v, g, gamma, dout, pos=p, theta=300.0, tau=tau)
    tq, tk, tv, tg, tgam = (T(a).requires_grad_() for a in (q, k, v, g, gamma))
    o = _sdpa_ref(tq, tk, tv, tg, tgam, tau, torch.from_numpy(pos) if rope else None, 300.0)
    (o * T(dout)).sum().backward()
    for got, ref in ((dq, tq), (dk, tk), (dv, tv), (dg, tg), (dgam, tgam)):
        np.testing.assert_allclose(got, ref.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_bwd_straight_through_rounding(oracle_mod):
    B, M, Hq, Hkv, D = 1, 10, 2, 1, 8
    q, k, v, g, gamma, pos = _inputs(23, B, M, Hq, Hkv, D)
    dout = np.random.default_rng(24).standard_normal((B, M, Hq, D))
    got = oracle_mod.attn_bwd(q, k, v, g, gamma, dout, pos=pos, theta=1e4, tau=1.0, round_bf16=True)
    tq, tk, tv, tg, tgam = (T(a).requires_grad_() for a in (q, k, v, g, gamma))
    o = _sdpa_ref(tq, tk, tv, tg, tgam, 1.0, torch.from_numpy(pos), 1e4, round_=True, st_round=True)
    (o * T(dout)).sum().backward()
    for a, ref in zip(got, (tq, tk, tv, tg, tgam)):
        np.testing.assert_allclose(a, ref.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_bwd_finite_differences(oracle_mod):
    B, M, Hq, Hkv, D = 1, 5, 2, 1, 4
    q, k, v, g, gamma, pos = _inputs(25, B, M, Hq, Hkv, D)
    dout = np.random.default_rng(26).standard_normal((B, M, Hq, D))
    grads = oracle_mod.attn_bwd(q, k, v, g, gamma, dout, pos=pos, theta=50.0, tau=1.2)
    args = [q, k, v, g, gamma]

    def loss(a):
        o, _ = oracle_mod.attn_fwd(*a, pos=pos, theta=50.0, tau=1.2)
        return float((o * dout).sum())

    h = 1e-6
    rng = np.random.default_rng(27)
    for which in range(5):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in args[which].shape)
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[which][idx] += h
            am[which][idx] -= h
            fd = (loss(ap) - loss(am)) / (2 * h)
            assert abs(fd - grads[which][idx]) < 1e-6 * max(1.0, abs(fd)), (which, idx, fd, grads[which][idx])


def test_bwd_invariants(oracle_mod):
    B, M, Hq, Hkv, D = 2, 16, 4, 2, 8
    q, k, v, g, gamma, pos = _inputs(28, B, M, Hq, Hkv, D)
    dout = np.random.default_rng(29).standard_normal((B, M, Hq, D))
    dq, dk, dv, dg, dgam = oracle_mod.attn_bwd(q, k, v, g, gamma, dout, pos=pos, theta=1e4)
    # softmax shift invariance: sum_j g_j dg_j = 0 for every batch row
    np.testing.assert_allclose((g * dg).sum(axis=1), 0.0, atol=1e-11)
    # gamma = 0: the gate has no effect, so dg = 0
    _, _, _, dg0, _ = oracle_mod.attn_bwd(q, k, v, g, np.zeros(Hq), dout)
    assert np.abs(dg0).max() < 1e-12
    # dgamma_h = sum_j colsum_h(j) ln g_j and dg_j = sum_h gamma_h colsum_h(j) / g_j:
    # with a single head, dgamma = sum_j g_j dg_j ln g_j / gamma
    q1, k1, v1, g1, gam1, _ = _inputs(30, 1, 9, 1, 1, 4)
    d1 = np.random.default_rng(31).standard_normal((1, 9, 1, 4))
    _, _, _, dg1, dgam1 = oracle_mod.attn_bwd(q1, k1, v1, g1, gam1, d1)
    np.testing.assert_allclose(dgam1[0], (g1 * dg1 * np.log(g1)).sum() / gam1[0], rtol=1e-10)


# ---------------------------------------------------------------------------
# The operative rule with the pruning-ratio temperature (DeepDive section 3.2,
# Eq. 7 and Eq. 8): S_ij = tau_ih (q^.k^ / (sqrt(D) tau) + gamma_h ln g_j),
# tau_ih = softplus(sigma_h) ln m_i / ln max(2, p_i), m_i = i + 1, p_i = pos_i + 1.
# ---------------------------------------------------------------------------
def _temp(sigma, pos, B, M):
    """tau [B, M, Hq] from Eq. 7 (torch, differentiable in sigma)."""
    m = torch.arange(1, M + 1, dtype=torch.float64)[None, :].expand(B, M)
    p = (pos.to(torch.float64) + 1.0) if pos is not None else m
    r = torch.log(m) / torch.log(torch.clamp(p, min=2.0))
    return F.softplus(sigma)[None, None, :] * r[:, :, None]


def _sdpa_temp_ref(q, k, v, g, gamma, sigma, tau, pos=None, theta=1e6):
    """SDPA with the temperature folded in: the query scaled by tau_ih / (sqrt(D) tau) and the
    additive mask tau_ih gamma_h ln g_j (both per row and head)."""
    B, M, Hq, D = q.shape
    grp = Hq // k.shape[2]
    t = _temp(sigma, pos, B, M)  # [B, M, Hq]
    if pos is not None:
        q = _rope_complex(q, pos, theta)
        k = _rope_complex(k, pos, theta)
    qh = (q * t[..., None] / (math.sqrt(D) * tau)).permute(0, 2, 1, 3)
    kh = k.repeat_interleave(grp, dim=2).permute(0, 2, 1, 3)
    vh = v.repeat_interleave(grp, dim=2).permute(0, 2, 1, 3)
    bias = t.permute(0, 2, 1)[..., None] * gamma[None, :, None, None] * torch.log(g)[:, None, None, :]
    causal = torch.ones(M, M, dtype=torch.bool).tril()
    mask = torch.where(causal[None, None], bias, torch.tensor(float("-inf"), dtype=torch.float64))
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=1.0)
    return o.permute(0, 2, 1, 3)


@pytest.mark.parametrize("rope", [False, True])
def test_temp_fwd_matches_sdpa(oracle_mod, rope):
    B, M, Hq, Hkv, D = 2, 14, 4, 2, 8
    q, k, v, g, gamma, pos = _inputs(41, B, M, Hq, Hkv, D)
    sigma = np.random.default_rng(42).normal(0.0, 1.0, Hq)
    p = pos if rope else None
    o, lse = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=p, theta=400.0, tau=1.1, sigma=sigma)
    ref = _sdpa_temp_ref(T(q), T(k), T(v), T(g), T(gamma), T(sigma), 1.1, torch.from_numpy(pos) if rope else None,
                         400.0)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)


def test_temp_closed_form_and_reductions(oracle_mod):
    B, M, Hq, Hkv, D = 1, 9, 2, 1, 4
    q, k, v, g, gamma, pos = _inputs(43, B, M, Hq, Hkv, D)
    sigma = np.array([0.3, -0.7])
    # q = 0: S_ij = tau_i gamma_h ln g_j, so P_ij is proportional to g_j^(tau_i gamma_h)
    pos = np.array([[0, 3, 4, 10, 11, 40, 41, 42, 300]], dtype=np.int32)
    o, _ = oracle_mod.attn_fwd(np.zeros_like(q), k, v, g, gamma, pos=pos, sigma=sigma)
    sp = np.log1p(np.exp(sigma))
    for h in range(Hq):
        for i in range(M):
            t = sp[h] * math.log(i + 1) / math.log(max(2.0, pos[0, i] + 1.0))
            w = g[0, : i + 1] ** (t * gamma[h])
            ref = (w[:, None] * v[0, : i + 1, 0]).sum(0) / w.sum()
            np.testing.assert_allclose(o[0, i, h], ref, rtol=1e-12, atol=1e-13)
    # softplus(sigma) = 1 and no positions (p_i = m_i): tau = 1 on every row that sees more
    # than one key, so the output is the temperature-free one
    one = np.full(Hq, math.log(math.e - 1.0))
    o1, l1 = oracle_mod.attn_fwd(q, k, v, g, gamma, sigma=one)
    o0, l0 = oracle_mod.attn_fwd(q, k, v, g, gamma)
    np.testing.assert_allclose(o1, o0, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1[:, :, 1:], l0[:, :, 1:], rtol=1e-12, atol=1e-13)
    assert np.all(l1[:, :, 0] == 0.0)  # row 0: tau = 0, one key, logit 0


@pytest.mark.parametrize("rope", [False, True])
def test_temp_bwd_matches_autograd(oracle_mod, rope):
    B, M, Hq, Hkv, D = 2, 12, 4, 2, 8
    q, k, v, g, gamma, pos = _inputs(44, B, M, Hq, Hkv, D)
    sigma = np.random.default_rng(45).normal(0.0, 1.0, Hq)
    dout = np.random.default_rng(46).standard_normal((B, M, Hq, D))
    p = pos if rope else None
    got = oracle_mod.attn_bwd(q, k, v, g, gamma, dout, pos=p, theta=300.0, tau=0.9, sigma=sigma)
    leaves = [T(a).requires_grad_() for a in (q, k, v, g, gamma, sigma)]
    o = _sdpa_temp_ref(*leaves[:5], leaves[5], 0.9, torch.from_numpy(pos) if rope else None, 300.0)
    (o * T(dout)).sum().backward()
    assert len(got) == 6
    for a, ref in zip(got, leaves):
        np.testing.assert_allclose(a, ref.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_temp_bwd_finite_differences(oracle_mod):
    B, M, Hq, Hkv, D = 1, 6, 2, 1, 4
    q, k, v, g, gamma, pos = _inputs(47, B, M, Hq, Hkv, D)
    sigma = np.array([0.4, -1.2])
    dout = np.random.default_rng(48).standard_normal((B, M, Hq, D))
    grads = oracle_mod.attn_bwd(q, k, v, g, gamma, dout, pos=pos, theta=60.0, sigma=sigma)

    def loss(s):
        o, _ = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=pos, theta=60.0, sigma=s)
        return float((o * dout).sum())

    h = 1e-6
    for j in range(Hq):
        sp, sm = sigma.copy(), sigma.copy()
        sp[j] += h
        sm[j] -= h
        fd = (loss(sp) - loss(sm)) / (2 * h)
        assert abs(fd - grads[5][j]) < 1e-6 * max(1.0, abs(fd)), (j, fd, grads[5][j])
    # dg under the temperature: sum_j g_j dg_j = 0 still holds (each row's softmax is shift-free)
    np.testing.assert_allclose((g * grads[3]).sum(axis=1), 0.0, atol=1e-11)


# --- packed variable-length sequences (the training path packs both budgets in one call) ---

def _sdpa_varlen_ref(q, k, v, g, gamma, cu, tau, pos=None, theta=1e6, sigma=None):
    """fp64 SDPA over all packed tokens as one sequence, with a mask that is causal inside each
    sequence and -inf across sequences; the temperature's m_i counts from the sequence start."""
    T_, Hq, D = q.shape
    grp = Hq // k.shape[1]
    seg = torch.from_numpy(np.repeat(np.arange(len(cu) - 1), np.diff(cu)))
    idx = torch.arange(T_) - torch.from_numpy(np.asarray(cu[:-1]))[seg]
    if pos is not None:
        q = _rope_complex(q[None], pos[None], theta)[0]
        k = _rope_complex(k[None], pos[None], theta)[0]
    t = torch.ones(T_, Hq, dtype=torch.float64)
    if sigma is not None:
        p = (pos.to(torch.float64) if pos is not None else idx.to(torch.float64)) + 1.0
        ratio = torch.log(idx.to(torch.float64) + 1.0) / torch.log(torch.clamp(p, min=2.0))
        t = torch.nn.functional.softplus(sigma)[None, :] * ratio[:, None]
    qh = (q * t[..., None] / (math.sqrt(D) * tau)).permute(1, 0, 2)[None]
    kh = k.repeat_interleave(grp, dim=1).permute(1, 0, 2)[None]
    vh = v.repeat_interleave(grp, dim=1).permute(1, 0, 2)[None]
    allowed = (seg[:, None] == seg[None, :]) & (torch.arange(T_)[None, :] <= torch.arange(T_)[:, None])
    bias = t.permute(1, 0)[:, :, None] * gamma[:, None, None] * torch.log(g)[None, None, :]
    mask = torch.where(allowed[None], bias, torch.tensor(float("-inf"), dtype=torch.float64))[None]
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=1.0)
    return o[0].permute(1, 0, 2)


def _varlen_inputs(seed, lens, Hq=4, Hkv=2, D=8):
    rng = np.random.default_rng(seed)
    T_ = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    q = rng.standard_normal((T_, Hq, D))
    k = rng.standard_normal((T_, Hkv, D))
    v = rng.standard_normal((T_, Hkv, D))
    g = 1.0 / (1.0 + np.exp(-rng.standard_normal(T_)))
    gamma = rng.uniform(0.5, 1.5, Hq)
    pos = np.concatenate([np.sort(rng.choice(200, n, replace=False)) for n in lens]).astype(np.int32)
    sigma = rng.normal(0.0, 1.0, Hq)
    return q, k, v, g, gamma, cu, pos, sigma


@pytest.mark.parametrize("rope", [False, True])
@pytest.mark.parametrize("temp", [False, True])
def test_varlen_matches_blockdiag_sdpa(oracle_mod, rope, temp):
    lens = [5, 0, 9, 1, 7]
    q, k, v, g, gamma, cu, pos, sigma = _varlen_inputs(51, lens)
    p = pos if rope else None
    o, lse = oracle_mod.attn_fwd_varlen(q, k, v, g, gamma, cu, pos=p, theta=300.0, tau=1.2,
                                        sigma=sigma if temp else None)
    ref = _sdpa_varlen_ref(T(q), T(k), T(v), T(g), T(gamma), cu, 1.2, torch.from_numpy(pos) if rope else None,
                           300.0, T(sigma) if temp else None)
    np.testing.assert_allclose(o, ref.numpy(), rtol=1e-11, atol=1e-12)
    assert lse.shape == (4 * sum(lens),) and np.all(np.isfinite(lse))


def test_varlen_equal_lengths_is_the_batch(oracle_mod):
    q, k, v, g, gamma, pos = _inputs(52, 3, 11, 4, 2, 8)
    cu = np.arange(4) * 11
    o, lse = oracle_mod.attn_fwd_varlen(q.reshape(33, 4, 8), k.reshape(33, 2, 8), v.reshape(33, 2, 8), g.reshape(-1),
                                        gamma, cu, pos=pos.reshape(-1), theta=400.0)
    ob, lb = oracle_mod.attn_fwd(q, k, v, g, gamma, pos=pos, theta=400.0)
    np.testing.assert_allclose(o.reshape(3, 11, 4, 8), ob, rtol=1e-14, atol=1e-15)
    np.testing.assert_allclose(lse.reshape(3, 4, 11), lb, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("temp", [False, True])
def test_varlen_bwd_matches_autograd(oracle_mod, temp):
    lens = [6, 0, 4, 9]
    q, k, v, g, gamma, cu, pos, sigma = _varlen_inputs(53, lens)
    dout = np.random.default_rng(54).standard_normal(q.shape)
    got = oracle_mod.attn_bwd_varlen(q, k, v, g, gamma, dout, cu, pos=pos, theta=250.0, tau=0.8,
                                     sigma=sigma if temp else None)
    leaves = [T(a).requires_grad_() for a in (q, k, v, g, gamma, sigma)]
    o = _sdpa_varlen_ref(*leaves[:5], cu, 0.8, torch.from_numpy(pos), 250.0, leaves[5] if temp else None)
    (o * T(dout)).sum().backward()
    n = 6 if temp else 5
    assert len(got) == n
    for a, ref in zip(got, leaves[:n]):
        np.testing.assert_allclose(a, ref.grad.numpy(), rtol=1e-10, atol=1e-11)
