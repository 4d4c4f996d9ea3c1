"""GPU parity of token-gated attention (forward and backward) against the CPU oracle.

Tolerances: max-abs 2e-2 in bf16 and 1e-4 in fp32 for o and every gradient;
lse within the same bounds.  The oracle rounds the rotated q and k to bf16 for
bf16 inputs, the precision the matrix cores consume.
"""
import numpy as np
import pytest

import oracle
from learned_token_pruning_gatescore_amd import workloads as wl
from tests._gpu import assert_maxabs, dev_tensor, device, say, to_np

pytestmark = pytest.mark.gpu


def _wl(B, M, Hq, Hkv, D, dtype="bf16", tau=1.0, seed=21):
    return wl.Workload("attn", seed, B=B, N=max(4 * M, 64), n_forced=0, d=0, d_ff=0, Ks=(M,), Hq=Hq, Hkv=Hkv, D=D,
                       tau=tau, dtype=dtype, rope=True, M_fixed=M)


def _run_fwd(w, M, rope=True, theta=wl.ROPE_THETA, g_override=None, grad=False, seed_offset=0, temp=False,
             gamma_override=None, overrides=None, lo=False):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    dev = device()
    a = wl.attn_inputs(w, M, with_grad=grad, seed_offset=seed_offset)
    if g_override is not None:
        a["g"] = g_override
    if gamma_override is not None:
        a["gamma"] = gamma_override
    a.update(overrides or {})
    q, k, v = (dev_tensor(a[n], w.dtype, dev) for n in ("q", "k", "v"))
    g = torch.from_numpy(a["g"]).to(dev)
    gamma = torch.from_numpy(a["gamma"]).to(dev)
    pos = torch.from_numpy(a["pos"]).to(dev) if rope else None
    sigma = torch.from_numpy(a["sigma"]).to(dev) if temp else None
    o = torch.full_like(q, float("nan"))
    lse = torch.full((w.B, w.Hq, M), float("nan"), device=dev)
    o_lo = torch.full_like(q, float("nan")) if lo else None
    ws = tg.attn_workspace(w.B, M, w.Hq, w.Hkv, w.D, True, dev)
    say("attn_fwd", w.dtype, w.B, M, w.Hq, w.Hkv, w.D, "rope" if rope else "no-rope", "temp" if temp else "",
        "o_lo" if lo else "")
    tg.tg_gated_attn_fwd(q, k, v, g, gamma, pos, theta, w.tau, o, lse, ws, sigma=sigma, o_lo=o_lo)
    torch.cuda.synchronize()
    out = dict(a=a, q=q, k=k, v=v, g=g, gamma=gamma, pos=pos, sigma=sigma, o=o, lse=lse, ws=ws, theta=theta,
               o_lo=o_lo)
    return out


def _oracle_fwd(w, r, rows=None, rope=True):
    a = r["a"]
    f = lambda x: wl.as_float(x, w.dtype)
    sig = None if r["sigma"] is None else a["sigma"]
    return oracle.attn_fwd(f(a["q"]), f(a["k"]), f(a["v"]), a["g"], a["gamma"], pos=a["pos"] if rope else None,
                           theta=r["theta"], tau=w.tau, round_bf16=(w.dtype == "bf16"), rows=rows, sigma=sig)


def _tol(w):
    return 2e-2 if w.dtype == "bf16" else 1e-4


def test_fwd_tiny_f32():
    w = wl.WORKLOADS["tiny_f32"]
    r = _run_fwd(w, 96, rope=False)
    o_ref, l_ref = _oracle_fwd(w, r, rope=False)
    assert_maxabs(to_np(r["o"]), o_ref, 1e-4, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 1e-4, "lse")


@pytest.mark.parametrize("B,M,Hq,Hkv,D,rope", [
    (1, 1, 2, 1, 128, True), (1, 63, 4, 4, 64, False), (2, 100, 4, 2, 128, True), (1, 257, 8, 2, 128, True),
    (2, 130, 16, 4, 64, True), (1, 200, 8, 1, 128, False), (1, 333, 16, 16, 128, True)])
def test_fwd_bf16_shapes(B, M, Hq, Hkv, D, rope):
    w = _wl(B, M, Hq, Hkv, D, tau=1.3)
    r = _run_fwd(w, M, rope=rope)
    o_ref, l_ref = _oracle_fwd(w, r, rope=rope)
    assert_maxabs(to_np(r["o"]), o_ref, 2e-2, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 2e-2, "lse")


def test_fwd_f32_rope_gqa():
    w = _wl(2, 70, 6, 2, 32, dtype="f32", tau=0.9)
    r = _run_fwd(w, 70, rope=True, theta=1e4)
    o_ref, l_ref = _oracle_fwd(w, r)
    assert_maxabs(to_np(r["o"]), o_ref, 1e-4, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 1e-4, "lse")


def test_fwd_zero_gate_rows():
    w = _wl(1, 150, 4, 2, 128)
    g = wl.attn_inputs(w, 150)["g"].copy()
    g[0, 0] = 0.0      # row 0 sees nothing: o = 0, lse = -inf
    g[0, 70:80] = 0.0  # masked keys inside the sequence
    r = _run_fwd(w, 150, g_override=g)
    o_ref, l_ref = _oracle_fwd(w, r)
    o = to_np(r["o"])
    assert np.all(o[0, 0] == 0.0) and np.all(np.isneginf(to_np(r["lse"])[0, :, 0]))
    assert_maxabs(o, o_ref, 2e-2, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 2e-2, "lse")


def test_fwd_split_row_with_a_dead_piece():
    # M = 1024 with 8 kv heads splits the rows of 16, 24 and 32 tiles (query blocks 3, 5, 7)
    # into 8-tile pieces; keys 0..255 (exactly their first piece) have g = 0 and every other key
    # a bias of 2 log2 2^-120 = -240, so the live logits lie far below 0.  A piece with no live
    # key must not set the merged reference (the softmax is shift invariant); the rows of keys
    # < 256 only (blocks 0, 1) are empty.  Blocks 2, 4, 6 split at 6 or 7 tiles, so one of their
    # pieces starts on a dead tile while later keys are live: that piece takes its reference from
    # its first live key.  Every row is checked.
    w = _wl(1, 1024, 16, 8, 128)
    g = np.full((1, 1024), 2.0 ** -120, np.float32)
    g[0, :256] = 0.0
    r = _run_fwd(w, 1024, g_override=g, gamma_override=np.full(16, 2.0, np.float32))
    o_ref, l_ref = _oracle_fwd(w, r)
    o, lse = to_np(r["o"]), to_np(r["lse"])
    assert np.all(o[0, :256] == 0.0) and np.all(np.isneginf(lse[0, :, :256]))
    assert np.all(np.isfinite(lse[0][:, 256:])) and np.all(lse[0][:, 256:] < -100.0)
    assert_maxabs(o, o_ref, 2e-2, "o")
    assert_maxabs(lse, l_ref, 2e-2, "lse")


def _far_logits(w, M, seed=5):
    """Gates in [0.5, 0.52] with a gain of 150 on every head: biases of 150 log2 g between -150 and
    -141.5 (log2 units), so every live logit lies far below zero while the weights stay spread over
    the keys; the gradients keep their usual size (dg = gain colsum / g).  Keys 0..31 get g = 0, so
    a piece's first tile holds no live key for any query."""
    rng = np.random.default_rng(seed)
    g = rng.uniform(0.5, 0.52, (w.B, M)).astype(np.float32)
    g[:, :32] = 0.0
    return dict(g=g, gamma=np.full(w.Hq, 150.0, np.float32))


@pytest.mark.parametrize("B,M,Hq,Hkv,temp", [(1, 200, 4, 2, False), (1, 200, 4, 2, True), (2, 333, 16, 8, True),
                                             (1, 1024, 16, 8, False)])
def test_fwd_bwd_dead_first_tile_far_logits(B, M, Hq, Hkv, temp):
    # unsplit rows (M = 200, 333) and split rows (M = 1024): the first tile of every row (and of
    # the first piece of a split row) is dead, the live logits lie about 204 (log2) below zero
    w = _wl(B, M, Hq, Hkv, 128)
    ov = _far_logits(w, M)
    r = _run_bwd(w, M, rope=False, temp=temp, overrides=ov)
    o_ref, l_ref = _oracle_fwd(w, r, rope=False)
    lse = to_np(r["lse"])
    assert np.all(np.isneginf(lse[:, :, :32])) and np.all(lse[:, :, 32:] < -20.0)
    assert_maxabs(to_np(r["o"]), o_ref, 2e-2, "o")
    assert_maxabs(lse, l_ref, 2e-2, "lse")
    _check_bwd(w, r, rope=False, dg_scale=ov["g"] / 150.0)


@pytest.mark.parametrize("name,K", [("qwen3_8k", 1024), ("qwen3_32k", 2048)])
def test_fwd_full_size(name, K):
    w = wl.WORKLOADS[name]
    M = w.M(K)
    r = _run_fwd(w, M)
    o_ref, l_ref = _oracle_fwd(w, r)
    assert_maxabs(to_np(r["o"]), o_ref, 2e-2, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 2e-2, "lse")


@pytest.mark.parametrize("K", [256, 1024, 4096, 16384])
def test_fwd_sweep_128k_sampled(K):
    w = wl.WORKLOADS["sweep_128k"]
    M = w.M(K)
    r = _run_fwd(w, M)
    rng = np.random.default_rng(K)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, M - 1], rng.choice(M, min(M, 48), replace=False)]))
    o_ref, l_ref = _oracle_fwd(w, r, rows=rows)
    assert_maxabs(to_np(r["o"])[0, rows], o_ref[0, rows], 2e-2, "o")
    assert_maxabs(to_np(r["lse"])[0][:, rows], l_ref[0][:, rows], 2e-2, "lse")


def test_fwd_deterministic():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = wl.WORKLOADS["qwen3_8k"]
    r = _run_fwd(w, 1088)
    o1 = r["o"].clone()
    tg.tg_gated_attn_fwd(r["q"], r["k"], r["v"], r["g"], r["gamma"], r["pos"], r["theta"], w.tau, r["o"], r["lse"],
                         r["ws"])
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), r["o"].view(torch.int16))


def _run_bwd(w, M, rope=True, theta=wl.ROPE_THETA, temp=False, g_override=None, overrides=None, use_o=False):
    """use_o: the forward also writes o_lo and the backward takes D_i from o + o_lo."""
    import torch
    import learned_token_pruning_gatescore_amd as tg

    r = _run_fwd(w, M, rope=rope, theta=theta, grad=True, temp=temp, g_override=g_override, overrides=overrides,
                 lo=use_o)
    dev = r["q"].device
    dout = dev_tensor(r["a"]["dout"], w.dtype, dev)
    dq = torch.full(r["q"].shape, float("nan"), device=dev)
    dk = torch.full(r["k"].shape, float("nan"), device=dev)
    dv = torch.full(r["v"].shape, float("nan"), device=dev)
    dg = torch.full(r["g"].shape, float("nan"), device=dev)
    dgam = torch.full(r["gamma"].shape, float("nan"), device=dev)
    dsig = torch.full(r["gamma"].shape, float("nan"), device=dev) if temp else None
    say("attn_bwd", w.dtype, w.B, M, w.Hq, w.Hkv, w.D, "temp" if temp else "", "D from o" if use_o else "")
    tg.tg_gated_attn_bwd(r["q"], r["k"], r["v"], r["g"], r["gamma"], r["pos"], theta, w.tau, r["lse"], dout, dq, dk,
                         dv, dg, dgam, r["ws"], sigma=r["sigma"], dsigma=dsig, o=r["o"] if use_o else None,
                         o_lo=r["o_lo"] if use_o else None)
    torch.cuda.synchronize()
    r.update(dout=dout, dq=dq, dk=dk, dv=dv, dg=dg, dgamma=dgam, dsigma=dsig)
    return r


def _check_bwd(w, r, rope=True, dg_scale=None):
    """Every gradient within the tolerance (max-abs); dg_scale (if given) multiplies both sides of dg
    first -- g / gain turns dg = gain colsum / g back into the column sums of dS, of size one, for
    inputs whose gain / g is large."""
    a = r["a"]
    f = lambda x: wl.as_float(x, w.dtype)
    temp = r["sigma"] is not None
    ref = oracle.attn_bwd(f(a["q"]), f(a["k"]), f(a["v"]), a["g"], a["gamma"], f(a["dout"]),
                          pos=a["pos"] if rope else None, theta=r["theta"], tau=w.tau, round_bf16=(w.dtype == "bf16"),
                          sigma=a["sigma"] if temp else None)
    tol = _tol(w)
    names = ("dq", "dk", "dv", "dg", "dgamma") + (("dsigma",) if temp else ())
    errs = {}
    for name, rf in zip(names, ref):
        got = to_np(r[name])
        if name == "dg" and dg_scale is not None:
            got, rf = got * dg_scale, rf * dg_scale
        errs[name] = assert_maxabs(got, rf, tol, name)
    return errs


def test_bwd_tiny_f32():
    w = wl.WORKLOADS["tiny_f32"]
    r = _run_bwd(w, 96, rope=False)
    _check_bwd(w, r, rope=False)


@pytest.mark.parametrize("B,M,Hq,Hkv,D,rope", [
    (1, 1, 2, 1, 128, True), (2, 100, 4, 2, 128, True), (1, 257, 8, 2, 128, False), (1, 190, 4, 4, 64, True),
    (1, 150, 8, 1, 128, True)])
def test_bwd_bf16_shapes(B, M, Hq, Hkv, D, rope):
    w = _wl(B, M, Hq, Hkv, D, tau=1.1)
    r = _run_bwd(w, M, rope=rope)
    _check_bwd(w, r, rope=rope)


def test_bwd_zero_gate_rows():
    w = _wl(1, 150, 4, 2, 128)
    g = wl.attn_inputs(w, 150)["g"].copy()
    g[0, 0] = 0.0
    g[0, 70:80] = 0.0
    r = _run_bwd(w, 150, g_override=g)
    _check_bwd(w, r)


def test_bwd_f32_rope_gqa():
    w = _wl(1, 80, 4, 2, 64, dtype="f32", tau=1.2)
    r = _run_bwd(w, 80, rope=True, theta=1e4)
    _check_bwd(w, r)


def test_bwd_train_b4_full():
    w = wl.WORKLOADS["train_b4"]
    r = _run_bwd(w, 2048)
    errs = _check_bwd(w, r)
    say("train_b4 bwd max-abs errors", errs)


# --- the row terms D_i from the forward's o and its rounding residual o_lo ---

def _bf16_ulp(x):
    """The spacing of bf16 numbers at |x| (x given as float32 values of bf16 numbers)."""
    e = np.floor(np.log2(np.maximum(np.abs(x), np.float32(2.0 ** -126))))
    return np.float32(2.0) ** (e - 7)


@pytest.mark.parametrize("B,M,Hq,Hkv,D,temp", [(2, 300, 16, 8, 128, False), (1, 1000, 16, 8, 128, True),
                                               (1, 190, 4, 4, 64, False)])
def test_fwd_o_lo_residual(B, M, Hq, Hkv, D, temp):
    """o and lse are unchanged by asking for o_lo; |o_lo| is at most half a bf16 step of o (it is the
    residual of o's rounding); o + o_lo (the fp32 output) matches the oracle at least as closely as
    o.  The 1000-token case splits its long rows into pieces merged at the end."""
    import torch

    w = _wl(B, M, Hq, Hkv, D, tau=1.1)
    r0 = _run_fwd(w, M, temp=temp)
    r = _run_fwd(w, M, temp=temp, lo=True)
    assert torch.equal(r0["o"].view(torch.int16), r["o"].view(torch.int16))
    assert torch.equal(r0["lse"], r["lse"])
    o, lo = to_np(r["o"]), to_np(r["o_lo"])
    assert np.all(np.isfinite(lo))
    assert np.all(np.abs(lo) <= 0.5 * _bf16_ulp(o))
    o_ref, _ = _oracle_fwd(w, r)
    e_o = assert_maxabs(o, o_ref, 2e-2, "o")
    e_lo = assert_maxabs(o + lo, o_ref, 2e-2, "o + o_lo")
    say("o_lo: max-abs error of o", e_o, "of o + o_lo", e_lo)
    assert e_lo <= e_o


@pytest.mark.parametrize("B,M,Hq,Hkv,D,rope,temp", [
    (1, 1, 2, 1, 128, True, False), (2, 100, 4, 2, 128, True, False), (1, 257, 8, 2, 128, False, True),
    (1, 190, 4, 4, 64, True, False), (2, 300, 16, 8, 128, True, True)])
def test_bwd_d_from_o_shapes(B, M, Hq, Hkv, D, rope, temp):
    w = _wl(B, M, Hq, Hkv, D, tau=1.1)
    r = _run_bwd(w, M, rope=rope, temp=temp, use_o=True)
    _check_bwd(w, r, rope=rope)


def test_bwd_d_from_o_zero_gate_rows():
    w = _wl(1, 150, 4, 2, 128)
    g = wl.attn_inputs(w, 150)["g"].copy()
    g[0, 0] = 0.0
    g[0, 70:80] = 0.0
    r = _run_bwd(w, 150, g_override=g, use_o=True)
    _check_bwd(w, r)


@pytest.mark.parametrize("temp", [False, True])
def test_bwd_d_from_o_train_b4_full(temp):
    w = wl.WORKLOADS["train_b4"]
    r = _run_bwd(w, 2048, temp=temp, use_o=True)
    errs = _check_bwd(w, r)
    say("train_b4 bwd (D from o) max-abs errors", errs)


@pytest.mark.parametrize("temp", [False, True])
def test_bwd_d_from_o_agrees_with_recomputed_d(temp):
    """Both forms take the exact D_i for dk, dv, dg, dgamma and dsigma, so these agree to fp32
    summation order (1e-4 of their largest value).  dq keeps D_o = dO . (o + o_lo), which differs
    from D_i by the forward's bf16 rounding of P (about 3e-3 in dq at these inputs, by an fp64
    model of that rounding); each form also rounds its own dS to bf16 for the products, so the two
    dq differ by up to about 1e-2, within the bf16 bound of either (both are checked against the
    oracle elsewhere)."""
    w = _wl(2, 300, 16, 8, 128, tau=1.1)
    r1 = _run_bwd(w, 300, temp=temp)
    r2 = _run_bwd(w, 300, temp=temp, use_o=True)
    names = ("dk", "dv", "dg", "dgamma") + (("dsigma",) if temp else ())
    for n in names:
        a, b = to_np(r1[n]), to_np(r2[n])
        assert_maxabs(b, a, 1e-4 * max(1.0, float(np.abs(a).max())), n)
    e = assert_maxabs(to_np(r2["dq"]), to_np(r1["dq"]), 2e-2, "dq")
    say("dq difference (D_o against the recomputed D)", e)


def test_bwd_d_from_o_deterministic():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = _wl(2, 300, 16, 8, 128)
    r = _run_bwd(w, 300, use_o=True)
    first = [t.clone() for t in (r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"])]
    tg.tg_gated_attn_bwd(r["q"], r["k"], r["v"], r["g"], r["gamma"], r["pos"], r["theta"], w.tau, r["lse"],
                         r["dout"], r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"], r["ws"], o=r["o"],
                         o_lo=r["o_lo"])
    torch.cuda.synchronize()
    for a, b in zip(first, (r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"])):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


def test_bwd_deterministic():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = _wl(2, 300, 16, 8, 128)
    r = _run_bwd(w, 300)
    first = [t.clone() for t in (r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"])]
    tg.tg_gated_attn_bwd(r["q"], r["k"], r["v"], r["g"], r["gamma"], r["pos"], r["theta"], w.tau, r["lse"],
                         r["dout"], r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"], r["ws"])
    torch.cuda.synchronize()
    for a, b in zip(first, (r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"])):
        assert torch.equal(a.view(torch.int32), b.view(torch.int32))


# --- pruning-ratio temperature (deep dive section 3.2, Eq. 7/8): sigma per head ---

@pytest.mark.parametrize("B,M,Hq,Hkv,D,rope", [
    (1, 1, 2, 1, 128, True), (1, 63, 4, 4, 64, False), (2, 100, 4, 2, 128, True), (1, 257, 8, 2, 128, True),
    (2, 130, 16, 4, 64, True), (1, 333, 16, 16, 128, False)])
def test_temp_fwd_bf16_shapes(B, M, Hq, Hkv, D, rope):
    w = _wl(B, M, Hq, Hkv, D, tau=1.3)
    r = _run_fwd(w, M, rope=rope, temp=True)
    o_ref, l_ref = _oracle_fwd(w, r, rope=rope)
    assert_maxabs(to_np(r["o"]), o_ref, 2e-2, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 2e-2, "lse")


@pytest.mark.parametrize("rope", [True, False])
def test_temp_fwd_f32(rope):
    w = _wl(2, 70, 6, 2, 32, dtype="f32", tau=0.9)
    r = _run_fwd(w, 70, rope=rope, theta=1e4, temp=True)
    o_ref, l_ref = _oracle_fwd(w, r, rope=rope)
    assert_maxabs(to_np(r["o"]), o_ref, 1e-4, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 1e-4, "lse")


def test_temp_fwd_zero_gate_rows():
    w = _wl(1, 150, 4, 2, 128)
    g = wl.attn_inputs(w, 150)["g"].copy()
    g[0, 0] = 0.0
    g[0, 70:80] = 0.0
    r = _run_fwd(w, 150, g_override=g, temp=True)
    o_ref, l_ref = _oracle_fwd(w, r)
    o = to_np(r["o"])
    assert np.all(o[0, 0] == 0.0) and np.all(np.isneginf(to_np(r["lse"])[0, :, 0]))
    assert_maxabs(o, o_ref, 2e-2, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 2e-2, "lse")


def test_temp_fwd_full_size():
    w = wl.WORKLOADS["qwen3_32k"]
    M = w.M(2048)
    r = _run_fwd(w, M, temp=True)
    o_ref, l_ref = _oracle_fwd(w, r)
    assert_maxabs(to_np(r["o"]), o_ref, 2e-2, "o")
    assert_maxabs(to_np(r["lse"]), l_ref, 2e-2, "lse")


def test_temp_fwd_sweep_128k_sampled():
    w = wl.WORKLOADS["sweep_128k"]
    M = w.M(16384)
    r = _run_fwd(w, M, temp=True)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([[0, 1, 63, 64, M - 1], rng.choice(M, 48, replace=False)]))
    o_ref, l_ref = _oracle_fwd(w, r, rows=rows)
    assert_maxabs(to_np(r["o"])[0, rows], o_ref[0, rows], 2e-2, "o")
    assert_maxabs(to_np(r["lse"])[0][:, rows], l_ref[0][:, rows], 2e-2, "lse")


@pytest.mark.parametrize("B,M,Hq,Hkv,D,rope", [
    (1, 1, 2, 1, 128, True), (2, 100, 4, 2, 128, True), (1, 257, 8, 2, 128, False), (1, 190, 4, 4, 64, True),
    (1, 150, 8, 1, 128, True)])
def test_temp_bwd_bf16_shapes(B, M, Hq, Hkv, D, rope):
    w = _wl(B, M, Hq, Hkv, D, tau=1.1)
    r = _run_bwd(w, M, rope=rope, temp=True)
    _check_bwd(w, r, rope=rope)


@pytest.mark.parametrize("rope", [True, False])
def test_temp_bwd_f32(rope):
    w = _wl(1, 80, 4, 2, 64, dtype="f32", tau=1.2)
    r = _run_bwd(w, 80, rope=rope, theta=1e4, temp=True)
    _check_bwd(w, r, rope=rope)


def test_temp_bwd_zero_gate_rows():
    w = _wl(1, 150, 4, 2, 128)
    g = wl.attn_inputs(w, 150)["g"].copy()
    g[0, 0] = 0.0
    g[0, 70:80] = 0.0
    r = _run_bwd(w, 150, temp=True, g_override=g)
    _check_bwd(w, r)


def test_temp_bwd_train_b4_full():
    w = wl.WORKLOADS["train_b4"]
    r = _run_bwd(w, 2048, temp=True)
    errs = _check_bwd(w, r)
    say("train_b4 temperature bwd max-abs errors", errs)


def test_temp_bwd_deterministic():
    import torch
    import learned_token_pruning_gatescore_amd as tg

    w = _wl(2, 300, 16, 8, 128)
    r = _run_bwd(w, 300, temp=True)
    names = ("dq", "dk", "dv", "dg", "dgamma", "dsigma")
    first = [r[n].clone() for n in names]
    tg.tg_gated_attn_bwd(r["q"], r["k"], r["v"], r["g"], r["gamma"], r["pos"], r["theta"], w.tau, r["lse"],
                         r["dout"], r["dq"], r["dk"], r["dv"], r["dg"], r["dgamma"], r["ws"], sigma=r["sigma"],
                         dsigma=r["dsigma"])
    torch.cuda.synchronize()
    for a, n in zip(first, names):
        assert torch.equal(a.view(torch.int32), r[n].view(torch.int32)), n


# --- packed variable-length sequences (both training budgets in one call) ---

def _varlen_case(lens, Hq, Hkv, D, dtype="bf16", seed=61, rope=True, temp=False, grad=False, use_o=False,
                 dout_scale=1.0):
    import torch
    import learned_token_pruning_gatescore_amd as tg

    rng = np.random.default_rng(seed)
    T_ = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    store = (lambda x: wl.bf16_bits(x)) if dtype == "bf16" else (lambda x: x.astype(np.float32))
    a = dict(q=store(rng.standard_normal((T_, Hq, D), dtype=np.float32)),
             k=store(rng.standard_normal((T_, Hkv, D), dtype=np.float32)),
             v=store(rng.standard_normal((T_, Hkv, D), dtype=np.float32)),
             dout=store(rng.standard_normal((T_, Hq, D), dtype=np.float32) * np.float32(dout_scale)),
             g=(1.0 / (1.0 + np.exp(-rng.standard_normal(T_)))).astype(np.float32),
             gamma=rng.uniform(0.5, 1.5, Hq).astype(np.float32),
             pos=np.concatenate([np.sort(rng.choice(max(4 * n, 64), n, replace=False)) for n in lens]).astype(np.int32),
             sigma=(0.54 + 0.5 * rng.standard_normal(Hq)).astype(np.float32))
    dev = device()
    q, k, v, dout = (dev_tensor(a[n], dtype, dev) for n in ("q", "k", "v", "dout"))
    g, gamma = torch.from_numpy(a["g"]).to(dev), torch.from_numpy(a["gamma"]).to(dev)
    pos = torch.from_numpy(a["pos"]).to(dev) if rope else None
    sigma = torch.from_numpy(a["sigma"]).to(dev) if temp else None
    o = torch.full_like(q, float("nan"))
    lse = torch.full((Hq * T_,), float("nan"), device=dev)
    ws = tg.attn_varlen_workspace(cu, Hq, Hkv, D, True, dev)
    say("attn_fwd_varlen", dtype, lens, Hq, Hkv, D, "rope" if rope else "", "temp" if temp else "")
    o_lo = torch.full_like(q, float("nan")) if use_o else None
    tg.tg_gated_attn_fwd_varlen(q, k, v, g, gamma, pos, wl.ROPE_THETA, 1.1, cu, o, lse, ws, sigma=sigma, o_lo=o_lo)
    torch.cuda.synchronize()
    f = lambda x: wl.as_float(x, dtype)
    o_ref, l_ref = oracle.attn_fwd_varlen(f(a["q"]), f(a["k"]), f(a["v"]), a["g"], a["gamma"], cu,
                                          pos=a["pos"] if rope else None, theta=wl.ROPE_THETA, tau=1.1,
                                          round_bf16=(dtype == "bf16"), sigma=a["sigma"] if temp else None)
    tol = 2e-2 if dtype == "bf16" else 1e-4
    assert_maxabs(to_np(o), o_ref, tol, "o")
    assert_maxabs(to_np(lse), l_ref, tol, "lse")
    if not grad:
        return
    dq = torch.full(q.shape, float("nan"), device=dev)
    dk = torch.full(k.shape, float("nan"), device=dev)
    dv = torch.full(v.shape, float("nan"), device=dev)
    dg = torch.full(g.shape, float("nan"), device=dev)
    dgam = torch.full(gamma.shape, float("nan"), device=dev)
    dsig = torch.full(gamma.shape, float("nan"), device=dev) if temp else None
    say("attn_bwd_varlen", dtype, lens)
    tg.tg_gated_attn_bwd_varlen(q, k, v, g, gamma, pos, wl.ROPE_THETA, 1.1, lse, dout, cu, dq, dk, dv, dg, dgam, ws,
                                sigma=sigma, dsigma=dsig, o=o if use_o else None, o_lo=o_lo)
    torch.cuda.synchronize()
    ref = oracle.attn_bwd_varlen(f(a["q"]), f(a["k"]), f(a["v"]), a["g"], a["gamma"], f(a["dout"]), cu,
                                 pos=a["pos"] if rope else None, theta=wl.ROPE_THETA, tau=1.1,
                                 round_bf16=(dtype == "bf16"), sigma=a["sigma"] if temp else None)
    got = (dq, dk, dv, dg, dgam) + ((dsig,) if temp else ())
    for name, gt, rf in zip(("dq", "dk", "dv", "dg", "dgamma", "dsigma"), got, ref):
        assert_maxabs(to_np(gt), rf, tol, name)


# two budgets packed by budget (two runs), interleaved lengths (one run per sequence),
# empty and one-token sequences, a single sequence
@pytest.mark.parametrize("lens,Hq,Hkv,D", [([300, 300, 150, 150], 8, 4, 128), ([130, 70, 130, 70], 4, 2, 128),
                                           ([0, 1, 257, 0, 257, 33], 8, 2, 64), ([517], 16, 8, 128)])
def test_varlen_bf16(lens, Hq, Hkv, D):
    _varlen_case(lens, Hq, Hkv, D, grad=True)


@pytest.mark.parametrize("temp,rope", [(True, True), (True, False), (False, False)])
def test_varlen_bf16_temperature_and_rope(temp, rope):
    _varlen_case([200, 200, 96], 8, 4, 128, temp=temp, rope=rope, grad=True, seed=62)


def test_varlen_f32():
    _varlen_case([40, 40, 17, 0, 9], 6, 2, 32, dtype="f32", temp=True, grad=True, seed=63)


def test_varlen_two_budgets_train_shape():
    """Batch 4 at two budgets packed by budget: 4 x 2048 then 4 x 1024 kept tokens (sampled checks are
    the full oracle here: 12288 tokens, 16 / 8 heads, D = 128)."""
    _varlen_case([2048] * 4 + [1024] * 4, 16, 8, 128, temp=True, grad=True, seed=64)


@pytest.mark.parametrize("use_o", [False, True])
def test_varlen_many_distinct_lengths(use_o):
    """20 sequences of distinct lengths (600 .. 1300 tokens): 20 runs, so the packed schedules take
    them in two groups of runs (16 + 4), each group one launch per kernel."""
    lens = [int(x) for x in np.random.default_rng(66).choice(np.arange(600, 1301), 20, replace=False)]
    _varlen_case(lens, 8, 4, 128, temp=True, grad=True, seed=66, use_o=use_o)


def test_varlen_backward_several_launches():
    """16 sequences of distinct lengths at 8 query heads per kv head (32-query blocks): the
    query-outer backward kernel's work-group table needs more than 256 ranges, so it runs as two
    launches.  dO is scaled by 1/4 (every gradient is linear in it) so that the gradients stay in the
    range the fixed max-abs bound was stated for (at 8 heads per kv head and rows of up to 933 keys
    |dv| would otherwise pass 15)."""
    lens = [379, 720, 927, 933, 947, 701, 520, 737, 847, 522, 460, 865, 904, 404, 385, 668]
    _varlen_case(lens, 16, 2, 64, temp=True, grad=True, seed=69, dout_scale=0.25)


def test_varlen_forward_g8_split_runs():
    """15 sequences of distinct lengths at 8 query heads per kv head (32-query blocks): one
    forward launch over 15 runs, split blocks in three of them.  Forward only: with dO unscaled,
    |dv| reaches 12.5 here (8 heads x up to 654 rows summed per key), where the backward's bf16
    rounding of P in dV = P^T dO alone is about 2e-2, the fixed max-abs bound of the training shapes
    (measured 2.08e-2, 1.7e-3 of |dv|); the backward at this head ratio is checked above."""
    lens = [281, 654, 122, 425, 574, 50, 213, 117, 83, 158, 343, 603, 218, 622, 47]
    _varlen_case(lens, 32, 4, 64, temp=True, seed=67)


def test_varlen_runs_over_groups_g1_no_rope():
    """40 sequences (4205 tokens) forming 32 runs, 8 of them of two equal-length sequences: two
    groups of 16 runs, with runs of n > 1 in both; one query head per kv head (256-query blocks),
    no positions, the temperature; forward and backward against the oracle."""
    lens = [149, 149, 84, 164, 89, 84, 84, 213, 188, 168, 137, 137, 102, 61, 143, 20, 20, 176, 75, 66, 98, 98,
            107, 88, 144, 54, 54, 29, 140, 67, 120, 120, 138, 163, 204, 53, 53, 24, 106, 36]
    _varlen_case(lens, 4, 4, 64, rope=False, temp=True, grad=True, seed=70)


def test_varlen_fwd_deterministic():
    """The packed forward twice on the same inputs (20 distinct lengths: two groups of runs, split
    blocks merged in the second group, the temperature, o_lo): o, o_lo and lse bitwise equal."""
    import torch
    import learned_token_pruning_gatescore_amd as tg

    lens = [int(x) for x in np.random.default_rng(66).choice(np.arange(600, 1301), 20, replace=False)]
    Hq, Hkv, D = 8, 4, 128
    rng = np.random.default_rng(68)
    T_ = int(sum(lens))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    dev = device()
    q, k, v = (dev_tensor(wl.bf16_bits(rng.standard_normal((T_, h, D), dtype=np.float32)), "bf16", dev)
               for h in (Hq, Hkv, Hkv))
    g = torch.from_numpy((1.0 / (1.0 + np.exp(-rng.standard_normal(T_)))).astype(np.float32)).to(dev)
    gamma = torch.from_numpy(rng.uniform(0.5, 1.5, Hq).astype(np.float32)).to(dev)
    pos = torch.from_numpy(np.concatenate([np.sort(rng.choice(4 * n, n, replace=False)) for n in lens])
                           .astype(np.int32)).to(dev)
    sigma = torch.from_numpy((0.54 + 0.5 * rng.standard_normal(Hq)).astype(np.float32)).to(dev)
    ws = tg.attn_varlen_workspace(cu, Hq, Hkv, D, False, dev)
    outs = []
    for _ in range(2):
        o, o_lo = torch.full_like(q, float("nan")), torch.full_like(q, float("nan"))
        lse = torch.full((Hq * T_,), float("nan"), device=dev)
        tg.tg_gated_attn_fwd_varlen(q, k, v, g, gamma, pos, wl.ROPE_THETA, 1.1, cu, o, lse, ws, sigma=sigma,
                                    o_lo=o_lo)
        torch.cuda.synchronize()
        outs.append((o, o_lo, lse))
    for a, b_ in zip(outs[0], outs[1]):
        assert torch.equal(a.view(torch.int16 if a.dtype == torch.bfloat16 else torch.int32),
                           b_.view(torch.int16 if b_.dtype == torch.bfloat16 else torch.int32))
    assert not torch.isnan(outs[0][2]).any()


@pytest.mark.parametrize("lens,temp", [([300, 300, 150, 150], False), ([0, 1, 257, 0, 257, 33], True),
                                       ([2048] * 4 + [1024] * 4, True)])
def test_varlen_d_from_o(lens, temp):
    """Packed sequences with the row terms from the forward's o + o_lo."""
    _varlen_case(lens, 16, 8, 128, temp=temp, grad=True, seed=65, use_o=True)
