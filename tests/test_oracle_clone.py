"""Pins of the oracle's clone scorer (CPU only).

DeepDive = "TokenGate: Learnable Token Pruning for Fast, Memory-Efficient LLM Prefill",
section 3.4 (a scoring branch cloned from the gate layer's MLP) and the section 3 pipeline
figure ("MLP clone of gate-layer MLP").  The pages give no shape for it; the reading pinned
here is the gated (SwiGLU) MLP followed by a head projection:
b~^h = P[h] . (Wd (SiLU(Wg a) * (Wu a))).  What the pins fix:
  * a hand-worked example (d = 3, d_i = 2, H = 2, two tokens) whose values follow from
    sigmoid(ln 3) = 3/4: a gate/up swap, a transposed Wd or P, or a token mix-up changes it;
  * P = 0 (the head projection's zero start) gives zero scores for any input;
  * a joint permutation of the d_i units (rows of Wg and Wu, columns of Wd) changes nothing,
    an unmatched one (Wu's rows only) does;
  * the scores are linear in P and in Wu and in Wd;
  * with a constant input channel routed to Wu (up = 1) and Wd an embedding, the clone reduces
    to the per-head scorer w2[h] . SiLU(W1 a), which its own pins tie to the single-head scorer.
"""
import math

import numpy as np
import pytest

import oracle


@pytest.fixture(scope="module")
def o():
    oracle.build(force=False)
    return oracle


def _rand(seed, T, d, d_i, H):
    rng = np.random.default_rng(seed)
    h = rng.normal(0.0, 1.0, (T, d))
    wg = rng.normal(0.0, 1.0 / math.sqrt(d), (d_i, d))
    wu = rng.normal(0.0, 1.0 / math.sqrt(d), (d_i, d))
    wd = rng.normal(0.0, 1.0 / math.sqrt(d_i), (d, d_i))
    wh = rng.normal(0.0, 1.0 / math.sqrt(d), (H, d))
    return h, wg, wu, wd, wh


def test_clone_hand_worked_example(o):
    L = math.log(3.0)  # sigmoid(L) = 3/4, sigmoid(-L) = 1/4
    h = np.array([[L, 1.0, 0.0], [-L, -1.0, 0.0]])
    wg = np.array([[1.0, 0.0, 0.0], [-1.0, 0.0, 5.0]])  # gate: (L, -L) and (-L, L)
    wu = np.array([[0.0, 2.0, 0.0], [0.0, -1.0, 1.0]])  # up: (2, -1) and (-2, 1)
    wd = np.array([[1.0, 0.0], [0.0, 1.0], [2.0, -4.0]])  # [d = 3, d_i = 2]
    wh = np.array([[1.0, 1.0, 1.0], [0.0, 0.0, 1.0]])  # [H = 2, d = 3]
    # token 0: m = (SiLU(L) * 2, SiLU(-L) * -1) = (1.5 L, 0.25 L); y = (1.5 L, 0.25 L, 2 L)
    # token 1: m = (SiLU(-L) * -2, SiLU(L) * 1) = (0.5 L, 0.75 L); y = (0.5 L, 0.75 L, -2 L)
    want = np.array([[3.75 * L, -0.75 * L], [2.0 * L, -2.0 * L]])
    got = o.gate_score_clone(h, wg, wu, wd, wh)
    assert got.shape == (2, 2)
    np.testing.assert_allclose(got, want, rtol=1e-14, atol=1e-15)


def test_clone_zero_head_projection_scores_zero(o):
    h, wg, wu, wd, _ = _rand(1, 17, 24, 40, 3)
    got = o.gate_score_clone(h * 50.0, wg, wu, wd, np.zeros((3, 24)))
    assert np.all(got == 0.0)


def test_clone_unit_permutation(o):
    h, wg, wu, wd, wh = _rand(2, 13, 20, 36, 4)
    ref = o.gate_score_clone(h, wg, wu, wd, wh)
    perm = np.random.default_rng(3).permutation(36)
    np.testing.assert_allclose(o.gate_score_clone(h, wg[perm], wu[perm], wd[:, perm], wh), ref, rtol=1e-12,
                               atol=1e-13)
    # permuting only the up rows breaks the gate/up pairing
    bad = o.gate_score_clone(h, wg, wu[perm], wd, wh)
    assert np.max(np.abs(bad - ref)) > 1e-3 * np.max(np.abs(ref))


def test_clone_linear_in_head_up_and_down(o):
    h, wg, wu, wd, wh = _rand(4, 11, 16, 28, 2)
    ref = o.gate_score_clone(h, wg, wu, wd, wh)
    cases = [(3.0, (wg, 3.0 * wu, wd, wh)), (-2.5, (wg, wu, -2.5 * wd, wh)), (0.5, (wg, wu, wd, 0.5 * wh))]
    for scale, args in cases:
        np.testing.assert_allclose(o.gate_score_clone(h, *args), scale * ref, rtol=1e-12, atol=1e-13)
    # two head projections add
    wh2 = np.random.default_rng(5).normal(0.0, 1.0, wh.shape)
    np.testing.assert_allclose(o.gate_score_clone(h, wg, wu, wd, wh + wh2),
                               ref + o.gate_score_clone(h, wg, wu, wd, wh2), rtol=1e-11, atol=1e-12)


def test_clone_reduces_to_per_head_scorer(o):
    T, d, d_i, H = 9, 12, 8, 3
    rng = np.random.default_rng(6)
    h = rng.normal(0.0, 1.0, (T, d))
    h[:, -1] = 1.0  # a constant channel
    wg = rng.normal(0.0, 0.5, (d_i, d))
    wg[:, -1] = 0.0
    wu = np.zeros((d_i, d))
    wu[:, -1] = 1.0  # up_k = 1 for every unit
    wd = np.zeros((d, d_i))
    wd[:d_i, :] = np.eye(d_i)  # y = (m, 0, ...)
    w2 = rng.normal(0.0, 1.0, (H, d_i))
    wh = np.zeros((H, d))
    wh[:, :d_i] = w2
    np.testing.assert_allclose(o.gate_score_clone(h, wg, wu, wd, wh), o.gate_score_heads(h, wg, w2), rtol=1e-13,
                               atol=1e-14)


def test_clone_one_head_vector_and_shape_errors(o):
    h, wg, wu, wd, wh = _rand(7, 5, 8, 6, 1)
    np.testing.assert_array_equal(o.gate_score_clone(h, wg, wu, wd, wh[0]), o.gate_score_clone(h, wg, wu, wd, wh))
    with pytest.raises(ValueError):
        o.gate_score_clone(h, wg, wu, wd.T, wh)
