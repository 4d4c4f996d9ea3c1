"""Pins of the oracle's scoring MLP and gate value (CPU only).

TokenGate deep dive, section 3.1 Eq. 3 (first part): a small MLP maps each
token's normalised residual to a scalar score.  Reading: d -> d_ff -> 1 with
SiLU and no biases; gate g = sigmoid(s); a forced token's gate is 1 (its score
enters attention as zero bias).
"""
import math

import numpy as np


def test_score_matches_numpy_matmul(oracle_mod):
    rng = np.random.default_rng(0)
    T, d, d_ff = 37, 48, 20
    h = rng.standard_normal((T, d))
    W1 = rng.standard_normal((d_ff, d)) / math.sqrt(d)
    w2 = rng.standard_normal(d_ff) / math.sqrt(d_ff)
    forced = (rng.random(T) < 0.3).astype(np.uint8)
    s, g = oracle_mod.gate_score(h, W1, w2, forced)
    u = h @ W1.T                                  # library matmul
    ref = (u * (1.0 / (1.0 + np.exp(-u)))) @ w2   # SiLU(u) = u * sigmoid(u)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-13)
    gref = np.where(forced != 0, 1.0, 1.0 / (1.0 + np.exp(-ref)))
    np.testing.assert_allclose(g, gref, rtol=1e-12, atol=0)
    assert np.all(g[forced != 0] == 1.0)


def test_score_unit_w2_picks_one_unit(oracle_mod):
    rng = np.random.default_rng(1)
    T, d, d_ff = 9, 16, 8
    h = rng.standard_normal((T, d))
    W1 = rng.standard_normal((d_ff, d))
    for k in (0, 5, 7):
        w2 = np.zeros(d_ff)
        w2[k] = 1.0
        s, _ = oracle_mod.gate_score(h, W1, w2)
        u = np.array([np.dot(W1[k], h[t]) for t in range(T)])
        np.testing.assert_allclose(s, u / (1.0 + np.exp(-u)), rtol=1e-13)


def test_score_closed_forms(oracle_mod):
    # W1 = 0: every score is 0 and every prunable gate is exactly 1/2
    s, g = oracle_mod.gate_score(np.ones((4, 3)), np.zeros((2, 3)), np.ones(2), np.array([0, 1, 0, 0], np.uint8))
    assert np.all(s == 0.0)
    np.testing.assert_array_equal(g, [0.5, 1.0, 0.5, 0.5])
    # one unit with u = 1: s = SiLU(1) = e / (1 + e); g = 1 / (1 + exp(-s))
    s, g = oracle_mod.gate_score(np.ones((1, 1)), np.ones((1, 1)), np.ones(1))
    e = math.e
    assert abs(s[0] - e / (1 + e)) < 1e-15
    assert abs(g[0] - 1 / (1 + math.exp(-e / (1 + e)))) < 1e-15
    # a zero-initialised output layer (w2 = 0): all scores 0, no preferred position
    rng = np.random.default_rng(2)
    s, _ = oracle_mod.gate_score(rng.standard_normal((5, 6)), rng.standard_normal((4, 6)), np.zeros(4))
    assert np.all(s == 0.0)


def test_bf16_rounding_helper(oracle_mod):
    r = oracle_mod.round_bf16
    assert r(1.0) == 1.0
    assert r(1.0 + 2**-8) == 1.0                    # tie -> even (1.0)
    assert r(1.0 + 3 * 2**-8) == 1.0 + 2**-6        # tie -> even (1 + 4*2^-8)
    assert r(1.0 + 2**-8 + 2**-30) == 1.0 + 2**-7   # above the tie -> up
    assert r(-1.0 - 2**-8 - 2**-30) == -(1.0 + 2**-7)
    assert r(0.0) == 0.0 and math.isinf(r(float("inf")))
    # against an arithmetic rounding: frexp mantissa scaled to 8 significant bits, numpy's
    # round-half-to-even, scaled back
    rng = np.random.default_rng(5)
    xs = rng.standard_normal(2000) * np.exp(rng.uniform(-20, 20, 2000))
    xs = np.concatenate([xs, (rng.integers(-2**12, 2**12, 500) + 0.5) / 2**4])  # exact ties
    for x in xs:
        m, e = np.frexp(x)
        ref = np.ldexp(np.round(m * 256.0) / 256.0, e)
        assert r(float(x)) == ref, x
