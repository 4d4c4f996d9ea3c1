"""Pins of the oracle's selection and compaction (CPU only).

Selection follows the TokenGate deep dive, section 3.1 Eq. 4 (top-K over the
prunable set, united with the non-prunable set) and section 3.4 (budget clamp,
keep mask in original order).  The oracle is checked against a brute-force
rank count written independently here, against closed forms, and against
invariants over tie-heavy random inputs.
"""
import math

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st


def _beats(a, ia, b, ib):
    """True when (score a, index ia) ranks above (b, ib): non-NaN above NaN, larger score
    above smaller (IEEE compare, so -0 == +0), then lower index."""
    an, bn = math.isnan(a), math.isnan(b)
    if an != bn:
        return bn
    if not an and a != b:
        return a > b
    return ia < ib


def _brute(scores, forced, K):
    """keep n <=> forced, or fewer than K' prunable tokens rank above it."""
    N = len(scores)
    P = [n for n in range(N) if not forced[n]]
    Kc = min(K, len(P))
    keep = []
    for n in range(N):
        if forced[n]:
            keep.append(n)
            continue
        above = sum(1 for m in P if m != n and _beats(float(scores[m]), m, float(scores[n]), n))
        if above < Kc:
            keep.append(n)
    return np.array(keep, np.int32)


SPECIALS = [0.0, -0.0, 1.0, -1.0, 0.5, float("inf"), float("-inf"), float("nan"), 2.0, 1.0]


@pytest.mark.parametrize("seed", range(12))
def test_select_matches_brute_force(oracle_mod, seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 200))
    # tie-heavy: values drawn from a small pool, plus specials
    pool = np.concatenate([rng.integers(-3, 4, 8).astype(np.float32), np.array(SPECIALS, np.float32)])
    scores = pool[rng.integers(0, len(pool), N)].astype(np.float32)
    forced = (rng.random(N) < 0.2).astype(np.uint8)
    K = int(rng.integers(0, N + 3))
    kept, cnt = oracle_mod.select_topk(scores, forced, K)
    ref = _brute(scores, forced, K)
    assert cnt == len(ref)
    np.testing.assert_array_equal(kept, ref)


def test_select_closed_forms(oracle_mod):
    N, nF = 100, 10
    forced = np.zeros(N, np.uint8)
    forced[:nF] = 1
    doc = np.arange(nF, N)
    # all scores equal (e.g. a zero-initialised scorer: every score is 0) -> first K' documents
    kept, _ = oracle_mod.select_topk(np.zeros(N, np.float32), forced, 7)
    np.testing.assert_array_equal(kept, np.concatenate([np.arange(nF), doc[:7]]))
    # strictly decreasing -> first K'
    kept, _ = oracle_mod.select_topk(np.arange(N, 0, -1).astype(np.float32), forced, 5)
    np.testing.assert_array_equal(kept, np.concatenate([np.arange(nF), doc[:5]]))
    # strictly increasing -> last K'
    kept, _ = oracle_mod.select_topk(np.arange(N).astype(np.float32), forced, 5)
    np.testing.assert_array_equal(kept, np.concatenate([np.arange(nF), doc[-5:]]))
    # K >= |P| -> everything; K = 0 -> the scaffold only
    kept, cnt = oracle_mod.select_topk(np.random.default_rng(0).random(N).astype(np.float32), forced, 10**6)
    np.testing.assert_array_equal(kept, np.arange(N))
    assert cnt == N
    kept, cnt = oracle_mod.select_topk(np.ones(N, np.float32), forced, 0)
    np.testing.assert_array_equal(kept, np.arange(nF))
    assert cnt == nF


def test_select_nan_inf_signed_zero(oracle_mod):
    s = np.array([np.nan, -0.0, 0.0, -np.inf, np.inf, np.nan, 1.0], np.float32)
    f = np.zeros(7, np.uint8)
    # ranking: +inf(4) > 1(6) > -0(1) == +0(2) [index order] > -inf(3) > NaN(0) > NaN(5)
    order = [4, 6, 1, 2, 3, 0, 5]
    for K in range(8):
        kept, _ = oracle_mod.select_topk(s, f, K)
        np.testing.assert_array_equal(kept, np.sort(np.array(order[:K], np.int32)))


def test_select_forced_count_mismatch_pads(oracle_mod):
    N = 20
    forced = np.zeros(N, np.uint8)
    forced[[3, 7, 11]] = 1
    s = np.arange(N, dtype=np.float32)
    # caller allocates for 5 forced + 4 documents = 9 but only 3 are forced: true M = 7
    kept, cnt = oracle_mod.select_topk(s, forced, 4, M=9)
    assert cnt == 7
    np.testing.assert_array_equal(kept, np.array([3, 7, 11, 16, 17, 18, 19, -1, -1], np.int32))
    # more forced than allocated: truncated, true count reported
    kept, cnt = oracle_mod.select_topk(s, forced, 4, M=5)
    assert cnt == 7
    np.testing.assert_array_equal(kept, np.array([3, 7, 11, 16, 17], np.int32))


@settings(max_examples=150, deadline=None)
@given(
    vals=st.lists(st.sampled_from([0.0, -0.0, 1.0, 0.25, -2.0, 3.5, float("inf"), float("-inf"), float("nan")]),
                  min_size=1, max_size=120),
    fmask=st.lists(st.booleans(), min_size=120, max_size=120),
    K=st.integers(min_value=0, max_value=130),
)
def test_select_invariants(oracle_mod, vals, fmask, K):
    s = np.array(vals, np.float32)
    N = len(s)
    forced = np.array(fmask[:N], np.uint8)
    kept, cnt = oracle_mod.select_topk(s, forced, K)
    nF = int(forced.sum())
    Kc = min(K, N - nF)
    assert cnt == nF + Kc == len(kept)
    assert np.all(np.diff(kept) > 0)                    # strictly ascending (original order kept)
    assert set(np.flatnonzero(forced)) <= set(kept)     # every scaffold token survives
    doc_kept = [n for n in kept if not forced[n]]
    assert len(doc_kept) == Kc                          # exactly K' documents
    dropped = [n for n in range(N) if not forced[n] and n not in set(kept)]
    for a in doc_kept:                                  # every kept document ranks above every dropped one
        for b in dropped:
            assert _beats(float(s[a]), a, float(s[b]), b)


def test_compact_matches_fancy_indexing(oracle_mod):
    rng = np.random.default_rng(3)
    B, N, d, M = 2, 50, 24, 17
    hidden = rng.integers(0, 2**16, (B, N, d), dtype=np.uint16)
    pos = rng.integers(0, 10**6, (B, N)).astype(np.int32)
    gates = rng.random((B, N)).astype(np.float32)
    kept = np.stack([np.sort(rng.choice(N, M, replace=False)) for _ in range(B)]).astype(np.int32)
    ho, po, go = oracle_mod.compact(hidden, pos, gates, kept)
    for b in range(B):
        np.testing.assert_array_equal(ho[b], hidden[b][kept[b]])
        np.testing.assert_array_equal(po[b], pos[b][kept[b]])
        np.testing.assert_array_equal(go[b].view(np.uint32), gates[b][kept[b]].view(np.uint32))
    # pos=None means position = original index
    _, po, _ = oracle_mod.compact(hidden, None, gates, kept)
    np.testing.assert_array_equal(po, kept)
    # padding rows (-1) give zero rows, position -1, gate 0
    kp = kept.copy()
    kp[:, -3:] = -1
    ho, po, go = oracle_mod.compact(hidden, pos, gates, kp)
    assert np.all(ho[:, -3:] == 0) and np.all(po[:, -3:] == -1) and np.all(go[:, -3:] == 0)
