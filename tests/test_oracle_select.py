"""Pins for the oracle's Selector: sparse-state parts (O3), prior (O4),
fusion (O5) and top-k (O6).

Pins: hand-worked examples, the prior's closed-form normaliser and symmetry,
an exhaustive search over all subsets on tiny inputs (with tie-heavy integer
scores from hypothesis), the lambda = 0 and lambda = 1 closed forms, and the
set invariants of the support.
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle as O


# ----------------------------------------------------------------- prior (O4)
def test_prior_hand_examples(golden):
    for key in ("prior_n4", "prior_n1"):
        ex = golden[key]
        r = O.positional_prior(ex["n"])
        assert np.max(np.abs(r - np.array(ex["r"]))) < 1e-15


@pytest.mark.parametrize("n", [1, 2, 3, 10, 255, 1980, 32496, 130800])
def test_prior_normalised_symmetric_monotone(n):
    r = O.positional_prior(n)
    assert abs(r.sum() - 1.0) < 1e-12
    assert np.array_equal(r, r[::-1])                       # r(a) == r(n+1-a) bitwise
    half = r[: (n + 1) // 2]
    assert np.all(np.diff(half) < 0) or n <= 2              # strictly decreasing to the middle


def test_harmonic_exact_small():
    for n in range(1, 30):
        exact = sum(Fraction(1, i) for i in range(1, n + 1))
        assert abs(O.harmonic(n) - float(exact)) <= 1e-15 * float(exact)


# ------------------------------------------------------ sparse-state parts (O3)
@pytest.mark.parametrize("t,ns,w", [(10, 2, 3), (5, 2, 3), (4, 4, 64), (2, 4, 64), (2048, 4, 64),
                                    (0, 4, 4), (100, 0, 0), (100, 0, 10), (100, 10, 0), (7, 3, 4)])
def test_parts_partition_the_context(t, ns, w):
    s = O.sink_positions(t, ns)
    r = O.recent_positions(t, ns, w)
    c = O.candidate_positions(t, ns, w)
    allpos = np.concatenate([s, c, r])
    assert sorted(allpos.tolist()) == list(range(t))        # disjoint cover of [0, t)
    assert len(s) == min(ns, t)
    assert len(c) == max(0, t - ns - w)


# -------------------------------------------------------------- top-k (O6)
def _brute_force_topk(score, positions, k):
    """Exhaustive search: the unique subset of size min(k, n) in which every
    chosen element precedes every unchosen one under (score desc, pos asc)."""
    n = len(positions)
    m = min(k, n)
    winners = []
    for comb in itertools.combinations(range(n), m):
        chosen = set(comb)
        ok = True
        for i in chosen:
            for j in range(n):
                if j in chosen:
                    continue
                better = score[i] > score[j] or (score[i] == score[j] and positions[i] < positions[j])
                if not better:
                    ok = False
                    break
            if not ok:
                break
        if ok:
            winners.append(sorted(positions[i] for i in comb))
    assert len(winners) == 1
    return winners[0]


@settings(max_examples=150, deadline=None)
@given(st.lists(st.integers(min_value=0, max_value=3), min_size=0, max_size=9),
       st.integers(min_value=0, max_value=10), st.integers(min_value=0, max_value=5))
def test_topk_equals_exhaustive_search_tie_heavy(vals, k, offset):
    score = np.array(vals, dtype=np.float64)
    positions = np.arange(offset, offset + len(vals), dtype=np.int64)
    got = O.topk_select(score, positions, k).tolist()
    assert got == _brute_force_topk(vals, positions.tolist(), k)


def test_select_hand_example(golden):
    ex = golden["select_small"]
    f = np.array(ex["f_full"])
    for k, key in ((3, "top3"), (1, "top1")):
        sel, _, _ = O.select(f, ex["T"], ex["n_sink"], ex["n_recent"], k, ex["lambda"])
        assert sel.tolist() == ex[key]


def test_lambda_zero_is_topk_of_evidence():
    rng = np.random.default_rng(3)
    T, ns, w, k = 500, 4, 16, 37
    f = rng.random(T); f /= f.sum()
    sel, _, cand = O.select(f, T, ns, w, k, 0.0)
    # an independent ranking with Python's sort on (−f, j) tuples
    ranked = sorted(cand.tolist(), key=lambda j: (-f[j], j))[:k]
    assert sel.tolist() == sorted(ranked)


@pytest.mark.parametrize("n,k", [(1980, 255), (1980, 256), (101, 10), (101, 11), (7, 3)])
def test_lambda_one_closed_form(n, k):
    """With lambda = 1 only the prior counts: the top-k are the ceil(k/2)
    candidates next to the sinks and the floor(k/2) next to the recent
    window (the tie at an odd k goes to the lower position)."""
    ns, w = 4, 64
    T = n + ns + w
    rng = np.random.default_rng(n + k)
    f = rng.random(T); f /= f.sum()
    sel, _, _ = O.select(f, T, ns, w, k, 1.0)
    a = sel - ns + 1
    expect = list(range(1, math.ceil(k / 2) + 1)) + list(range(n - k // 2 + 1, n + 1))
    assert a.tolist() == expect


def test_uniform_evidence_reduces_to_prior():
    """Uniform evidence (a zero query) with any lambda > 0 ranks like the prior."""
    T, ns, w, k = 300, 4, 20, 33
    f = np.full(T, 1.0 / T)
    a = O.select(f, T, ns, w, k, 0.1)[0]
    b = O.select(f, T, ns, w, k, 1.0)[0]
    assert a.tolist() == b.tolist()


def test_fused_score_is_the_mixture():
    f = np.array([0.5, 0.25, 0.25]); r = np.array([0.2, 0.3, 0.5])
    assert np.allclose(O.fused_score(f, r, 0.25), [0.425, 0.2625, 0.3125], atol=1e-16, rtol=0)
    assert abs(O.fused_score(f, r, 0.3).sum() - 1.0) < 1e-15


@pytest.mark.parametrize("T,ns,w,k", [(50, 4, 8, 100), (12, 4, 8, 3), (10, 4, 8, 3), (3, 4, 8, 3)])
def test_small_contexts(T, ns, w, k):
    f = np.full(T, 1.0 / T)
    sel, _, cand = O.select(f, T, ns, w, k, 0.1)
    n = max(0, T - ns - w)
    assert len(cand) == n and len(sel) == min(k, n)
    if n <= k:
        assert sel.tolist() == cand.tolist()


# ------------------------------------------------------------ support (O7 set)
@settings(max_examples=100, deadline=None)
@given(st.integers(1, 300), st.integers(0, 20), st.integers(0, 40), st.integers(0, 60), st.integers(0, 10 ** 6))
def test_support_invariants(T, ns, w, k, seed):
    rng = np.random.default_rng(seed)
    f = rng.random(T); f /= f.sum()
    sel, _, cand = O.select(f, T, ns, w, k, 0.1)
    S = O.support(T, ns, w, sel)
    n = len(cand)
    assert len(S) == min(T, ns + w) + min(k, n)
    assert len(set(S.tolist())) == len(S)                    # no duplicates
    assert np.all(np.diff(S) > 0) and (len(S) == 0 or (S[0] >= 0 and S[-1] < T))
    assert set(range(min(ns, T))) <= set(S.tolist())         # sinks always kept
    assert set(range(max(ns, T - w), T)) <= set(S.tolist())  # recent window always kept
    assert not (set(sel.tolist()) & set(O.sink_positions(T, ns).tolist()))
    assert not (set(sel.tolist()) & set(O.recent_positions(T, ns, w).tolist()))
