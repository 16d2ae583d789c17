"""The pins catch plausible mistakes: each test plants one mistake in a copy
of an oracle function (on the CPU only) and checks that a pin fails."""
import math

import numpy as np
import pytest

import oracle as O
import oracle.sfi_oracle as OS
from tests import test_oracle_dense as TD
from tests import test_oracle_fast_sched as TF
from tests import test_oracle_select as TS


def _dense_variant(map_head, use_scale=True):
    def dense(q, K, V, scale=None):
        q = np.asarray(q, np.float64); K = np.asarray(K, np.float64); V = np.asarray(V, np.float64)
        Hq, D = q.shape
        Hkv, T, _ = K.shape
        sc = (1.0 / math.sqrt(D) if scale is None else scale) if use_scale else 1.0
        out = np.empty((Hq, D)); P = np.empty((Hq, T))
        for h in range(Hq):
            g = map_head(h, Hq, Hkv)
            s = (K[g] @ q[h]) * sc
            e = np.exp(s - s.max()); p = e / e.sum()
            P[h] = p; out[h] = p @ V[g]
        return out, P
    return dense


def _expect_failure(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_wrong_gqa_mapping_caught(monkeypatch, golden):
    monkeypatch.setattr(O, "dense_attention", _dense_variant(lambda h, Hq, Hkv: h % Hkv))
    _expect_failure(TD.test_gqa_mapping_is_contiguous_groups)
    _expect_failure(TD.test_dense_matches_library_sdpa, 8, 2, 37, 64, 0)


def test_missing_scale_caught(monkeypatch, golden):
    monkeypatch.setattr(O, "dense_attention", _dense_variant(lambda h, Hq, Hkv: h // (Hq // Hkv), False))
    _expect_failure(TD.test_dense_matches_library_sdpa, 8, 2, 37, 64, 0)
    _expect_failure(TD.test_dense_hand_examples, golden)


def test_wrong_tie_break_caught(monkeypatch):
    def topk(score, positions, k):
        m = min(k, len(positions))
        order = np.lexsort((-np.asarray(positions), -np.asarray(score, np.float64)))
        return np.sort(np.asarray(positions)[order[:m]])
    monkeypatch.setattr(O, "topk_select", topk)
    _expect_failure(TS.test_topk_equals_exhaustive_search_tie_heavy.hypothesis.inner_test, [1, 1, 1], 1, 0)


def test_prior_off_by_one_caught(monkeypatch, golden):
    def prior(n):
        a = np.arange(1, n + 1, dtype=np.float64)
        return (1.0 / a + 1.0 / np.maximum(n - a, 1)) / (2.0 * O.harmonic(n))
    monkeypatch.setattr(O, "positional_prior", prior)
    _expect_failure(TS.test_prior_hand_examples, golden)


def test_swapped_mixture_weights_caught(monkeypatch):
    monkeypatch.setattr(OS, "fused_score", lambda f, r, lam: lam * np.asarray(f) + (1 - lam) * np.asarray(r))
    monkeypatch.setattr(O, "fused_score", OS.fused_score)
    _expect_failure(TS.test_lambda_zero_is_topk_of_evidence)
    _expect_failure(TS.test_fused_score_is_the_mixture)


def test_recent_window_off_by_one_caught(monkeypatch):
    monkeypatch.setattr(O, "recent_positions",
                        lambda t, ns, w: np.arange(max(ns, t - w + 1), t, dtype=np.int64))
    _expect_failure(TS.test_parts_partition_the_context, 10, 2, 3)


def test_fast_step_with_dense_normaliser_caught(monkeypatch):
    def sparse(q, K, V, supports, scale=None):
        Hq, D = q.shape
        G = Hq // K.shape[0]
        out = np.empty((Hq, D))
        for h in range(Hq):
            g = h // G
            s = (K[g] @ q[h]) / math.sqrt(D)
            e = np.exp(s - s.max())
            S = np.asarray(supports[g])
            out[h] = (e[S] / e.sum()) @ V[g][S]     # normalised over all T, not the support
        return out
    monkeypatch.setattr(OS, "sparse_attention", sparse)
    _expect_failure(TF.test_fast_equals_library_sdpa_on_gathered_rows)


def test_splitmix_constant_typo_caught(monkeypatch):
    def bad(state):
        state = (state + 0x9E3779B97F4A7C15) & OS.MASK64
        z = state
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & OS.MASK64
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EA) & OS.MASK64
        return state, z ^ (z >> 31)
    monkeypatch.setattr(O, "splitmix64_next", bad)
    _expect_failure(TF.test_splitmix64_published_sequence)


def test_span_length_off_by_one_caught(monkeypatch):
    orig = OS.SpanSchedule._draw_span
    monkeypatch.setattr(OS.SpanSchedule, "_draw_span", lambda self: orig(self) + 1)
    _expect_failure(TF.test_fixed_spans_slow_positions)


# ------------------------------------------------------------------ optional Selector steps
from tests import test_oracle_discretize as TX  # noqa: E402


def test_nms_suppressed_by_lower_neighbours_caught(monkeypatch, golden):
    def nms(score, radius, decay):
        s = np.asarray(score, np.float64)
        n = len(s)
        if radius <= 0 or decay == 0 or n == 0:
            return s.copy()
        fac = np.ones(n)
        for d in range(1, radius + 1):
            f_d = 1.0 - decay * (1.0 - d / (radius + 1))
            below = np.zeros(n, bool); below[d:] = s[:-d] <= s[d:]
            above = np.zeros(n, bool); above[:-d] = s[d:] < s[:-d]
            fac = np.where(below | above, np.minimum(fac, f_d), fac)
        return s * fac
    monkeypatch.setattr(O, "soft_nms", nms)
    _expect_failure(TX.test_soft_nms_hand_examples, golden)


def test_nms_tie_rule_reversed_caught(monkeypatch, golden):
    def nms(score, radius, decay):
        s = np.asarray(score, np.float64)
        n = len(s)
        fac = np.ones(n)
        for d in range(1, radius + 1):
            f_d = 1.0 - decay * (1.0 - d / (radius + 1))
            below = np.zeros(n, bool); below[d:] = s[:-d] > s[d:]
            above = np.zeros(n, bool); above[:-d] = s[d:] >= s[:-d]
            fac = np.where(below | above, np.minimum(fac, f_d), fac)
        return s * fac
    monkeypatch.setattr(O, "soft_nms", nms)
    _expect_failure(TX.test_soft_nms_hand_examples, golden)


def test_exclusivity_share_of_the_maximum_caught(monkeypatch, golden):
    def excl(S, eps):
        S = np.asarray(S, np.float64)
        if eps == 0 or S.shape[0] <= 1:
            return S.copy()
        return S * (S / S.max(axis=0)) ** eps
    monkeypatch.setattr(O, "cross_head_exclusivity", excl)
    _expect_failure(TX.test_exclusivity_hand_example, golden)


def test_keynorm_on_raw_norms_caught(monkeypatch, golden):
    def prior(n, nu, beta, c):
        if beta == 0 or n == 0:
            return O.positional_prior(n)
        nu = np.asarray(nu, np.float64)
        a = np.arange(1, n + 1, dtype=np.float64)
        w = (1.0 / a + 1.0 / (n + 1 - a)) * np.exp(-beta * np.maximum(0.0, nu - nu.mean() - c))
        return w / w.sum()
    monkeypatch.setattr(O, "keynorm_prior", prior)
    _expect_failure(TX.test_keynorm_prior_hand_example, golden)
    _expect_failure(TX.test_keynorm_prior_invariants.hypothesis.inner_test, 10, 2.0, 0.5, 3)


def test_keynorm_without_renormalising_caught(monkeypatch, golden):
    def prior(n, nu, beta, c):
        if beta == 0 or n == 0:
            return O.positional_prior(n)
        nu = np.asarray(nu, np.float64)
        z = (nu - nu.mean()) / nu.std()
        return O.positional_prior(n) * np.exp(-beta * np.maximum(0.0, z - c))
    monkeypatch.setattr(O, "keynorm_prior", prior)
    _expect_failure(TX.test_keynorm_prior_hand_example, golden)
