"""Pins of the oracle's optional Selector steps (gist.science technical
summary, 2.B): the key-norm correction of the prior, the Soft-NMS round
within a head and the exclusivity across heads.  The pages give no formula
for any of them; each is pinned by hand-worked examples of its stated
reading and by invariants that a plausible mistake would break."""
import math

import numpy as np
from hypothesis import given, settings
from hypothesis import strategies as st

import oracle as O


# ------------------------------------------------------------------ key-norm prior
def test_keynorm_prior_hand_example(golden):
    e = golden["keynorm_prior_n4"]
    r = O.keynorm_prior(4, e["nu"], e["beta"], e["c"])
    assert np.allclose(r, e["r"], rtol=0, atol=1e-12)


def test_keynorm_prior_off_is_the_positional_prior():
    nu = np.random.default_rng(0).gamma(2.0, 3.0, 97)
    for n in (1, 2, 5, 97):
        assert np.array_equal(O.keynorm_prior(n, nu[:n], 0.0, 1.0), O.positional_prior(n))


@given(st.integers(2, 60), st.floats(0.1, 5.0), st.floats(0.0, 3.0), st.integers(0, 2 ** 31))
@settings(max_examples=60, deadline=None)
def test_keynorm_prior_invariants(n, beta, c, seed):
    rng = np.random.default_rng(seed)
    nu = rng.gamma(2.0, 2.0, n) + 0.1
    r = O.keynorm_prior(n, nu, beta, c)
    assert abs(r.sum() - 1.0) < 1e-12 and np.all(r > 0)
    # z is scale and shift free: the prior depends on the norms' pattern only
    assert np.allclose(O.keynorm_prior(n, 7.0 * nu + 3.0, beta, c), r, rtol=1e-10, atol=0)
    # relative to the positional shape, candidates at or below c standard
    # deviations keep equal weight; above it the weight falls with the norm
    base = O.positional_prior(n)
    ratio = r / base
    z = (nu - nu.mean()) / nu.std()
    low = z <= c
    if low.sum() >= 2:
        assert np.allclose(ratio[low], ratio[low][0], rtol=1e-10, atol=0)
    order = np.argsort(z)
    assert np.all(np.diff(ratio[order]) <= 1e-12 * ratio.max())


def test_keynorm_prior_equal_norms():
    n = 50
    r = O.keynorm_prior(n, np.full(n, 3.0), 2.0, 0.5)
    assert np.allclose(r, O.positional_prior(n), rtol=1e-14, atol=0)


def test_key_norms():
    K = np.array([[3.0, 4.0], [0.0, 0.0], [1.0, -1.0]])
    assert np.allclose(O.key_norms(K), [5.0, 0.0, math.sqrt(2.0)], rtol=0, atol=1e-15)


# ------------------------------------------------------------------ Soft-NMS
def test_soft_nms_hand_examples(golden):
    for key in ("soft_nms_radius1", "soft_nms_radius2"):
        e = golden[key]
        out = O.soft_nms(e["score"], e["radius"], e["decay"])
        assert np.allclose(out, e["out"], rtol=0, atol=1e-12), key


@given(st.lists(st.integers(0, 6), min_size=1, max_size=40), st.integers(0, 5), st.floats(0.0, 1.0))
@settings(max_examples=150, deadline=None)
def test_soft_nms_invariants(vals, radius, decay):
    s = np.asarray(vals, np.float64)
    out = O.soft_nms(s, radius, decay)
    assert np.all(out <= s) and np.all(out >= (1.0 - decay) * s - 1e-15)
    if radius == 0 or decay == 0:
        assert np.array_equal(out, s)
    n = len(s)
    for j in range(n):
        nb = [i for i in range(max(0, j - radius), min(n, j + radius + 1)) if i != j]
        beaten = [i for i in nb if s[i] > s[j] or (s[i] == s[j] and i < j)]
        if not beaten:
            assert out[j] == s[j]          # the local maximum (in top-k order) keeps its score
        elif decay > 1e-9 and s[j] > 0:
            assert out[j] < s[j]


# ------------------------------------------------------------------ exclusivity
def test_exclusivity_hand_example(golden):
    e = golden["exclusivity_2x2"]
    assert np.allclose(O.cross_head_exclusivity(e["S"], 1.0), e["eps1"], rtol=0, atol=1e-15)
    assert np.allclose(O.cross_head_exclusivity(e["S"], 2.0), e["eps2"], rtol=0, atol=1e-15)


@given(st.integers(1, 5), st.integers(1, 20), st.floats(0.0, 3.0), st.integers(0, 2 ** 31))
@settings(max_examples=80, deadline=None)
def test_exclusivity_invariants(H, n, eps, seed):
    rng = np.random.default_rng(seed)
    S = rng.random((H, n)) * (rng.random((H, n)) > 0.3)
    out = O.cross_head_exclusivity(S, eps)
    if eps == 0 or H == 1:
        assert np.array_equal(out, S)
    assert np.all(out <= S + 1e-15) and np.all(out >= 0)
    # equivariant under a permutation of the heads
    perm = rng.permutation(H)
    assert np.allclose(O.cross_head_exclusivity(S[perm], eps), out[perm], rtol=1e-14, atol=0)
    # a position scored by one head only keeps that head's score
    only = (S > 0).sum(axis=0) == 1
    assert np.allclose(out[:, only], S[:, only], rtol=1e-14, atol=0)


# ------------------------------------------------------------------ composition
def test_discretised_selection_hand_example(golden):
    e = golden["discretise_composite"]
    f = np.asarray(e["f_full"])
    K = np.zeros((2, e["T"], 4))
    for k, key in ((2, "top2"), (1, "top1")):
        sels, S, cand = O.select_heads(f, K, e["T"], e["n_sink"], e["n_recent"], k, e["lambda"],
                                       nms_radius=e["radius"], nms_decay=e["decay"], excl=e["eps"])
        assert cand.tolist() == [1, 2, 3]
        assert np.allclose(S, e["scores"], rtol=0, atol=1e-12)
        assert [s.tolist() for s in sels] == e[key]


@given(st.integers(1, 3), st.integers(1, 60), st.integers(0, 4), st.integers(0, 6), st.integers(0, 70),
       st.sampled_from([0.0, 0.1, 0.5, 1.0]), st.integers(0, 2 ** 31))
@settings(max_examples=80, deadline=None)
def test_all_options_off_is_the_plain_selector(H, T, ns, W, k, lam, seed):
    rng = np.random.default_rng(seed)
    f = rng.random((H, T))
    f /= f.sum(axis=1, keepdims=True)
    K = rng.standard_normal((H, T, 8))
    sels, _, _ = O.select_heads(f, K, T, ns, W, k, lam)
    for g in range(H):
        assert np.array_equal(sels[g], O.select(f[g], T, ns, W, k, lam)[0])


def test_options_change_the_selection_as_stated():
    """Each option moves a small selection the way its reading says: the
    key-norm correction drops a candidate kept only for its prior weight once
    its key norm is extreme; Soft-NMS thins a run of equally heavy
    neighbours; exclusivity moves a head off positions that another head
    scores more strongly."""
    rng = np.random.default_rng(5)
    T, ns, W = 200, 4, 16
    K = rng.standard_normal((2, T, 16))
    # flat evidence: the prior alone decides, and its peaks are the two ends
    flat = np.full((2, T), 1.0 / T)
    base, _, _ = O.select_heads(flat, K, T, ns, W, 2, 0.5)
    assert base[0].tolist() == [ns, T - W - 1]
    K[0, ns] *= 40.0                                   # an extreme key norm at the first candidate
    kn, _, _ = O.select_heads(flat, K, T, ns, W, 2, 0.5, knorm_beta=50.0, knorm_c=1.0)
    assert ns not in kn[0] and T - W - 1 in kn[0]
    f = np.full((2, T), 1e-4)
    f[0, 50:54] = 0.05                                 # a run of four equally heavy neighbours (head 0)
    f[0, 120] = 0.04
    f[1, 50:54] = 0.2                                  # head 1 scores the same run more strongly
    f[1, 150] = 0.03
    f /= f.sum(axis=1, keepdims=True)
    base, _, _ = O.select_heads(f, K, T, ns, W, 2, 0.0)
    assert base[0].tolist() == [50, 51]
    nms, _, _ = O.select_heads(f, K, T, ns, W, 2, 0.0, nms_radius=1, nms_decay=0.9)
    assert nms[0].tolist() == [50, 120]
    one, _, _ = O.select_heads(f, K, T, ns, W, 1, 0.0)
    ex, _, _ = O.select_heads(f, K, T, ns, W, 1, 0.0, excl=4.0)
    assert one[0].tolist() == [50] and ex[0].tolist() == [120]
    assert one[1].tolist() == [50] and ex[1].tolist() == [150]    # both heads move to positions of their own
