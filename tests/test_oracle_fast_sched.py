"""Pins for the oracle's fast step (O7), span schedule (O8) and loop (O9).

Fast step: equals the dense step when the support covers the context, equals
library SDPA over the gathered sub-cache, and reduces to one value row for a
one-position support.  Schedule: the published splitmix64 sequence, exact
span positions for fixed spans, the geometric law's mean and first-step
probability, and the forced-refresh rule.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _cache(rng, Hq, Hkv, T, D):
    return (rng.standard_normal((Hq, D)) * 2, rng.standard_normal((Hkv, T, D)),
            rng.standard_normal((Hkv, T, D)))


# --------------------------------------------------------------- fast (O7)
@pytest.mark.parametrize("T,ns,w,k", [(300, 4, 16, 280), (300, 4, 16, 10 ** 6), (64, 0, 0, 64), (40, 4, 64, 5)])
def test_fast_equals_dense_when_support_covers_context(T, ns, w, k):
    rng = np.random.default_rng(T + k)
    q, K, V = _cache(rng, 8, 2, T, 32)
    out_d, f, sels = O.slow_step(q, K, V, T, ns, w, k, 0.1)
    out_f = O.fast_step(q, K, V, T, ns, w, sels)
    assert np.max(np.abs(out_f - out_d)) < 1e-12


def test_fast_equals_library_sdpa_on_gathered_rows():
    rng = np.random.default_rng(21)
    Hq, Hkv, T, D = 8, 2, 500, 64
    q, K, V = _cache(rng, Hq, Hkv, T, D)
    _, _, sels = O.slow_step(q, K, V, T, 4, 32, 50, 0.1)
    out = O.fast_step(q, K, V, T, 4, 32, sels)
    for g in range(Hkv):
        S = O.support(T, 4, 32, sels[g])
        qt = torch.from_numpy(q[4 * g:4 * g + 4])[:, None, :]
        kt = torch.from_numpy(K[g][S])[None].expand(4, -1, -1)
        vt = torch.from_numpy(V[g][S])[None].expand(4, -1, -1)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)[:, 0].numpy()
        assert np.max(np.abs(out[4 * g:4 * g + 4] - ref)) < 1e-12


def test_single_position_support_returns_that_value_row():
    """No sinks, no window, k = 1: the support is the position with the most
    mass and the output is exactly its value row."""
    rng = np.random.default_rng(4)
    Hq, Hkv, T, D = 4, 1, 100, 16
    K = rng.standard_normal((Hkv, T, D)) * 0.1
    V = rng.standard_normal((Hkv, T, D))
    j_star = 61
    K[0, j_star] = 0.0; K[0, j_star, 3] = 20.0
    q = np.zeros((Hq, D)); q[:, 3] = 1.0
    _, f, sels = O.slow_step(q, K, V, T, 0, 0, 1, 0.0)
    assert sels[0].tolist() == [j_star]
    out = O.fast_step(q, K, V, T, 0, 0, sels)
    assert np.array_equal(out, np.repeat(V[0, j_star][None], Hq, axis=0))


def test_fast_uses_only_the_support():
    """Changing K/V outside the support leaves the fast step unchanged."""
    rng = np.random.default_rng(9)
    q, K, V = _cache(rng, 8, 2, 400, 32)
    _, _, sels = O.slow_step(q, K, V, 400, 4, 16, 20, 0.1)
    out1 = O.fast_step(q, K, V, 400, 4, 16, sels)
    K2, V2 = K.copy(), V.copy()
    for g in range(2):
        S = set(O.support(400, 4, 16, sels[g]).tolist())
        outside = [j for j in range(400) if j not in S]
        K2[g, outside] = rng.standard_normal((len(outside), 32)) * 5
        V2[g, outside] = 1e3
    out2 = O.fast_step(q, K2, V2, 400, 4, 16, sels)
    assert np.array_equal(out1, out2)


def test_kv_append_then_attend_sees_new_token():
    rng = np.random.default_rng(1)
    Hq, Hkv, cap, D = 4, 1, 20, 8
    K = np.zeros((Hkv, cap, D)); V = np.zeros((Hkv, cap, D))
    K[:, :10] = rng.standard_normal((Hkv, 10, D)); V[:, :10] = rng.standard_normal((Hkv, 10, D))
    kn = np.zeros((Hkv, D)); kn[0, 0] = 50.0
    vn = np.full((Hkv, D), 3.0)
    O.kv_append(K, V, 10, kn, vn)
    q = np.zeros((Hq, D)); q[:, 0] = 1.0
    out, _ = O.dense_attention(q, K[:, :11], V[:, :11])
    assert np.max(np.abs(out - 3.0)) < 1e-6


# ---------------------------------------------------------- schedule (O8)
def test_splitmix64_published_sequence():
    with open(os.path.join(HERE, "golden", "splitmix64.json")) as fh:
        ex = json.load(fh)
    st = ex["seed"]
    for want in ex["outputs"]:
        st, x = O.splitmix64_next(st)
        assert x == want


def test_fixed_spans_slow_positions():
    flags = O.schedule("fixed", 16, 123, 64)
    assert [i for i, s in enumerate(flags) if s] == [0, 16, 32, 48]


def test_geometric_mean_and_first_step_probability():
    mu = 18.0
    n_spans, lens = 0, []
    s = O.SpanSchedule("geometric", mu, 1003)
    cur = None
    for _ in range(2_000_000):
        if s.step():
            if cur is not None:
                lens.append(cur)
            cur = 1
        else:
            cur += 1
    lens = np.array(lens)
    n = len(lens)
    assert n > 100_000
    # geometric on {1,2,...} with p = 1/mu: mean mu, sd sqrt(1-p)/p
    p = 1.0 / mu
    sd = math.sqrt(1 - p) / p
    assert abs(lens.mean() - mu) < 3.3 * sd / math.sqrt(n)
    frac1 = np.mean(lens == 1)
    assert abs(frac1 - p) < 3.3 * math.sqrt(p * (1 - p) / n)


def test_geometric_threshold_exact():
    assert O.SpanSchedule("geometric", 18, 0).threshold == (1 << 64) // 18
    assert O.SpanSchedule("geometric", 1, 0).threshold == 1 << 64
    assert O.SpanSchedule("geometric", 2.5, 0).threshold == (2 * (1 << 64)) // 5
    assert all(O.schedule("geometric", 1.0, 5, 50))                 # mean 1: every step slow


def test_forced_refresh_after_t_max_fast_steps():
    flags = O.schedule("fixed", 100, 0, 30, t_max=5)
    assert [i for i, s in enumerate(flags) if s] == [0, 6, 12, 18, 24]
    s = O.SpanSchedule("fixed", 10, 0)
    seq = [s.step() for _ in range(3)]
    s.force_slow()
    seq += [s.step() for _ in range(12)]
    assert [i for i, x in enumerate(seq) if x] == [0, 3, 13]


def test_sequences_are_independent():
    a = O.schedule("geometric", 18, 1000, 5000)
    b = O.schedule("geometric", 18, 1001, 5000)
    assert a != b and a[0] and b[0]


# ---------------------------------------------------------- loop (O9)
def test_loop_span_refresh_semantics():
    """A slow step returns the dense output; the selection it makes is what
    the following fast steps of the span use."""
    rng = np.random.default_rng(2)
    Hq, Hkv, T, D = 8, 2, 256, 16
    q, K, V = _cache(rng, Hq, Hkv, T, D)
    flags = O.schedule("fixed", 4, 0, 8)
    sels = None
    for t, slow in enumerate(flags):
        qt = q * (1 + 0.01 * t)
        if slow:
            out, f, sels = O.slow_step(qt, K, V, T, 4, 8, 16, 0.1)
            dense, _ = O.dense_attention(qt, K, V)
            assert np.array_equal(out, dense)
        else:
            out = O.fast_step(qt, K, V, T, 4, 8, sels)
            assert out.shape == (Hq, D)
