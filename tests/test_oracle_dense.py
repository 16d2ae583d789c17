"""Pins for the oracle's dense slow step (O1) and its evidence (O2).

The dense step is exact softmax attention, so it is pinned to a library
routine (torch's scaled_dot_product_attention in float64 on the CPU), to
hand-worked examples, and to closed forms (one position, zero query, one
dominant logit).
"""
import math

import numpy as np
import pytest
import torch

import oracle as O


def _sdpa_reference(q, K, V):
    """torch CPU float64 SDPA with GQA expanded by repeat_interleave."""
    Hq, D = q.shape
    Hkv, T, _ = K.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q)[:, None, :]                       # [Hq, 1, D]
    kt = torch.from_numpy(K).repeat_interleave(G, dim=0)       # [Hq, T, D]
    vt = torch.from_numpy(V).repeat_interleave(G, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt)
    return o[:, 0, :].numpy()


@pytest.mark.parametrize("Hq,Hkv,T,D,seed", [
    (8, 2, 37, 64, 0), (4, 4, 1, 16, 1), (6, 3, 300, 32, 2), (32, 8, 129, 128, 3), (2, 1, 5, 8, 4)])
def test_dense_matches_library_sdpa(Hq, Hkv, T, D, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((Hq, D)) * 2
    K = rng.standard_normal((Hkv, T, D))
    V = rng.standard_normal((Hkv, T, D))
    out, P = O.dense_attention(q, K, V)
    ref = _sdpa_reference(q, K, V)
    assert np.max(np.abs(out - ref)) < 1e-12
    assert np.max(np.abs(P.sum(axis=1) - 1.0)) < 1e-12


def test_dense_hand_examples(golden):
    for key in ("dense_two_positions", "dense_gqa_three_positions"):
        ex = golden[key]
        out, P = O.dense_attention(np.array(ex["q"]), np.array(ex["K"]), np.array(ex["V"]))
        assert np.allclose(out, np.array(ex["out"]), atol=1e-14, rtol=0), key
        if "P" in ex:
            assert np.allclose(P, np.array(ex["P"]), atol=1e-15, rtol=0)
        if "f" in ex:
            f = O.group_mass(P, np.array(ex["K"]).shape[0])
            assert np.allclose(f, np.array(ex["f"]), atol=1e-15, rtol=0)


def test_dense_closed_forms():
    rng = np.random.default_rng(7)
    Hq, Hkv, D = 8, 2, 16
    # one position: the output is that position's value row
    K = rng.standard_normal((Hkv, 1, D)); V = rng.standard_normal((Hkv, 1, D))
    q = rng.standard_normal((Hq, D))
    out, _ = O.dense_attention(q, K, V)
    for h in range(Hq):
        assert np.array_equal(out[h], V[h // 4, 0])
    # zero query: uniform weights, output = mean of the value rows
    T = 50
    K = rng.standard_normal((Hkv, T, D)); V = rng.standard_normal((Hkv, T, D))
    out, P = O.dense_attention(np.zeros((Hq, D)), K, V)
    for h in range(Hq):
        assert np.max(np.abs(out[h] - V[h // 4].mean(axis=0))) < 1e-14
        assert np.max(np.abs(P[h] - 1.0 / T)) < 1e-16
    # one logit 60 above the rest: output = that value row (e^-60 ~ 1e-26)
    K = np.zeros((Hkv, T, D)); j_star = 17
    K[:, j_star, 0] = 60.0 * math.sqrt(D)
    q = np.zeros((Hq, D)); q[:, 0] = 1.0
    out, _ = O.dense_attention(q, K, V)
    for h in range(Hq):
        assert np.max(np.abs(out[h] - V[h // 4, j_star])) < 1e-12


def test_gqa_mapping_is_contiguous_groups():
    """Query heads 0..G-1 read KV head 0, G..2G-1 read KV head 1, and so on."""
    Hq, Hkv, T, D = 6, 3, 4, 2
    K = np.zeros((Hkv, T, D))
    V = np.zeros((Hkv, T, D))
    for g in range(Hkv):
        V[g, :, 0] = 10.0 * (g + 1)
    out, _ = O.dense_attention(np.ones((Hq, D)), K, V)
    assert list(out[:, 0]) == [10.0, 10.0, 20.0, 20.0, 30.0, 30.0]


def test_mass_sums_and_group_mean():
    rng = np.random.default_rng(11)
    Hq, Hkv, T, D = 8, 2, 200, 32
    q = rng.standard_normal((Hq, D)) * 3
    K = rng.standard_normal((Hkv, T, D)); V = rng.standard_normal((Hkv, T, D))
    _, P = O.dense_attention(q, K, V)
    f = O.group_mass(P, Hkv)
    assert np.max(np.abs(f.sum(axis=1) - 1.0)) < 1e-12
    for g in range(Hkv):
        explicit = (P[4 * g] + P[4 * g + 1] + P[4 * g + 2] + P[4 * g + 3]) / 4.0
        assert np.max(np.abs(f[g] - explicit)) < 1e-16
    # the mass of a head group depends only on that group's query heads
    q2 = q.copy(); q2[4:] = 0.0
    _, P2 = O.dense_attention(q2, K, V)
    f2 = O.group_mass(P2, Hkv)
    assert np.array_equal(f2[0], f[0])
    assert np.max(np.abs(f2[1] - 1.0 / T)) < 1e-16


def test_scale_is_inverse_sqrt_head_dim():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 64)); K = rng.standard_normal((1, 9, 64)); V = rng.standard_normal((1, 9, 64))
    a, _ = O.dense_attention(q, K, V)
    b, _ = O.dense_attention(q, K, V, scale=1.0 / 8.0)
    c, _ = O.dense_attention(q * 0.125, K, V, scale=1.0)
    assert np.array_equal(a, b)
    assert np.max(np.abs(a - c)) < 1e-14


def test_empty_context_rejected():
    with pytest.raises(ValueError):
        O.dense_attention(np.zeros((2, 4)), np.zeros((1, 0, 4)), np.zeros((1, 0, 4)))
