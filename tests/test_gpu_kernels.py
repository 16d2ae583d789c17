"""GPU parity of each kernel against the CPU oracle on small seeded inputs that
span several tiles and splits with ragged tails, plus edge cases."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import (OUT_TOL, check_mass, check_support, np64, oracle_slow, random_cache,
                               run_slow)

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_slow_step_shapes(dtype, D, G):
    Hkv = 2
    ctx = [1000, 3001, 17]
    kv, q = random_cache(3, G * Hkv, Hkv, 3072, D, DT[dtype], ctx, seed=100 + D + G, q_scale=2.0)
    out, mass = run_slow(kv, q, [0, 1, 2])
    for b in range(3):
        o_ref, f_ref = oracle_slow(kv, q, b)
        T = ctx[b]
        assert np.max(np.abs(np64(out[b]) - o_ref)) < OUT_TOL
        check_mass(np64(mass[b, :, :T]), f_ref, b)
        assert torch.all(mass[b, :, T:] == -1.0)          # beyond ctx untouched


@pytest.mark.parametrize("T", [1, 2, 255, 256, 257, 4097])
def test_slow_step_context_edges(T):
    kv, q = random_cache(1, 8, 2, 4200, 128, torch.bfloat16, [T], seed=T, q_scale=3.0)
    out, mass = run_slow(kv, q, [0])
    o_ref, f_ref = oracle_slow(kv, q, 0)
    assert np.max(np.abs(np64(out[0]) - o_ref)) < OUT_TOL
    check_mass(np64(mass[0, :, :T]), f_ref, T)
    if T == 1:
        assert np.max(np.abs(np64(out[0]) - np.repeat(np64(kv.v[0, :, 0]), 4, axis=0))) < 1e-6


def test_slow_without_mass_and_subset_rows():
    kv, q = random_cache(4, 32, 8, 2048, 128, torch.bfloat16, [2048, 1500, 999, 64], seed=7)
    dev = kv.k.device
    out = torch.full((4, 32, 128), 7.0, device=dev)
    ws = S.alloc_workspace(kv)
    S.sfi_slow_step(kv, [2, 0], q, out, None, ws)
    torch.cuda.synchronize()
    for b in (0, 2):
        o_ref, _ = oracle_slow(kv, q, b)
        assert np.max(np.abs(np64(out[b]) - o_ref)) < OUT_TOL
    assert torch.all(out[1] == 7.0) and torch.all(out[3] == 7.0)    # unlisted rows untouched


def test_context_beyond_the_logit_buffer():
    """600000 rows: with at most 512 splits per head, each split is longer
    than the 1024 rows whose logits a workgroup buffers in LDS, so the slow
    partial stores its logits block by block.  Separate calls and the fused
    refresh (with a Selector over ~600K candidates) against the oracle."""
    T, Hq, Hkv, D, ns, W, k = 600000, 4, 1, 64, 16, 256, 2048
    kv, q = random_cache(1, Hq, Hkv, T, D, torch.float32, [T], seed=42, q_scale=2.0)
    splits = S.sfi_slow_plan(kv, [0])[0]
    assert splits <= 512 and -(-T // splits) > 1024
    out, mass = run_slow(kv, q, [0])
    o_ref, f_ref = oracle_slow(kv, q, 0)
    assert np.max(np.abs(np64(out[0]) - o_ref)) < OUT_TOL
    check_mass(np64(mass[0]), f_ref, T)
    sp = S.support_params(ns, W, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    dev = kv.k.device
    out2 = torch.empty_like(out)
    mass2 = torch.empty_like(mass)
    sel = torch.empty(1, Hkv, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, Hkv, dtype=torch.int32, device=dev)
    pk = torch.empty(1, Hkv, k, D, dtype=torch.float32, device=dev)
    pv = torch.empty_like(pk)
    S.sfi_slow_step_select(kv, sp, [0], q, out2, mass2, sel, cnt, pk, pv, ws)
    torch.cuda.synchronize()
    assert torch.equal(out2, out) and torch.equal(mass2, mass)
    got = sel[0, 0, :int(cnt[0, 0])].cpu().numpy()
    assert int(cnt[0, 0]) == k and np.all(np.diff(got) > 0)
    check_support(got, f_ref[0], T, ns, W, k, 0.1, "T=600000")
    assert torch.equal(pk[0, 0], kv.k[0, 0][torch.from_numpy(got).to(dev).long()])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_explicit_logit_scale(dtype):
    """A caller-given logit scale (not 1/sqrt(D)) reaches the slow partial, the
    mass, the Selector and both fast steps."""
    T, Hq, Hkv, D, ns, W, k, scale = 5000, 16, 4, 128, 8, 64, 300, 0.21
    kv0, q = random_cache(1, Hq, Hkv, T, D, DT[dtype], [T], seed=21, q_scale=1.0)
    kv = S.KVDesc(kv0.k, kv0.v, [T], Hq, scale=scale)
    sp = S.support_params(ns, W, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    dev = kv.k.device
    out = torch.empty(1, Hq, D, device=dev)
    mass = torch.empty(1, Hkv, T, device=dev)
    sel = torch.empty(1, Hkv, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, Hkv, dtype=torch.int32, device=dev)
    pk = torch.empty(1, Hkv, k, D, dtype=DT[dtype], device=dev)
    pv = torch.empty_like(pk)
    S.sfi_slow_step_select(kv, sp, [0], q, out, mass, sel, cnt, pk, pv, ws)
    out_p = torch.empty_like(out)
    out_g = torch.empty_like(out)
    S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out_p, ws)
    S.sfi_fast_step(kv, sp, [0], q, sel, cnt, out_g, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_g)
    K64, V64, q64 = np64(kv.k[0]), np64(kv.v[0]), np64(q[0])
    o_ref, P = O.dense_attention(q64, K64, V64, scale=scale)
    f_ref = O.group_mass(P, Hkv)
    assert np.max(np.abs(np64(out[0]) - o_ref)) < OUT_TOL
    check_mass(np64(mass[0]), f_ref, "scale")
    sels = []
    for g in range(Hkv):
        got = sel[0, g, :int(cnt[0, g])].cpu().numpy()
        check_support(got, f_ref[g], T, ns, W, k, 0.1, f"g{g}")
        sels.append(got.astype(np.int64))
    ref = O.fast_step(q64, K64, V64, T, ns, W, sels, scale=scale)
    assert np.max(np.abs(np64(out_p[0]) - ref)) < OUT_TOL
    # the default scale gives a different result on these inputs
    o_def, _ = O.dense_attention(q64, K64, V64)
    assert np.max(np.abs(o_def - o_ref)) > 10 * OUT_TOL


def test_slow_deterministic():
    kv, q = random_cache(1, 32, 8, 40000, 128, torch.bfloat16, [39999], seed=3)
    a_out, a_mass = run_slow(kv, q, [0])
    b_out, b_mass = run_slow(kv, q, [0])
    assert torch.equal(a_out, b_out) and torch.equal(a_mass, b_mass)


# ------------------------------------------------------------------ select
def _select_gpu(kv, sp, ids, mass):
    dev = kv.k.device
    sel = torch.full((kv.batch, kv.n_kv_heads, sp.top_k), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((kv.batch, kv.n_kv_heads), -7, dtype=torch.int32, device=dev)
    S.sfi_select(kv, sp, ids, mass, sel, cnt, S.alloc_workspace(kv, sp))
    torch.cuda.synchronize()
    return sel.cpu().numpy(), cnt.cpu().numpy()


def _mass_cache(B, Hkv, cap, ctx):
    dev = torch.device("cuda:0")
    K = torch.zeros(B, Hkv, cap, 64, device=dev)
    kv = S.KVDesc(K, K.clone(), ctx, Hkv * 4)
    return kv


@pytest.mark.parametrize("lam", [0.0, 0.1, 0.5, 1.0])
@pytest.mark.parametrize("T,ns,W,k", [(5000, 4, 64, 256), (5000, 16, 256, 2048), (300, 4, 16, 1),
                                      (100, 4, 16, 200), (20, 4, 16, 5), (10, 4, 16, 5), (70000, 16, 256, 2048)])
def test_select_random_mass(lam, T, ns, W, k):
    rng = np.random.default_rng(T + k)
    Hkv, cap = 3, T + 5
    f = rng.gamma(0.3, size=(1, Hkv, cap)).astype(np.float32)
    f /= f[..., :T].sum(axis=-1, keepdims=True)
    kv = _mass_cache(1, Hkv, cap, [T])
    mass = torch.from_numpy(f).cuda()
    sp = S.support_params(ns, W, k, lam)
    sel, cnt = _select_gpu(kv, sp, [0], mass)
    n = max(0, T - ns - W)
    for g in range(Hkv):
        c = int(cnt[0, g])
        assert c == min(k, n)
        assert np.all(sel[0, g, c:] == -1)
        assert np.all(np.diff(sel[0, g, :c]) > 0)            # ascending
        check_support(sel[0, g, :c], f[0, g].astype(np.float64), T, ns, W, k, lam, f"g{g}")


@pytest.mark.parametrize("k", [1, 7, 64, 1000])
def test_select_ties_exact(k):
    """Evidence with heavy exact ties and lambda = 0: the fp32 and fp64 scores
    coincide, so the lowest-index rule must match bit for bit."""
    rng = np.random.default_rng(k)
    T, ns, W, Hkv = 6000, 4, 64, 2
    f = (rng.integers(0, 4, size=(1, Hkv, T)).astype(np.float32) / 8.0)
    kv = _mass_cache(1, Hkv, T, [T])
    sel, cnt = _select_gpu(kv, S.support_params(ns, W, k, 0.0), [0], torch.from_numpy(f).cuda())
    for g in range(Hkv):
        ora = O.select(f[0, g].astype(np.float64), T, ns, W, k, 0.0)[0]
        assert sel[0, g, :cnt[0, g]].tolist() == ora.tolist()


@pytest.mark.parametrize("lam", [0.0, 0.1])
@pytest.mark.parametrize("T", [5000, 60000])
def test_select_large_threshold_bin_with_keys_above(T, lam):
    """Flat evidence plus heavy positions spread over every chunk.  With
    lambda = 0 the k-th key's bin holds every flat candidate: at T = 5000 a
    few thousand keys, resolved by radix levels in LDS; at T = 60000 more
    than fit in LDS, resolved by radix passes over all candidates.  Keys
    above that bin sit in every chunk, so each chunk's output offset has both
    kinds of keys before it.  Checked against the oracle, set and order."""
    rng = np.random.default_rng(11)
    ns, W, k, Hkv = 16, 256, 2048, 2
    n = T - ns - W
    f = np.full((1, Hkv, T), 1.0, dtype=np.float32)
    for g in range(Hkv):
        heavy = rng.choice(n, size=900 + 300 * g, replace=False) + ns
        f[0, g, heavy] = 3.0
    f /= f.sum(axis=-1, keepdims=True)
    kv = _mass_cache(1, Hkv, T, [T])
    sp = S.support_params(ns, W, k, lam)
    sel, cnt = _select_gpu(kv, sp, [0], torch.from_numpy(f).cuda())
    for g in range(Hkv):
        got = sel[0, g].tolist()
        assert cnt[0, g] == k and got == sorted(got), g
        if lam == 0.0:  # fp32 and fp64 scores coincide: the set is unique
            assert got == O.select(f[0, g].astype(np.float64), T, ns, W, k, lam)[0].tolist(), g
        else:
            check_support(np.asarray(got), f[0, g].astype(np.float64), T, ns, W, k, lam, f"g{g}")


def test_select_all_equal_and_prior_closed_form():
    """Uniform evidence: with lambda > 0 the choice follows the prior (both ends
    of the candidate range); with lambda = 0 every score ties and the lowest k
    positions win.  Exercises the deepest radix path (no early LDS copy)."""
    T, ns, W, k, Hkv = 20000, 16, 256, 2048, 1
    f = np.full((1, Hkv, T), 1.0 / T, dtype=np.float32)
    kv = _mass_cache(1, Hkv, T, [T])
    n = T - ns - W
    sel, cnt = _select_gpu(kv, S.support_params(ns, W, k, 0.0), [0], torch.from_numpy(f).cuda())
    assert sel[0, 0].tolist() == list(range(ns, ns + k))
    sel, cnt = _select_gpu(kv, S.support_params(ns, W, k, 1.0), [0], torch.from_numpy(f).cuda())
    a = sel[0, 0] - ns + 1
    assert a.tolist() == list(range(1, k // 2 + 1)) + list(range(n - k // 2 + 1, n + 1))


# ------------------------------------------------------------------ fast step
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_fast_step_with_oracle_support(dtype, D, G):
    Hkv, ns, W, k = 2, 4, 64, 200
    ctx = [3000, 700, 50]
    kv, q = random_cache(3, G * Hkv, Hkv, 3000, D, DT[dtype], ctx, seed=G * D, q_scale=2.0)
    dev = kv.k.device
    sel = torch.full((3, Hkv, k), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(3, Hkv, dtype=torch.int32, device=dev)
    sels = {}
    for b in range(3):
        T = ctx[b]
        _, f = oracle_slow(kv, q, b)
        for g in range(Hkv):
            s = O.select(f[g], T, ns, W, k, 0.1)[0]
            sels[(b, g)] = s
            sel[b, g, :len(s)] = torch.from_numpy(s.astype(np.int32))
            cnt[b, g] = len(s)
    sp = S.support_params(ns, W, k, 0.1)
    out = torch.full((3, G * Hkv, D), float("nan"), device=dev)
    ws = S.alloc_workspace(kv, sp)
    S.sfi_fast_step(kv, sp, [0, 1, 2], q, sel, cnt, out, ws)
    S.sfi_fast_step(kv, sp, [0, 1, 2], q, sel, cnt, out, ws)   # counters reset by the first call
    torch.cuda.synchronize()
    for b in range(3):
        T = ctx[b]
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, ns, W,
                          [sels[(b, g)] for g in range(Hkv)])
        assert np.max(np.abs(np64(out[b]) - ref)) < OUT_TOL


def test_fast_equals_slow_when_support_covers_context():
    kv, q = random_cache(2, 32, 8, 2500, 128, torch.bfloat16, [2500, 1234], seed=5, q_scale=2.0)
    sp = S.support_params(16, 256, 4096, 0.1)
    ws = S.alloc_workspace(kv, sp)
    dev = kv.k.device
    out_s, mass = run_slow(kv, q, [0, 1], ws=ws)
    sel = torch.empty(2, 8, 4096, dtype=torch.int32, device=dev)
    cnt = torch.empty(2, 8, dtype=torch.int32, device=dev)
    S.sfi_select(kv, sp, [0, 1], mass, sel, cnt, ws)
    out_f = torch.empty_like(out_s)
    S.sfi_fast_step(kv, sp, [0, 1], q, sel, cnt, out_f, ws)
    torch.cuda.synchronize()
    assert torch.max(torch.abs(out_f - out_s)).item() < OUT_TOL


def test_fast_ignores_out_of_range_indices_and_counts():
    kv, q = random_cache(1, 8, 2, 1000, 64, torch.float32, [900], seed=9)
    dev = kv.k.device
    ns, W, k = 4, 16, 8
    sp = S.support_params(ns, W, k, 0.1)
    good = np.array([10, 20, 30, 40], dtype=np.int32)
    sel = torch.full((1, 2, k), -1, dtype=torch.int32, device=dev)
    sel[0, :, :4] = torch.from_numpy(good)
    sel[0, :, 4] = 950          # beyond the context: ignored
    sel[0, :, 5] = -5           # negative: ignored
    cnt = torch.tensor([[6, 4]], dtype=torch.int32, device=dev)
    out = torch.empty(1, 8, 64, device=dev)
    S.sfi_fast_step(kv, sp, [0], q, sel, cnt, out, S.alloc_workspace(kv, sp))
    torch.cuda.synchronize()
    ref = O.fast_step(np64(q[0]), np64(kv.k[0, :, :900]), np64(kv.v[0, :, :900]), 900, ns, W, [good, good])
    assert np.max(np.abs(np64(out[0]) - ref)) < OUT_TOL


def test_debug_support_matches_oracle_sets():
    T, ns, W, k, Hkv = 5000, 16, 256, 100, 2
    kv = _mass_cache(1, Hkv, T, [T])
    rng = np.random.default_rng(1)
    f = rng.random((1, Hkv, T)).astype(np.float32)
    sp = S.support_params(ns, W, k, 0.1)
    sel, cnt = _select_gpu(kv, sp, [0], torch.from_numpy(f).cuda())
    dev = torch.device("cuda:0")
    sup = torch.full((1, Hkv, 512), -9, dtype=torch.int32, device=dev)
    scnt = torch.zeros(1, Hkv, dtype=torch.int32, device=dev)
    S.sfi_debug_support(kv, sp, [0], torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(), sup, scnt)
    torch.cuda.synchronize()
    for g in range(Hkv):
        c = int(scnt[0, g])
        got = sup[0, g, :c].cpu().numpy()
        assert sorted(got.tolist()) == O.support(T, ns, W, sel[0, g, :cnt[0, g]]).tolist()


# ------------------------------------------------------------------ append
def test_kv_append_then_slow_step():
    kv, q = random_cache(2, 8, 2, 600, 128, torch.bfloat16, [500, 300], seed=11)
    dev = kv.k.device
    kn = torch.randn(2, 2, 128, device=dev).to(torch.bfloat16)
    vn = torch.randn(2, 2, 128, device=dev).to(torch.bfloat16)
    S.sfi_kv_append(kv, [0, 1], kn, vn)
    torch.cuda.synchronize()
    assert torch.equal(kv.k[0, :, 500], kn[0]) and torch.equal(kv.v[1, :, 300], vn[1])
    kv.ctx[:] = [501, 301]
    out, _ = run_slow(kv, q, [0, 1])
    for b in range(2):
        o_ref, _ = oracle_slow(kv, q, b)
        assert np.max(np.abs(np64(out[b]) - o_ref)) < OUT_TOL


# ------------------------------------------------------------------ errors
def test_invalid_arguments_raise_before_launch():
    kv, q = random_cache(1, 8, 2, 100, 64, torch.float32, [100], seed=1)
    out = torch.empty(1, 8, 64, device=kv.k.device)
    with pytest.raises(S.SFIError):
        S.sfi_slow_step(kv, [1], q, out, None, S.alloc_workspace(kv))   # id out of range
    with pytest.raises(S.SFIError):
        S.sfi_slow_step(kv, [0], q, out, None, None)                       # no workspace
    kv.ctx[0] = 101
    with pytest.raises(S.SFIError):
        S.sfi_slow_step(kv, [0], q, out, None, S.alloc_workspace(kv))    # ctx beyond capacity


@pytest.mark.parametrize("G,k", [(4, 10000), (8, 5000), (1, 33000)])
def test_fast_step_large_support(G, k):
    """Supports of 5K to 33K rows per KV head: more chunk partials per head
    than the merge gathers in its first round trip (64 for G = 4, 32 for
    G = 8, 256 for G = 1), so the merge loops.  Fused refresh, then packed
    and gather fast steps against each other and the oracle."""
    Hkv, ns, W, D = 2, 16, 256, 128
    ctx = [k + 9000, k // 2 + 400]
    B = len(ctx)
    kv, q = random_cache(B, G * Hkv, Hkv, max(ctx), D, torch.bfloat16, ctx, seed=G + k, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(ns, W, k, 0.1)
    chunks = S.sfi_fast_plan(kv, sp, [0])[0]
    assert chunks > {1: 256, 4: 64, 8: 32}[G]
    ws = S.alloc_workspace(kv, sp)
    ids = list(range(B))
    out = torch.empty(B, G * Hkv, D, device=dev)
    mass = torch.empty(B, Hkv, max(ctx), device=dev)
    sel = torch.empty(B, Hkv, k, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)
    pk = torch.empty(B, Hkv, k, D, dtype=torch.bfloat16, device=dev)
    pv = torch.empty_like(pk)
    S.sfi_slow_step_select(kv, sp, ids, q, out, mass, sel, cnt, pk, pv, ws)
    out_g = torch.full_like(out, float("nan"))
    out_p = torch.full_like(out, float("nan"))
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_g, ws)
    S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, out_p, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out_p)
    for b in range(B):
        T = ctx[b]
        c = cnt[b].cpu().numpy()
        sels = [sel[b, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(Hkv)]
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, ns, W, sels)
        assert np.max(np.abs(np64(out_p[b]) - ref)) < OUT_TOL


# ------------------------------------------------------------------ packed support
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_packed_fast_equals_gather_and_oracle(dtype, D, G):
    """Packing the selected rows and streaming them gives the gather kernel's
    result bit for bit (same support order and chunking), and the oracle's
    within tolerance; short contexts exercise the sink/window clipping."""
    Hkv, ns, W, k = 2, 4, 64, 200
    ctx = [3000, 700, 50, 3]
    B = len(ctx)
    kv, q = random_cache(B, G * Hkv, Hkv, 3000, D, DT[dtype], ctx, seed=3 * G + D, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(ns, W, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = list(range(B))
    _, mass = run_slow(kv, q, ids, ws=ws)
    sel = torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(B, Hkv, dtype=torch.int32, device=dev)
    S.sfi_select(kv, sp, ids, mass, sel, cnt, ws)
    pk = torch.zeros(B, Hkv, k, D, dtype=DT[dtype], device=dev)
    pv = torch.zeros_like(pk)
    S.sfi_pack_support(kv, sp, ids, sel, cnt, pk, pv)
    out_g = torch.full((B, G * Hkv, D), float("nan"), device=dev)
    out_p = torch.full_like(out_g, float("nan"))
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_g, ws)
    S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, out_p, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_g, out_p)
    for b in range(B):
        T = ctx[b]
        c = cnt[b].cpu().numpy()
        sels = [sel[b, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(Hkv)]
        for g in range(Hkv):
            rows = torch.from_numpy(sels[g]).to(dev)
            assert torch.equal(pk[b, g, :c[g]], kv.k[b, g].index_select(0, rows))
            assert torch.equal(pv[b, g, :c[g]], kv.v[b, g].index_select(0, rows))
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, ns, W, sels)
        assert np.max(np.abs(np64(out_p[b]) - ref)) < OUT_TOL


def test_packed_with_growing_context():
    """The window slides as tokens are appended after the pack; the packed
    selected rows stay valid and the result matches the oracle."""
    kv, q = random_cache(1, 32, 8, 5000, 128, torch.bfloat16, [4000], seed=21, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, 512, 0.1)
    ws = S.alloc_workspace(kv, sp)
    _, mass = run_slow(kv, q, [0], ws=ws)
    sel = torch.empty(1, 8, 512, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, 8, dtype=torch.int32, device=dev)
    S.sfi_select(kv, sp, [0], mass, sel, cnt, ws)
    pk = torch.empty(1, 8, 512, 128, dtype=torch.bfloat16, device=dev)
    pv = torch.empty_like(pk)
    S.sfi_pack_support(kv, sp, [0], sel, cnt, pk, pv)
    for _ in range(5):
        kn = torch.randn(1, 8, 128, device=dev).to(torch.bfloat16)
        S.sfi_kv_append(kv, [0], kn, kn)
        kv.ctx += 1
    out = torch.empty(1, 32, 128, device=dev)
    S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out, ws)
    torch.cuda.synchronize()
    T = int(kv.ctx[0])
    c = cnt[0].cpu().numpy()
    sels = [sel[0, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(8)]
    ref = O.fast_step(np64(q[0]), np64(kv.k[0, :, :T]), np64(kv.v[0, :, :T]), T, 16, 256, sels)
    assert np.max(np.abs(np64(out[0]) - ref)) < OUT_TOL


def test_kernel_timing_events():
    """With timing on, every launch group records one event pair; the summed
    durations are positive and the counts match the calls."""
    kv, q = random_cache(1, 32, 8, 20000, 128, torch.bfloat16, [20000], seed=2)
    dev = kv.k.device
    sp = S.support_params(16, 256, 1024, 0.1)
    ws = S.alloc_workspace(kv, sp)
    out = torch.empty(1, 32, 128, device=dev)
    mass = torch.empty(1, 8, 20000, device=dev)
    sel = torch.empty(1, 8, 1024, dtype=torch.int32, device=dev)
    cnt = torch.empty(1, 8, dtype=torch.int32, device=dev)
    S.sfi_profile_reset()
    S.sfi_profile_enable(True)
    try:
        for _ in range(3):
            S.sfi_slow_step(kv, [0], q, out, mass, ws)
            S.sfi_select(kv, sp, [0], mass, sel, cnt, ws)
            S.sfi_fast_step(kv, sp, [0], q, sel, cnt, out, ws)
    finally:
        S.sfi_profile_enable(False)
    torch.cuda.synchronize()
    for kid in (S.SFI_K_SLOW_PARTIAL, S.SFI_K_SLOW_COMBINE, S.SFI_K_SELECT, S.SFI_K_FAST):
        ms, n = S.sfi_profile_read(kid)
        assert n == 3 and ms > 0, (kid, ms, n)
    # a one-row fast step fits the GPU in one pass: its merge runs inside its kernel
    assert S.sfi_profile_read(S.SFI_K_FAST_MERGE) == (0.0, 0)
    S.sfi_profile_reset()
    assert S.sfi_profile_read(S.SFI_K_FAST) == (0.0, 0)
