"""Seeded random sweep over the whole path: for each drawn configuration
(dtype, head dim, query/KV heads, ragged batch, sinks, window, top-k, lambda,
query scale from 0, where every position ties, to 4, an unordered subset of
rows) one fused refresh and one fast step
of each kind (gather, packed, and gather with packing for a random subset of
the rows) run on the GPU and are checked against the oracle: dense output,
mass, support, packed rows, and the fast output over the GPU's own support
(once that support has passed the support check).  A second, wider set adds
contexts up to 300K rows, batches beyond one launch group and larger top-k."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, check_mass, check_support, np64, oracle_slow, random_cache

pytestmark = pytest.mark.gpu

N_CONFIGS = 80


def draw(seed):
    r = np.random.default_rng(1000 + seed)
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    cap = int(np.exp(r.uniform(np.log(64), np.log(40000))))  # log-uniform: many splits and chunks too
    B = int(r.integers(1, 6))
    ctx = [int(x) for x in r.integers(1, cap + 1, size=B)]
    if r.random() < 0.5:
        ctx[int(r.integers(0, B))] = cap                  # one row at full capacity
    ns = int(r.choice([0, 1, 4, 16, 33]))
    W = int(r.choice([0, 1, 64, 256, 511]))
    k = int(r.choice([0, 1, 17, 256, 1000, 2048, 5000]))
    if ns + W + k == 0:
        k = 8
    ids = [int(x) for x in r.permutation(B)[:int(r.integers(1, B + 1))]]
    return dict(dtype=torch.bfloat16 if r.random() < 0.6 else torch.float32, D=int(r.choice([64, 128])),
                Hkv=Hkv, G=G, cap=cap, ctx=ctx, ns=ns, W=W, k=k, lam=float(r.choice([0.0, 0.1, 0.37, 1.0])),
                q_scale=float(r.choice([0.0, 0.1, 0.5, 2.0, 4.0])), ids=ids)


N_WIDE = 40


def draw_wide(seed):
    """Wider ranges: contexts up to 300K rows (few rows), or batches of up to
    71 rows (more than one launch group of 64), top-k up to 20000, windows up
    to 2000, 100 sinks."""
    r = np.random.default_rng(50000 + seed)
    Hkv = int(r.choice([1, 2, 4, 8]))
    G = int(r.choice([1, 2, 4, 8]))
    big = r.random() < 0.4
    lo, hi = (20000, 300000) if big else (64, 20000)
    cap = int(np.exp(r.uniform(np.log(lo), np.log(hi))))
    B = int(r.integers(1, 4)) if big else int(r.integers(1, 72))
    if B > 8 and Hkv * G > 16:
        Hkv, G = 2, 4
    ctx = [int(x) for x in r.integers(1, cap + 1, size=B)]
    if r.random() < 0.5:
        ctx[int(r.integers(0, B))] = cap
    ns = int(r.choice([0, 1, 4, 16, 100]))
    W = int(r.choice([0, 1, 64, 256, 511, 2000]))
    k = int(r.choice([0, 1, 17, 256, 2048, 5000, 20000]))
    if ns + W + k == 0:
        k = 8
    ids = [int(x) for x in r.permutation(B)[:int(r.integers(1, B + 1))]]
    return dict(dtype=torch.bfloat16 if r.random() < 0.6 else torch.float32, D=int(r.choice([64, 128])),
                Hkv=Hkv, G=G, cap=cap, ctx=ctx, ns=ns, W=W, k=k, lam=float(r.choice([0.0, 0.1, 0.37, 1.0])),
                q_scale=float(r.choice([0.0, 0.1, 0.5, 2.0, 4.0])), ids=ids)


@pytest.mark.parametrize("seed", range(N_CONFIGS))
def test_random_config_against_oracle(seed):
    _run(draw(seed), seed)


@pytest.mark.parametrize("seed", range(N_WIDE))
def test_wide_random_config_against_oracle(seed):
    _run(draw_wide(seed), 50000 + seed)


def _run(c, seed):
    print("config", seed, {key: v for key, v in c.items() if key != "ctx"}, "ctx", c["ctx"], flush=True)
    B, Hkv, G, D, k = len(c["ctx"]), c["Hkv"], c["G"], c["D"], c["k"]
    kv, q = random_cache(B, G * Hkv, Hkv, c["cap"], D, c["dtype"], c["ctx"], seed=seed, q_scale=c["q_scale"])
    dev = kv.k.device
    sp = S.support_params(c["ns"], c["W"], k, c["lam"])
    ws = S.alloc_workspace(kv, sp)
    ids = c["ids"]
    out = torch.full((B, G * Hkv, D), 7.0, device=dev)
    mass = torch.full((B, Hkv, c["cap"]), -1.0, device=dev)
    sel = torch.full((B, Hkv, k), -7, dtype=torch.int32, device=dev)
    cnt = torch.full((B, Hkv), -7, dtype=torch.int32, device=dev)
    pk = torch.zeros(B, Hkv, k, D, dtype=c["dtype"], device=dev)
    pv = torch.zeros_like(pk)
    S.sfi_slow_step_select(kv, sp, ids, q, out, mass, sel, cnt, pk, pv, ws)
    out_p = torch.full_like(out, 7.0)
    out_g = torch.full_like(out, 7.0)
    S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, out_p, ws)
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_g, ws)
    # the packing fast step: some rows gather and pack, the others read the
    # rows the refresh packed (one launch)
    flags = [int(x) for x in np.random.default_rng(seed + 7).random(len(ids)) < 0.5]
    pk_d, pv_d = torch.zeros_like(pk), torch.zeros_like(pv)
    for b, f in zip(ids, flags):
        if not f:
            pk_d[b].copy_(pk[b])
            pv_d[b].copy_(pv[b])
    out_d = torch.full_like(out, 7.0)
    S.sfi_fast_step_pack(kv, sp, ids, q, sel, cnt, out_d, pk_d, pv_d, ws, pack_flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_g)
    assert torch.equal(out_d, out_g)
    assert torch.equal(pk_d, pk) and torch.equal(pv_d, pv)
    for b in range(B):
        if b not in ids:
            assert torch.all(out[b] == 7.0) and torch.all(cnt[b] == -7) and torch.all(mass[b] == -1.0)
            assert torch.all(out_p[b] == 7.0)
            continue
        T = c["ctx"][b]
        o_ref, f_ref = oracle_slow(kv, q, b)
        assert np.max(np.abs(np64(out[b]) - o_ref)) < OUT_TOL, b
        check_mass(np64(mass[b, :, :T]), f_ref, b)
        assert torch.all(mass[b, :, T:] == -1.0), b
        sels = []
        for g in range(Hkv):
            n_g = int(cnt[b, g])
            s = sel[b, g, :n_g].cpu().numpy().astype(np.int64)
            if k > 0:
                check_support(s, f_ref[g], T, c["ns"], c["W"], k, c["lam"], f"seed {seed} b{b} g{g}")
            else:
                assert n_g == 0
            assert np.all(np.diff(s) > 0), (b, g)
            rows = torch.from_numpy(s).to(dev)
            assert torch.equal(pk[b, g, :n_g], kv.k[b, g].index_select(0, rows))
            assert torch.equal(pv[b, g, :n_g], kv.v[b, g].index_select(0, rows))
            sels.append(s)
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, c["ns"], c["W"], sels)
        assert np.max(np.abs(np64(out_p[b]) - ref)) < OUT_TOL, b
