"""Context lengths held in device memory (the growing history of the decode
loop): kernels read each row's length when they run, sfi_kv_append advances
it on the device, and the host values are only the bounds the launches are
planned for.  Checked against the host-length path bit for bit when the bound
is exact, against the oracle when the bound is larger, and as a decode loop
with an append every step captured once per slow/fast pattern and replayed,
bit for bit against the same loop run eagerly."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
import synth
from synth import gen
from tests.gpu_helpers import OUT_TOL, check_mass, check_support, np64, random_cache

pytestmark = pytest.mark.gpu


def _buffers(kv, sp):
    dev = kv.k.device
    B, Hq, Hkv, D, k = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim, sp.top_k
    return dict(out=torch.full((B, Hq, D), float("nan"), device=dev),
                fast=torch.full((B, Hq, D), float("nan"), device=dev),
                gath=torch.full((B, Hq, D), float("nan"), device=dev),
                dense=torch.full((B, Hq, D), float("nan"), device=dev),
                mass=torch.full((B, Hkv, kv.capacity), -1.0, device=dev),
                sel=torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev),
                cnt=torch.zeros(B, Hkv, dtype=torch.int32, device=dev),
                pk=torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev),
                pv=torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev))


def _run_all(kv, sp, ids, q, ws):
    """The refresh with packing and the fast steps over its support, then the
    refresh without packing and the packing fast step over that support."""
    o = _buffers(kv, sp)
    S.sfi_slow_step_select(kv, sp, ids, q, o["out"], o["mass"], o["sel"], o["cnt"], o["pk"], o["pv"], ws)
    S.sfi_fast_step_packed(kv, sp, ids, q, o["pk"], o["pv"], o["cnt"], o["fast"], ws)
    S.sfi_fast_step(kv, sp, ids, q, o["sel"], o["cnt"], o["gath"], ws)
    S.sfi_slow_step(kv, ids, q, o["dense"], None, ws)
    d = _buffers(kv, sp)
    S.sfi_slow_step_select(kv, sp, ids, q, d["out"], d["mass"], d["sel"], d["cnt"], None, None, ws)
    S.sfi_fast_step_pack(kv, sp, ids, q, d["sel"], d["cnt"], d["fast"], d["pk"], d["pv"], ws)
    torch.cuda.synchronize()
    o.update({"d_" + key: d[key] for key in ("out", "mass", "sel", "cnt", "fast", "pk", "pv")})
    return o


def _same_both_packings(o):
    for key in ("out", "mass", "sel", "cnt", "pk", "pv"):
        assert torch.equal(o[key], o["d_" + key]), key
    assert torch.equal(o["d_fast"], o["gath"])


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_device_lengths_with_exact_bounds_equal_host_lengths(dtype):
    """Bounds equal to the device lengths: the same launch plans, so every
    output equals the host-length path's bit for bit (refresh, both fast
    steps, the dense step), on ragged rows including keep-all and
    no-candidate ones."""
    ctx = [9000, 2500, 300, 40]
    kv, q = random_cache(4, 16, 4, 9000, 128, dtype, ctx, seed=71, q_scale=2.0)
    sp = S.support_params(4, 64, 256, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = [0, 1, 2, 3]
    ref = _run_all(kv, sp, ids, q, ws)
    dev_ctx = torch.tensor(ctx, dtype=torch.int32, device=kv.k.device)
    kvd = S.KVDesc(kv.k, kv.v, ctx, kv.n_q_heads, ctx_dev=dev_ctx)
    got = _run_all(kvd, sp, ids, q, ws)
    for key in ref:
        assert torch.equal(ref[key], got[key]), key
    _same_both_packings(ref)


def test_device_lengths_below_their_bounds_match_the_oracle():
    """Bounds well above the device lengths (grids planned for the bound,
    surplus workgroups contribute nothing): every output against the oracle."""
    ctx = [9000, 2500, 300, 40]
    bound = [9800, 4000, 2000, 300]
    kv0, q = random_cache(4, 32, 8, 9800, 128, torch.bfloat16, bound, seed=72, q_scale=2.0)
    dev_ctx = torch.tensor(ctx, dtype=torch.int32, device=kv0.k.device)
    kv = S.KVDesc(kv0.k, kv0.v, bound, kv0.n_q_heads, ctx_dev=dev_ctx)
    ns, W, k, lam = 16, 256, 2048, 0.1
    sp = S.support_params(ns, W, k, lam)
    ws = S.alloc_workspace(kv, sp)
    ids = [0, 1, 2, 3]
    o = _run_all(kv, sp, ids, q, ws)
    assert torch.equal(o["fast"], o["gath"])
    _same_both_packings(o)
    for b, T in enumerate(ctx):
        K64, V64 = np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T])
        o_ref, P = O.dense_attention(np64(q[b]), K64, V64)
        f_ref = O.group_mass(P, kv.n_kv_heads)
        assert np.max(np.abs(np64(o["out"][b]) - o_ref)) < OUT_TOL, b
        assert np.max(np.abs(np64(o["dense"][b]) - o_ref)) < OUT_TOL, b
        check_mass(np64(o["mass"][b, :, :T]), f_ref, b)
        assert torch.all(o["mass"][b, :, T:] == -1.0), b      # nothing written past the length
        cnt = o["cnt"][b].cpu().numpy()
        sels = []
        for g in range(kv.n_kv_heads):
            s = o["sel"][b, g, :cnt[g]].cpu().numpy().astype(np.int64)
            check_support(s, f_ref[g], T, ns, W, k, lam, f"b{b} g{g}")
            sels.append(s)
        ref = O.fast_step(np64(q[b]), K64, V64, T, ns, W, sels)
        assert np.max(np.abs(np64(o["fast"][b]) - ref)) < OUT_TOL, b


def test_append_advances_device_lengths_and_skips_full_rows():
    """sfi_kv_append with device lengths writes row ctx_len[b], advances it by
    one, and leaves a full row (ctx_len[b] == capacity) unchanged."""
    kv0, _ = random_cache(3, 8, 2, 64, 64, torch.float32, [10, 63, 64], seed=73)
    dev = kv0.k.device
    dev_ctx = torch.tensor([10, 63, 64], dtype=torch.int32, device=dev)
    kv = S.KVDesc(kv0.k, kv0.v, [64, 64, 64], 8, ctx_dev=dev_ctx)
    before_k, before_v = kv.k.clone(), kv.v.clone()
    kn = torch.randn(3, 2, 64, device=dev)
    vn = torch.randn(3, 2, 64, device=dev)
    S.sfi_kv_append(kv, [0, 1, 2], kn, vn)
    torch.cuda.synchronize()
    assert dev_ctx.tolist() == [11, 64, 64]
    mask = torch.zeros(3, 2, 64, dtype=torch.bool, device=dev)
    mask[0, :, 10] = True
    mask[1, :, 63] = True
    assert torch.equal(kv.k[~mask], before_k[~mask]) and torch.equal(kv.v[~mask], before_v[~mask])
    assert torch.equal(kv.k[0, :, 10], kn[0]) and torch.equal(kv.v[1, :, 63], vn[1])


@pytest.mark.parametrize("packing", ["refresh", "deferred"])
def test_growing_history_layer_captured_once_and_replayed(packing):
    """One layer of the 32-layer loop (batch 4, 128K context growing by one
    token a step, k = 4096, window 512, its own span schedules): every decode
    step (append, refresh of the rows that open a span, one fast launch for
    the others) is captured once per row pattern and replayed across 20
    appends.  With deferred packing the refresh only selects and the fast
    launch packs the rows on their span's first fast step.  Each replayed
    step equals the same loop run eagerly, bit for bit, and sequence 0
    matches the oracle at the last steps."""
    w = synth.C5
    dev = torch.device("cuda:0")
    n_steps = 20
    sch = S.Scheduler(w.batch, w.seed, w.span_mode, w.span_param)
    plan = [sch.step() for _ in range(n_steps)]
    sch.close()
    flags = [[b in slow for slow, _ in plan] for b in range(w.batch)]
    span_ids = [gen.span_ids_from_flags(f) for f in flags]
    c = gen.build_cache(w, dev, layer=0)
    qs = gen.build_queries(w, dev, span_ids, c, layer=0)
    kn, vn = gen.append_rows(w, dev, layer=0, n_steps=n_steps)
    T0 = [int(x) for x in c["ctx_len"]]
    bound = [t + n_steps for t in T0]
    dev_ctx = torch.tensor(T0, dtype=torch.int32, device=dev)
    kv = S.KVDesc(c["K"], c["V"], bound, w.n_q_heads, ctx_dev=dev_ctx)
    sp = S.support_params(w.n_sink, w.n_recent, w.top_k, w.lam)
    ws = S.alloc_workspace(kv, sp)
    o = _buffers(kv, sp)
    q_buf = torch.empty_like(qs[0])
    kn_buf, vn_buf = torch.empty_like(kn[0]), torch.empty_like(vn[0])
    ids = list(range(w.batch))

    deferred = packing == "deferred"

    def step(slow, fast, first=()):
        S.sfi_kv_append(kv, ids, kn_buf, vn_buf)
        if slow:
            S.sfi_slow_step_select(kv, sp, list(slow), q_buf, o["out"], o["mass"], o["sel"], o["cnt"],
                                   None if deferred else o["pk"], None if deferred else o["pv"], ws)
        if fast and deferred and first:
            rows = sorted(fast)
            S.sfi_fast_step_pack(kv, sp, rows, q_buf, o["sel"], o["cnt"], o["out"], o["pk"], o["pv"], ws,
                                 pack_flags=[int(b in first) for b in rows])
        elif fast:
            S.sfi_fast_step_packed(kv, sp, list(fast), q_buf, o["pk"], o["pv"], o["cnt"], o["out"], ws)

    # rows on their span's first fast step (they refreshed the step before)
    firsts = [tuple(b for b in plan[t][1] if t > 0 and b in plan[t - 1][0]) for t in range(n_steps)]

    def stage(t):
        q_buf.copy_(qs[t])
        kn_buf.copy_(kn[t])
        vn_buf.copy_(vn[t])

    eager = []
    for t in range(n_steps):
        stage(t)
        step(*plan[t], firsts[t])
        eager.append(o["out"].clone())
    torch.cuda.synchronize()
    assert dev_ctx.tolist() == bound
    dev_ctx.copy_(torch.tensor(T0, dtype=torch.int32))
    graphs = {}
    for t in range(n_steps):
        key = (tuple(plan[t][0]), firsts[t] if deferred else ())
        if key not in graphs:
            torch.cuda.synchronize()
            gr = torch.cuda.CUDAGraph()
            with torch.cuda.graph(gr):
                step(*plan[t], firsts[t])
            graphs[key] = gr
        stage(t)
        o["out"].fill_(float("nan"))
        graphs[key].replay()
        torch.cuda.synchronize()
        assert torch.equal(o["out"], eager[t]), t
        if t >= n_steps - 2:
            T = int(dev_ctx[0])
            assert T == T0[0] + t + 1
            K64, V64 = np64(c["K"][0, :, :T]), np64(c["V"][0, :, :T])
            if 0 in plan[t][0]:
                o_ref, _ = O.dense_attention(np64(qs[t, 0]), K64, V64)
            else:
                cnt = o["cnt"][0].cpu().numpy()
                sels = [o["sel"][0, g, :cnt[g]].cpu().numpy().astype(np.int64) for g in range(w.n_kv_heads)]
                o_ref = O.fast_step(np64(qs[t, 0]), K64, V64, T, w.n_sink, w.n_recent, sels)
            assert np.max(np.abs(np64(o["out"][0]) - o_ref)) < OUT_TOL, t
    assert len(graphs) < n_steps  # patterns repeat: graphs are reused
