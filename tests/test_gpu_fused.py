"""GPU parity of the fused slow-step + Selector + pack entry point: bit for bit
equal to the three separate calls it replaces, and within tolerance of the
oracle, on ragged multi-sequence batches and the Selector's edge cases."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, check_support, np64, oracle_slow, random_cache

pytestmark = pytest.mark.gpu

DT = {"f32": torch.float32, "bf16": torch.bfloat16}


def _outputs(kv, sp, packed):
    dev = kv.k.device
    B, Hq, Hkv, D, k = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim, sp.top_k
    o = dict(out=torch.full((B, Hq, D), 7.0, device=dev),
             mass=torch.full((B, Hkv, kv.capacity), -1.0, device=dev),
             sel=torch.full((B, Hkv, k), -7, dtype=torch.int32, device=dev),
             cnt=torch.full((B, Hkv), -7, dtype=torch.int32, device=dev))
    if packed:
        o["pk"] = torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev)
        o["pv"] = torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev)
    return o


def _separate(kv, sp, ids, q, ws, packed=True):
    o = _outputs(kv, sp, packed)
    S.sfi_slow_step(kv, ids, q, o["out"], o["mass"], ws)
    S.sfi_select(kv, sp, ids, o["mass"], o["sel"], o["cnt"], ws)
    if packed:
        S.sfi_pack_support(kv, sp, ids, o["sel"], o["cnt"], o["pk"], o["pv"])
    return o


def _fused(kv, sp, ids, q, ws, packed=True):
    o = _outputs(kv, sp, packed)
    S.sfi_slow_step_select(kv, sp, ids, q, o["out"], o["mass"], o["sel"], o["cnt"], o.get("pk"), o.get("pv"), ws)
    return o


def _assert_same(a, b):
    torch.cuda.synchronize()
    for key in a:
        assert torch.equal(a[key], b[key]), key


def _check_oracle(kv, sp, q, o, ids):
    for b in ids:
        T = int(kv.ctx[b])
        o_ref, f_ref = oracle_slow(kv, q, b)
        assert np.max(np.abs(np64(o["out"][b]) - o_ref)) < OUT_TOL
        for g in range(kv.n_kv_heads):
            c = int(o["cnt"][b, g])
            sel = o["sel"][b, g, :c].cpu().numpy()
            check_support(sel, f_ref[g], T, sp.n_sink, sp.n_recent, sp.top_k, sp.lambda_, f"b{b} g{g}")
            if "pk" in o and c > 0:
                rows = torch.from_numpy(sel.astype(np.int64)).to(kv.k.device)
                assert torch.equal(o["pk"][b, g, :c], kv.k[b, g].index_select(0, rows))
                assert torch.equal(o["pv"][b, g, :c], kv.v[b, g].index_select(0, rows))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("G", [1, 4, 8])
def test_fused_equals_separate_calls(dtype, D, G):
    """Ragged batch: a long context (top-k over several Selector chunks), a
    medium one, one with fewer candidates than k (keep-all) and one shorter
    than sinks + window (no candidates)."""
    Hkv = 2
    ctx = [9000, 2500, 300, 40]
    kv, q = random_cache(len(ctx), G * Hkv, Hkv, 9000, D, DT[dtype], ctx, seed=40 + G + D, q_scale=2.0)
    sp = S.support_params(4, 64, 256, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = [0, 1, 2, 3]
    a = _separate(kv, sp, ids, q, ws)
    b = _fused(kv, sp, ids, q, ws)
    _assert_same(a, b)
    _check_oracle(kv, sp, q, b, ids)


@pytest.mark.parametrize("lam", [0.0, 0.1, 1.0])
def test_fused_uniform_attention_ties(lam):
    """q = 0 gives every position the same mass, so with lambda = 0 all scores
    tie and the lowest positions must win; with lambda > 0 the prior decides
    (both ends of the candidate range)."""
    T, ns, W, k = 20000, 16, 256, 2048
    kv, q = random_cache(1, 32, 8, T, 128, torch.bfloat16, [T], seed=5)
    q.zero_()
    sp = S.support_params(ns, W, k, lam)
    ws = S.alloc_workspace(kv, sp)
    a = _separate(kv, sp, [0], q, ws)
    b = _fused(kv, sp, [0], q, ws)
    _assert_same(a, b)
    n = T - ns - W
    sel = b["sel"][0].cpu().numpy()
    if lam == 0.0:
        assert all(sel[g].tolist() == list(range(ns, ns + k)) for g in range(8))
    else:
        pos = (sel - ns + 1)
        want = list(range(1, k // 2 + 1)) + list(range(n - k // 2 + 1, n + 1))
        assert all(pos[g].tolist() == want for g in range(8))


def test_fused_consecutive_calls_and_subsets():
    """The Selector's bookkeeping in the workspace is left clean: calls on
    different row subsets and lengths, one after another on one workspace,
    each match the separate calls; unlisted rows stay untouched."""
    ctx = [7000, 12000, 5000]
    kv, q = random_cache(3, 32, 8, 12000, 128, torch.bfloat16, ctx, seed=9, q_scale=2.0)
    sp = S.support_params(16, 256, 1024, 0.1)
    ws = S.alloc_workspace(kv, sp)
    for ids in ([0, 1], [2], [1, 2, 0], [1]):
        a = _separate(kv, sp, ids, q, ws)
        b = _fused(kv, sp, ids, q, ws)
        _assert_same(a, b)
        for r in set(range(3)) - set(ids):
            assert torch.all(b["cnt"][r] == -7) and torch.all(b["mass"][r] == -1.0)
            assert torch.all(b["out"][r] == 7.0)
    _check_oracle(kv, sp, q, b, [1])


@pytest.mark.parametrize("k,packed", [(0, True), (5000, True), (512, False)])
def test_fused_degenerate_k_and_no_packing(k, packed):
    """top_k = 0 (nothing selected), top_k above the candidate count (keep
    all), and the call without packed buffers."""
    kv, q = random_cache(2, 16, 4, 4000, 64, torch.float32, [4000, 1000], seed=k, q_scale=2.0)
    sp = S.support_params(8, 32, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    a = _separate(kv, sp, [0, 1], q, ws, packed)
    b = _fused(kv, sp, [0, 1], q, ws, packed)
    _assert_same(a, b)
    _check_oracle(kv, sp, q, b, [0, 1])


# ------------------------------------------------------------------ two streams
def _async(kv, sp, ids, q, ws, main, side, o=None):
    o = o if o is not None else _outputs(kv, sp, True)
    S.sfi_slow_step_select_async(kv, sp, ids, q, o["out"], o["mass"], o["sel"], o["cnt"], o["pk"], o["pv"], ws,
                                 main, side)
    return o


def test_async_equals_fused():
    """The Selector on a second stream gives the single-stream results bit for
    bit (ragged batch: top-k over chunks, keep-all and no candidates)."""
    ctx = [9000, 2500, 300, 40]
    kv, q = random_cache(len(ctx), 32, 8, 9000, 128, torch.bfloat16, ctx, seed=77, q_scale=2.0)
    sp = S.support_params(16, 256, 512, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ref = _fused(kv, sp, [0, 1, 2, 3], q, ws)
    torch.cuda.synchronize()
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    ws2 = S.alloc_workspace(kv, sp)
    torch.cuda.synchronize()
    o = _async(kv, sp, [0, 1, 2, 3], q, ws2, main, side)
    _assert_same(ref, o)


def _layers(n, ctx, seed):
    layers = []
    for l in range(n):
        kv, q = random_cache(1, 32, 8, ctx, 128, torch.bfloat16, [ctx - 3 * l], seed=seed + l, q_scale=2.0)
        layers.append((kv, q))
    return layers


def _pipelined(layers, sp, ws, outs, main, side, done):
    """Layer l's slow step on `main`, its Selector on `side`; layer l + 2 reuses
    layer l's workspace and mass buffer, so it waits for layer l's Selector."""
    for l, (kv, q) in enumerate(layers):
        if l >= 2:
            main.wait_event(done[l - 2])
        o = outs[l]
        o["mass"] = outs[l % 2]["mass_buf"]
        S.sfi_slow_step_select_async(kv, sp, [0], q, o["out"], o["mass"], o["sel"], o["cnt"], o["pk"], o["pv"],
                                     ws[l % 2], main, side)
        done[l].record(side)
    main.wait_stream(side)


def test_async_pipelined_layers_and_graph_replay():
    """Six layers pipelined over two streams with double-buffered workspaces and
    mass buffers give each layer's single-stream results bit for bit, eagerly
    and as a captured graph replayed several times with eager work between."""
    layers = _layers(6, 12000, seed=300)
    sp = S.support_params(16, 256, 1024, 0.1)
    kv0 = layers[0][0]
    ws_ref = S.alloc_workspace(kv0, sp)
    refs = []
    for kv, q in layers:
        refs.append(_fused(kv, sp, [0], q, ws_ref))
    torch.cuda.synchronize()
    ws = [S.alloc_workspace(kv0, sp), S.alloc_workspace(kv0, sp)]
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    outs = [_outputs(kv, sp, True) for kv, _ in layers]
    for l in range(2):
        outs[l]["mass_buf"] = torch.full_like(outs[l]["mass"], -1.0)
    done = [torch.cuda.Event() for _ in layers]
    torch.cuda.synchronize()
    with torch.cuda.stream(main):
        _pipelined(layers, sp, ws, outs, main, side, done)
    torch.cuda.synchronize()
    for l in range(6):
        for key in ("out", "sel", "cnt", "pk", "pv"):
            assert torch.equal(outs[l][key], refs[l][key]), (l, key)
    for l in (4, 5):   # the mass buffers hold the last two layers'
        T = int(layers[l][0].ctx[0])
        assert torch.equal(outs[l % 2]["mass_buf"][..., :T], refs[l]["mass"][..., :T])

    # the same pipeline captured once and replayed
    g = torch.cuda.CUDAGraph()
    for o in outs:
        for key in ("out", "sel", "cnt", "pk", "pv"):
            o[key].fill_(0)
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=main):
        _pipelined(layers, sp, ws, outs, main, side, done)
    for rep in range(3):
        for o in outs:
            o["out"].fill_(float(rep))
            o["sel"].fill_(-9)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for l in range(6):
            for key in ("out", "sel", "cnt", "pk", "pv"):
                assert torch.equal(outs[l][key], refs[l][key]), (rep, l, key)


def test_more_rows_than_one_launch_group():
    """70 sequences (more than one launch group of 64): the fused, separate,
    two-stream and fast paths agree bit for bit, rows of both groups match the
    oracle, and unlisted rows stay untouched."""
    B = 70
    rng = np.random.default_rng(70)
    ctx = [int(x) for x in rng.integers(300, 2600, size=B)]
    kv, q = random_cache(B, 8, 2, 2600, 64, torch.bfloat16, ctx, seed=70, q_scale=2.0)
    sp = S.support_params(4, 32, 64, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = [b for b in range(B) if b != 5]          # row 5 unlisted
    a = _separate(kv, sp, ids, q, ws)
    b = _fused(kv, sp, ids, q, ws)
    _assert_same(a, b)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()
    ws2 = S.alloc_workspace(kv, sp)
    torch.cuda.synchronize()
    c = _async(kv, sp, ids, q, ws2, main, side)
    _assert_same(a, c)
    assert torch.all(b["cnt"][5] == -7) and torch.all(b["out"][5] == 7.0)
    _check_oracle(kv, sp, q, b, [0, 63, 64, 69])
    # fast steps over both launch groups: packed == gather, and the oracle
    out_p = torch.full_like(b["out"], 7.0)
    out_g = torch.full_like(b["out"], 7.0)
    S.sfi_fast_step_packed(kv, sp, ids, q, b["pk"], b["pv"], b["cnt"], out_p, ws)
    S.sfi_fast_step(kv, sp, ids, q, b["sel"], b["cnt"], out_g, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_p, out_g) and torch.all(out_p[5] == 7.0)
    for r in (1, 64, 68):
        T = ctx[r]
        c_ = b["cnt"][r].cpu().numpy()
        sels = [b["sel"][r, g, :c_[g]].cpu().numpy().astype(np.int64) for g in range(2)]
        ref = O.fast_step(np64(q[r]), np64(kv.k[r, :, :T]), np64(kv.v[r, :, :T]), T, 4, 32, sels)
        assert np.max(np.abs(np64(out_p[r]) - ref)) < OUT_TOL


def test_refresh_and_fast_rows_on_two_streams():
    """A layer's refresh rows and fast rows touch disjoint rows of every
    output: the fused refresh on one stream and the packed fast step on
    another, each with its own workspace and running side by side, give the
    serial results bit for bit, over several decode steps that alternate which
    rows refresh."""
    ctx = [6000, 3000, 9000, 700, 5000, 8000]
    B = len(ctx)
    kv, q = random_cache(B, 32, 8, 9000, 128, torch.bfloat16, ctx, seed=88, q_scale=2.0)
    sp = S.support_params(16, 256, 512, 0.1)
    qs = [q] + [(2 * torch.randn_like(q.float())).to(q.dtype) for _ in range(3)]
    plan = [(list(range(B)), []), ([1, 4], [0, 2, 3, 5]), ([0, 2, 3], [1, 4, 5]), ([5], [0, 1, 2, 3, 4])]

    def run(two_streams):
        ws, ws2 = S.alloc_workspace(kv, sp), S.alloc_workspace(kv, sp)
        o = _outputs(kv, sp, True)
        main, side = torch.cuda.current_stream(), torch.cuda.Stream()
        outs = []
        torch.cuda.synchronize()
        for qt, (slow, fast) in zip(qs, plan):
            fork = two_streams and slow and fast
            if fork:
                side.wait_stream(main)
            S.sfi_slow_step_select(kv, sp, slow, qt, o["out"], o["mass"], o["sel"], o["cnt"], o["pk"], o["pv"],
                                   ws2 if fork else ws, side if fork else main)
            if fast:
                S.sfi_fast_step_packed(kv, sp, fast, qt, o["pk"], o["pv"], o["cnt"], o["out"], ws, main)
            if fork:
                main.wait_stream(side)
            outs.append({key: v.clone() for key, v in o.items()})
        torch.cuda.synchronize()
        return outs

    serial, forked = run(False), run(True)
    for t, (a, b) in enumerate(zip(serial, forked)):
        for key in a:
            assert torch.equal(a[key], b[key]), (t, key)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_chunks_with_more_kept_rows_than_the_emit_prefetch(dtype, D):
    """top_k close to the candidate count: every 4096-candidate chunk keeps
    far more rows above the threshold bin than the emit pass prefetches
    (128 to 512 rows by row size), so the rest are copied after K*, beside
    the kept threshold-bin rows.  Equal to the separate calls bit for bit
    (positions and packed rows) and to the oracle."""
    ctx = [20000, 13000]
    kv, q = random_cache(2, 4 * 2, 2, 20000, D, DT[dtype], ctx, seed=611 + D, q_scale=3.0)
    sp = S.support_params(16, 256, 9000, 0.1)
    ws = S.alloc_workspace(kv, sp)
    a = _separate(kv, sp, [0, 1], q, ws)
    b = _fused(kv, sp, [0, 1], q, ws)
    _assert_same(a, b)
    _check_oracle(kv, sp, q, b, [0, 1])


def test_chunks_longer_than_one_emission_pass():
    """Over 4.19M candidates per head, so each Selector chunk spans more than
    one 4096-candidate pass and the emit pass recomputes the chunk's keys from
    the evidence (the path that also serves threshold bins larger than LDS).
    The fused refresh equals the separate calls bit for bit and the oracle's
    selection; the packed rows are the cache rows at the selected
    positions."""
    T = 4_300_000
    kv, q = random_cache(1, 4, 1, T, 64, torch.bfloat16, [T], seed=613, q_scale=3.0)
    sp = S.support_params(16, 256, 3000, 0.1)
    ws = S.alloc_workspace(kv, sp)
    a = _separate(kv, sp, [0], q, ws)
    b = _fused(kv, sp, [0], q, ws)
    _assert_same(a, b)
    _check_oracle(kv, sp, q, b, [0])
