"""GPU parity of sfi_fast_step_pack, the fast step that also packs the rows it
reads (deferred packing: the first fast step of a span packs the support
instead of the refresh).  Its output equals sfi_fast_step's bit for bit, its
packed rows equal sfi_pack_support's, bit for bit, and sfi_fast_step_packed
over them equals the gather path; checked on ragged batches (one-row launches
that merge inside the kernel and multi-row launches that use the merge
kernel), with out-of-range indices, a keep-all selection under appends, and as
a replayed graph."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, np64, random_cache, run_slow

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _select(kv, sp, ids, q, ws):
    dev = kv.k.device
    _, mass = run_slow(kv, q, ids, ws=ws)
    sel = torch.full((kv.batch, kv.n_kv_heads, max(sp.top_k, 1)), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(kv.batch, kv.n_kv_heads, dtype=torch.int32, device=dev)
    S.sfi_select(kv, sp, ids, mass, sel, cnt, ws)
    return sel, cnt


def _packed_pair(kv, sp, fill):
    shape = (kv.batch, kv.n_kv_heads, sp.top_k, kv.head_dim)
    return (torch.full(shape, fill, dtype=kv.dtype, device=kv.k.device),
            torch.full(shape, fill, dtype=kv.dtype, device=kv.k.device))


def _check_three_ways(kv, sp, ids, q, sel, cnt, ws, packed_step=True):
    dev = kv.k.device
    B, Hq, D = kv.batch, kv.n_q_heads, kv.head_dim
    out_g = torch.full((B, Hq, D), 7.0, device=dev)
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_g, ws)
    out_d = torch.full((B, Hq, D), 7.0, device=dev)
    pk, pv = _packed_pair(kv, sp, 3.0)
    S.sfi_fast_step_pack(kv, sp, ids, q, sel, cnt, out_d, pk, pv, ws)
    rk, rv = _packed_pair(kv, sp, 3.0)
    S.sfi_pack_support(kv, sp, ids, sel, cnt, rk, rv)
    out_p = torch.full((B, Hq, D), 7.0, device=dev)
    S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, out_p, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_d, out_g)
    assert torch.equal(_bits(pk), _bits(rk)) and torch.equal(_bits(pv), _bits(rv))
    if packed_step:
        assert torch.equal(out_p, out_g)
    return out_g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
@pytest.mark.parametrize("one_row", [True, False])
def test_pack_step_equals_fast_step_and_pack_support(dtype, one_row):
    ctx = [9000, 2500, 300, 40, 20000]
    kv, q = random_cache(5, 16, 4, 20000, 128, dtype, ctx, seed=301, q_scale=2.0)
    sp = S.support_params(8, 128, 1024, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = [0, 1, 2, 3, 4]
    sel, cnt = _select(kv, sp, ids, q, ws)
    if one_row:
        out = torch.stack([_check_three_ways(kv, sp, [b], q, sel, cnt, ws)[b] for b in ids])
    else:
        out = _check_three_ways(kv, sp, ids, q, sel, cnt, ws)
    for b in ids:
        T = ctx[b]
        c = cnt[b].cpu().numpy()
        sels = [sel[b, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(kv.n_kv_heads)]
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, sp.n_sink, sp.n_recent, sels)
        assert np.max(np.abs(np64(out[b]) - ref)) < OUT_TOL, b


def test_pack_step_skips_indices_outside_the_context():
    """Caller-made selections with -1 and past-the-end indices: the gather path
    ignores them and the packing skips their slots, as sfi_pack_support does.
    (The packed step attends to every slot below the count, so it matches the
    gather path only for selections inside the context.)"""
    kv, q = random_cache(2, 8, 2, 5000, 128, torch.bfloat16, [5000, 3000], seed=303, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(4, 32, 200, 0.1)
    ws = S.alloc_workspace(kv, sp)
    g = torch.Generator(); g.manual_seed(304)
    sel = torch.randint(36, 2900, (2, 2, 200), generator=g, dtype=torch.int32).to(dev)
    sel, _ = torch.sort(sel, dim=-1)
    sel[0, 0, 10] = -1
    sel[1, 1, 50] = 4000        # past row 1's context
    sel[0, 1, 199] = 6000       # past the capacity
    cnt = torch.tensor([[200, 200], [150, 200]], dtype=torch.int32, device=dev)
    _check_three_ways(kv, sp, [0, 1], q, sel, cnt, ws, packed_step=False)


def test_pack_step_after_appends_with_keep_all_selection():
    """Keep-all selection at the slow step, then appends grow the context: the
    pack step packs exactly the selection's rows (slots past it untouched), and
    every later packed step equals the gather path."""
    T0, cap, k = 1500, 1600, 2048
    kv, q = random_cache(1, 32, 8, cap, 128, torch.bfloat16, [T0], seed=305, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    sel, cnt = _select(kv, sp, [0], q, ws)
    assert int(cnt.max()) == T0 - 16 - 256
    kn = torch.randn(1, 8, 128, device=dev).to(torch.bfloat16)
    S.sfi_kv_append(kv, [0], kn, kn.clone())
    kv.ctx += 1
    _check_three_ways(kv, sp, [0], q, sel, cnt, ws)


def test_pack_step_in_a_replayed_graph():
    """Captured once and replayed: the pack step rewrites the same packed rows
    and the same output every replay, with other fast steps in between."""
    kv, q = random_cache(1, 32, 8, 40000, 128, torch.bfloat16, [40000], seed=307, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, 2048, 0.1)
    ws = S.alloc_workspace(kv, sp)
    sel, cnt = _select(kv, sp, [0], q, ws)
    ref = _check_three_ways(kv, sp, [0], q, sel, cnt, ws)
    rk, rv = _packed_pair(kv, sp, 0.0)
    S.sfi_pack_support(kv, sp, [0], sel, cnt, rk, rv)
    pk, pv = _packed_pair(kv, sp, 0.0)
    out = torch.empty(1, 32, 128, device=dev)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        S.sfi_fast_step_pack(kv, sp, [0], q, sel, cnt, out, pk, pv, ws)
    for rep in range(4):
        pk.zero_(); pv.zero_(); out.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref[:1]) and torch.equal(_bits(pk), _bits(rk)) and torch.equal(_bits(pv), _bits(rv))
        S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref[:1]), rep


def _mixed_case(kv, sp, ids, q, flags, ws):
    """Rows flagged 1 gather and pack, rows flagged 0 read the packed rows an
    earlier sfi_pack_support wrote: the output equals the gather path's bit
    for bit, the flagged rows' packed rows equal sfi_pack_support's and the
    other rows' packed buffers are left as they were."""
    dev = kv.k.device
    B, Hq, D = kv.batch, kv.n_q_heads, kv.head_dim
    sel, cnt = _select(kv, sp, ids, q, ws)
    ref_k, ref_v = _packed_pair(kv, sp, 3.0)
    S.sfi_pack_support(kv, sp, ids, sel, cnt, ref_k, ref_v)
    pk, pv = _packed_pair(kv, sp, 3.0)
    for b, f in zip(ids, flags):
        if not f:  # the earlier pack of the rows past their span's first step
            pk[b].copy_(ref_k[b])
            pv[b].copy_(ref_v[b])
    before_k, before_v = pk.clone(), pv.clone()
    out_g = torch.full((B, Hq, D), 7.0, device=dev)
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_g, ws)
    out_m = torch.full((B, Hq, D), 7.0, device=dev)
    S.sfi_fast_step_pack(kv, sp, ids, q, sel, cnt, out_m, pk, pv, ws, pack_flags=flags)
    torch.cuda.synchronize()
    assert torch.equal(out_m, out_g)
    for b, f in zip(ids, flags):
        want_k, want_v = (ref_k[b], ref_v[b]) if f else (before_k[b], before_v[b])
        assert torch.equal(_bits(pk[b]), _bits(want_k)) and torch.equal(_bits(pv[b]), _bits(want_v)), b
    return out_g


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_mixed_rows_in_one_launch(dtype):
    """A ragged batch whose rows are at different points of their spans: one
    launch (merged inside the kernel) serves both kinds."""
    ctx = [9000, 2500, 300, 40, 20000]
    kv, q = random_cache(5, 16, 4, 20000, 128, dtype, ctx, seed=311, q_scale=2.0)
    sp = S.support_params(8, 128, 1024, 0.1)
    ws = S.alloc_workspace(kv, sp)
    out = _mixed_case(kv, sp, [0, 1, 2, 3, 4], q, [1, 0, 1, 0, 0], ws)
    for b in (0, 4):
        T = ctx[b]
        sel, cnt = _select(kv, sp, [b], q, ws)
        c = cnt[b].cpu().numpy()
        sels = [sel[b, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(kv.n_kv_heads)]
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, sp.n_sink, sp.n_recent, sels)
        assert np.max(np.abs(np64(out[b]) - ref)) < OUT_TOL, b


def test_mixed_rows_with_the_merge_kernel():
    """More workgroups than compute units: the chunk states go through the
    merge kernel; the listed order differs from the batch order."""
    B = 16
    ctx = [20000 - 900 * b for b in range(B)]
    kv, q = random_cache(B, 8, 2, 20000, 128, torch.bfloat16, ctx, seed=313, q_scale=2.0)
    sp = S.support_params(16, 256, 2048, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = [5, 0, 15, 3, 8, 1, 12, 7, 2, 9, 14, 4, 11, 6, 13, 10]
    assert sum(S.sfi_fast_plan(kv, sp, ids)) * kv.n_kv_heads > 256
    _mixed_case(kv, sp, ids, q, [(b * 7) % 3 == 0 for b in ids], ws)


def test_mixed_rows_over_several_launch_groups():
    """70 rows: the flags follow their rows into each launch group."""
    B = 70
    ctx = [300 + 37 * b for b in range(B)]
    kv, q = random_cache(B, 4, 2, 3000, 64, torch.bfloat16, ctx, seed=317, q_scale=2.0)
    sp = S.support_params(4, 32, 64, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = list(range(B))[::-1]
    _mixed_case(kv, sp, ids, q, [int(b % 3 == 1) for b in ids], ws)


@pytest.mark.parametrize("flag", [0, 1])
def test_uniform_flags_take_the_single_kind_kernels(flag):
    """All flags 0: the packed step's output and untouched buffers; all 1: the
    same as no flags."""
    ctx = [6000, 3000, 1200]
    kv, q = random_cache(3, 8, 2, 6000, 128, torch.bfloat16, ctx, seed=319, q_scale=2.0)
    sp = S.support_params(8, 64, 512, 0.1)
    ws = S.alloc_workspace(kv, sp)
    _mixed_case(kv, sp, [0, 1, 2], q, [flag] * 3, ws)


@pytest.mark.parametrize("lam", [0.0, 0.1, 1.0])
def test_selection_does_not_depend_on_the_launch(lam):
    """The Selector's output for a row does not depend on which rows share its
    launch (a batch larger than one pass of the CUs, or the row alone) nor on
    whether the refresh packs: bit for bit the same positions and counts."""
    B = 12
    ctx = [20000, 19000, 15000, 9000, 4500, 2400, 2300, 600, 20000, 11111, 8192, 16385]
    kv, q = random_cache(B, 16, 8, 20000, 64, torch.bfloat16, ctx, seed=331, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, 2048, lam)
    ws = S.alloc_workspace(kv, sp)
    ids = list(range(B))
    _, mass = run_slow(kv, q, ids, ws=ws)

    def sel_of(rows, packed):
        sel = torch.full((B, kv.n_kv_heads, sp.top_k), -7, dtype=torch.int32, device=dev)
        cnt = torch.full((B, kv.n_kv_heads), -7, dtype=torch.int32, device=dev)
        if packed:
            pk, pv = _packed_pair(kv, sp, 0.0)
            out = torch.empty(B, kv.n_q_heads, kv.head_dim, device=dev)
            m2 = torch.empty_like(mass)
            S.sfi_slow_step_select(kv, sp, rows, q, out, m2, sel, cnt, pk, pv, ws)
        else:
            S.sfi_select(kv, sp, rows, mass, sel, cnt, ws)
        torch.cuda.synchronize()
        return sel, cnt

    batch_sel, batch_cnt = sel_of(ids, False)
    pack_sel, pack_cnt = sel_of(ids, True)
    assert torch.equal(batch_sel, pack_sel) and torch.equal(batch_cnt, pack_cnt)
    for b in ids:
        one_sel, one_cnt = sel_of([b], False)
        assert torch.equal(one_sel[b], batch_sel[b]) and torch.equal(one_cnt[b], batch_cnt[b]), b
