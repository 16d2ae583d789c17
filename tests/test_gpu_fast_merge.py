"""GPU parity of the fast step's merge of its support chunks, both where it
runs inside the fast-step kernel (the last workgroup of each (sequence, KV
head) to finish merges the published chunk states) and where the merge kernel
does it.  Checked against the oracle across many consecutive calls on one
workspace (so the per-head chunk counters must come back to zero), with chunk
counts from 1 to the largest, bit for bit between the two merge paths, and for
stale packed slots that the current selection does not cover."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, np64, random_cache, run_slow

pytestmark = pytest.mark.gpu


def _select(kv, sp, ids, q, ws):
    dev = kv.k.device
    _, mass = run_slow(kv, q, ids, ws=ws)
    sel = torch.full((kv.batch, kv.n_kv_heads, max(sp.top_k, 1)), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(kv.batch, kv.n_kv_heads, dtype=torch.int32, device=dev)
    S.sfi_select(kv, sp, ids, mass, sel, cnt, ws)
    return sel, cnt


def _oracle_fast(kv, q, b, sp, sel, cnt):
    T = int(kv.ctx[b])
    c = cnt[b].cpu().numpy()
    sels = [sel[b, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(kv.n_kv_heads)]
    return O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, sp.n_sink, sp.n_recent, sels)


def test_keep_all_selection_then_appends_with_stale_packed_slots():
    """The slow step keeps every candidate (n <= top_k); appends then grow the
    context, so the fast step may take more selected rows than the span's
    selection wrote.  Packed slots past the selection hold NaN: the packed
    fast step must ignore them, give the gather step's bits and match the
    oracle."""
    Hq, Hkv, D, T0, cap, k = 32, 8, 128, 1500, 1600, 2048
    kv, q = random_cache(1, Hq, Hkv, cap, D, torch.bfloat16, [T0], seed=91, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, k, 0.1)
    ws = S.alloc_workspace(kv, sp)
    sel, cnt = _select(kv, sp, [0], q, ws)
    assert int(cnt.max()) == T0 - 16 - 256  # keep-all
    pk = torch.full((1, Hkv, k, D), float("nan"), dtype=torch.bfloat16, device=dev)
    pv = torch.full_like(pk, float("nan"))
    S.sfi_pack_support(kv, sp, [0], sel, cnt, pk, pv)
    for step in range(6):
        kn = torch.randn(1, Hkv, D, device=dev).to(torch.bfloat16)
        vn = torch.randn(1, Hkv, D, device=dev).to(torch.bfloat16)
        S.sfi_kv_append(kv, [0], kn, vn)
        kv.ctx += 1
        out_p = torch.full((1, Hq, D), float("nan"), device=dev)
        out_g = torch.full_like(out_p, float("nan"))
        S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out_p, ws)
        S.sfi_fast_step(kv, sp, [0], q, sel, cnt, out_g, ws)
        torch.cuda.synchronize()
        assert torch.isfinite(out_p).all(), step
        assert torch.equal(out_p, out_g), step
        ref = _oracle_fast(kv, q, 0, sp, sel, cnt)
        assert np.max(np.abs(np64(out_p[0]) - ref)) < OUT_TOL, step


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_consecutive_calls_with_changing_chunk_counts(dtype):
    """One workspace, many fast steps in a row whose supports span 1 chunk,
    a few chunks and hundreds of chunks, over ragged rows: each result matches
    the oracle, so every call found its chunk counters at zero."""
    Hq, Hkv, D = 16, 4, 128
    ctx = [70000, 9000, 300, 20]
    B = len(ctx)
    kv, q = random_cache(B, Hq, Hkv, max(ctx), D, dtype, ctx, seed=17, q_scale=2.0)
    dev = kv.k.device
    big = S.support_params(16, 256, 40000, 0.1)
    ws = S.alloc_workspace(kv, big)
    plans = [S.support_params(2, 8, 16, 0.1), S.support_params(16, 256, 2048, 0.1), big,
             S.support_params(4, 64, 256, 0.5), S.support_params(16, 256, 2048, 0.1)]
    # all rows in one launch (more workgroups than CUs: merge kernel) and one
    # row per launch (mostly fits the GPU: merge inside the kernel)
    for ids_list in ([list(range(B))], [[b] for b in range(B)]):
        for rep in range(2):
            for i, sp in enumerate(plans):
                for ids in ids_list:
                    sel, cnt = _select(kv, sp, ids, q, ws)
                    chunks = S.sfi_fast_plan(kv, sp, ids)
                    out = torch.full((B, Hq, D), float("nan"), device=dev)
                    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out, ws)
                    torch.cuda.synchronize()
                    for j, b in enumerate(ids):
                        ref = _oracle_fast(kv, q, b, sp, sel, cnt)
                        err = np.max(np.abs(np64(out[b]) - ref))
                        assert err < OUT_TOL, (rep, i, b, chunks[j], err)


def test_single_row_launch_repeated_and_replayed():
    """The one-row launch (its row table entry at fixed argument offsets):
    the same fast step called eagerly and replayed from a graph many times in
    a row gives the same bits every time, and the oracle's result."""
    Hq, Hkv, D, T = 32, 8, 128, 40000
    kv, q = random_cache(1, Hq, Hkv, T, D, torch.bfloat16, [T], seed=23, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, 2048, 0.1)
    ws = S.alloc_workspace(kv, sp)
    sel, cnt = _select(kv, sp, [0], q, ws)
    pk = torch.empty(1, Hkv, 2048, D, dtype=torch.bfloat16, device=dev)
    pv = torch.empty_like(pk)
    S.sfi_pack_support(kv, sp, [0], sel, cnt, pk, pv)
    out = torch.empty(1, Hq, D, device=dev)
    S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out, ws)
    torch.cuda.synchronize()
    ref_bits = out.clone()
    ref = _oracle_fast(kv, q, 0, sp, sel, cnt)
    assert np.max(np.abs(np64(out[0]) - ref)) < OUT_TOL
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        for _ in range(4):
            S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out, ws)
    for rep in range(5):
        out.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_bits), rep
        for _ in range(3):
            S.sfi_fast_step_packed(kv, sp, [0], q, pk, pv, cnt, out, ws)
        torch.cuda.synchronize()
        assert torch.equal(out, ref_bits), rep


def test_merge_inside_kernel_equals_merge_kernel():
    """The same rows merged inside the fast-step kernel (one row per launch)
    and by the merge kernel (all rows in one launch, more workgroups than the
    GPU has CUs) give the same bits."""
    Hq, Hkv, D, T = 32, 8, 128, 20000
    B = 6
    kv, q = random_cache(B, Hq, Hkv, T, D, torch.bfloat16, [T - 997 * b for b in range(B)], seed=29, q_scale=2.0)
    dev = kv.k.device
    sp = S.support_params(16, 256, 2048, 0.1)
    ws = S.alloc_workspace(kv, sp)
    ids = list(range(B))
    sel, cnt = _select(kv, sp, ids, q, ws)
    out_all = torch.full((B, Hq, D), float("nan"), device=dev)
    S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out_all, ws)
    out_one = torch.full_like(out_all, float("nan"))
    for b in ids:
        S.sfi_fast_step(kv, sp, [b], q, sel, cnt, out_one, ws)
    torch.cuda.synchronize()
    assert torch.equal(out_all, out_one)
