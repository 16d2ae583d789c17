"""The fast step that allocates nothing (sfi_fast_step_packed_noalloc, whose
chunk states live in the library's fixed per-device scratch) against the
workspace entry point it mirrors, sfi_fast_step_packed: the same bits on
consecutive calls of different sizes, through both merge paths, eagerly and
replayed from a HIP graph, and the oracle's result."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
from tests.gpu_helpers import OUT_TOL, np64, random_cache

pytestmark = pytest.mark.gpu


def _refresh(kv, sp, ids, q):
    dev = kv.k.device
    B, Hq, Hkv, D, k = kv.batch, kv.n_q_heads, kv.n_kv_heads, kv.head_dim, sp.top_k
    ws = S.alloc_workspace(kv, sp)
    out = torch.empty(B, Hq, D, device=dev)
    mass = torch.empty(B, Hkv, kv.capacity, device=dev)
    sel = torch.full((B, Hkv, k), -1, dtype=torch.int32, device=dev)
    cnt = torch.zeros(B, Hkv, dtype=torch.int32, device=dev)
    pk = torch.zeros(B, Hkv, k, D, dtype=kv.dtype, device=dev)
    pv = torch.zeros_like(pk)
    S.sfi_slow_step_select(kv, sp, ids, q, out, mass, sel, cnt, pk, pv, ws)
    return ws, sel, cnt, pk, pv


def _both(kv, sp, ids, q, ws, pk, pv, cnt):
    a = torch.full((kv.batch, kv.n_q_heads, kv.head_dim), float("nan"), device=kv.k.device)
    b = torch.full_like(a, float("nan"))
    S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, a, ws)
    S.sfi_fast_step_packed_noalloc(kv, sp, ids, q, pk, pv, cnt, b)
    torch.cuda.synchronize()
    return a, b


def _oracle_check(kv, sp, ids, q, sel, cnt, out):
    for b in ids:
        T = int(kv.ctx[b])
        c = cnt[b].cpu().numpy()
        sels = [sel[b, g, :c[g]].cpu().numpy().astype(np.int64) for g in range(kv.n_kv_heads)]
        ref = O.fast_step(np64(q[b]), np64(kv.k[b, :, :T]), np64(kv.v[b, :, :T]), T, sp.n_sink, sp.n_recent, sels)
        assert np.max(np.abs(np64(out[b]) - ref)) < OUT_TOL, b


def test_noalloc_equals_workspace_entry_point_twice_then_smaller():
    """Two calls in a row, the second with a smaller input (one row, a
    shorter context, a smaller support): each equals the workspace call bit
    for bit and matches the oracle."""
    ctx = [30000, 21000]
    kv, q = random_cache(2, 32, 8, 30000, 128, torch.bfloat16, ctx, seed=61, q_scale=2.0)
    sp = S.support_params(16, 256, 2048, 0.1)
    ws, sel, cnt, pk, pv = _refresh(kv, sp, [0, 1], q)
    for rep in range(2):
        a, b = _both(kv, sp, [0, 1], q, ws, pk, pv, cnt)
        assert torch.equal(a, b), rep
    _oracle_check(kv, sp, [0, 1], q, sel, cnt, b)
    kv2, q2 = random_cache(1, 16, 4, 5000, 64, torch.float32, [4000], seed=62, q_scale=2.0)
    sp2 = S.support_params(4, 64, 256, 0.1)
    ws2, sel2, cnt2, pk2, pv2 = _refresh(kv2, sp2, [0], q2)
    a, b = _both(kv2, sp2, [0], q2, ws2, pk2, pv2, cnt2)
    assert torch.equal(a, b)
    _oracle_check(kv2, sp2, [0], q2, sel2, cnt2, b)


def test_noalloc_merge_kernel_path_and_graph_replay():
    """More workgroups than the GPU has CUs (chunk states handed to the merge
    kernel through the fixed scratch), then the one-pass launch captured in a
    graph and replayed with eager calls in between."""
    ctx = [12000, 11000, 9000, 8000]
    kv, q = random_cache(4, 32, 8, 12000, 128, torch.bfloat16, ctx, seed=63, q_scale=2.0)
    sp = S.support_params(16, 256, 2048, 0.1)
    ids = [0, 1, 2, 3]
    ws, sel, cnt, pk, pv = _refresh(kv, sp, ids, q)
    a, b = _both(kv, sp, ids, q, ws, pk, pv, cnt)
    assert torch.equal(a, b)
    _oracle_check(kv, sp, ids, q, sel, cnt, b)
    out = torch.empty_like(a)
    ref = torch.empty_like(a)
    S.sfi_fast_step_packed(kv, sp, [2], q, pk, pv, cnt, ref, ws)
    S.sfi_fast_step_packed_noalloc(kv, sp, [2], q, pk, pv, cnt, out)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        S.sfi_fast_step_packed_noalloc(kv, sp, [2], q, pk, pv, cnt, out)
    for rep in range(4):
        out.fill_(float("nan"))
        gr.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[2], ref[2]), rep
        S.sfi_fast_step_packed_noalloc(kv, sp, [0, 1], q, pk, pv, cnt, out)
        torch.cuda.synchronize()
        assert torch.equal(out[:2], a[:2]), rep
