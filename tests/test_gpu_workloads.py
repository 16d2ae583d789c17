"""GPU parity on the five synthetic workloads, in the launch configuration the
bench uses (the fused refresh, which selects; the span's first fast step,
which gathers and packs the support; the later fast steps over the packed
support): the full 64-step loop of the tiny fp32 case, sampled steps of the
larger ones (every output the oracle can afford is compared element by
element; the rest is checked through properties that hold at any size), and
HIP-graph replay against eager results."""
import numpy as np
import pytest
import torch

import oracle as O
import sparse_kv_attention_sfi_amd as S
import synth
from synth import gen
from tests.gpu_helpers import MASS_SUM_TOL, OUT_TOL, TRIPWIRE, check_mass, check_support, np64

pytestmark = pytest.mark.gpu


def _schedules(w, n_steps):
    """Host scheduler flags per sequence, checked against the oracle's."""
    sch = S.Scheduler(w.batch, w.seed, w.span_mode, w.span_param)
    flags = [[False] * n_steps for _ in range(w.batch)]
    for t in range(n_steps):
        slow, _ = sch.step()
        for b in slow:
            flags[b][t] = True
    for b in range(w.batch):
        assert flags[b] == O.schedule(w.span_mode, w.span_param, w.seed + b, n_steps), b
    return flags


class Runner:
    """Buffers and calls of one layer of a workload through the C ABI, in the
    bench's configuration: the fused refresh (slow step + Selector), the
    span's first fast step gathering its support and packing it
    (sfi_fast_step_pack) and the later fast steps over the packed support.
    The refresh that also packs, the separate calls and the gather fast step
    serve as cross-checks."""

    def __init__(self, w, kv):
        dev = kv.k.device
        self.w, self.kv = w, kv
        self.sp = S.support_params(w.n_sink, w.n_recent, w.top_k, w.lam)
        self.ws = S.alloc_workspace(kv, self.sp)
        B = w.batch
        self.out = torch.full((B, w.n_q_heads, w.head_dim), float("nan"), device=dev)
        self.mass = torch.full((B, w.n_kv_heads, kv.capacity), -1.0, device=dev)
        self.sel = torch.full((B, w.n_kv_heads, w.top_k), -1, dtype=torch.int32, device=dev)
        self.cnt = torch.zeros(B, w.n_kv_heads, dtype=torch.int32, device=dev)
        shape = (B, w.n_kv_heads, w.top_k, w.head_dim)
        self.pk = torch.full(shape, float("nan"), dtype=kv.dtype, device=dev)
        self.pv = torch.full(shape, float("nan"), dtype=kv.dtype, device=dev)
        self.to_pack = set()   # rows whose next fast step is the first of their span

    def slow(self, ids, q):
        if ids:
            S.sfi_slow_step_select(self.kv, self.sp, ids, q, self.out, self.mass, self.sel, self.cnt, None, None,
                                   self.ws)
            self.to_pack.update(ids)

    def slow_packing(self, ids, q):
        if ids:
            S.sfi_slow_step_select(self.kv, self.sp, ids, q, self.out, self.mass, self.sel, self.cnt, self.pk,
                                   self.pv, self.ws)
            self.to_pack.difference_update(ids)

    def slow_separate(self, ids, q):
        if ids:
            S.sfi_slow_step(self.kv, ids, q, self.out, self.mass, self.ws)
            S.sfi_select(self.kv, self.sp, ids, self.mass, self.sel, self.cnt, self.ws)
            S.sfi_pack_support(self.kv, self.sp, ids, self.sel, self.cnt, self.pk, self.pv)
            self.to_pack.difference_update(ids)

    def fast(self, ids, q):
        """One launch for the rows, as the bench makes it; returns the rows
        that packed."""
        ids = sorted(ids)
        first = [b for b in ids if b in self.to_pack]
        if first:
            S.sfi_fast_step_pack(self.kv, self.sp, ids, q, self.sel, self.cnt, self.out, self.pk, self.pv, self.ws,
                                 pack_flags=[int(b in self.to_pack) for b in ids])
            self.to_pack.difference_update(first)
        elif ids:
            S.sfi_fast_step_packed(self.kv, self.sp, ids, q, self.pk, self.pv, self.cnt, self.out, self.ws)
        return first

    def packed_rows_ok(self, b):
        """The rows the first fast step packed for row b equal sfi_pack_support's."""
        pk, pv = torch.zeros_like(self.pk), torch.zeros_like(self.pv)
        S.sfi_pack_support(self.kv, self.sp, [b], self.sel, self.cnt, pk, pv)
        torch.cuda.synchronize()
        for g in range(self.w.n_kv_heads):
            c = int(self.cnt[b, g])
            if not (torch.equal(self.pk[b, g, :c], pk[b, g, :c]) and torch.equal(self.pv[b, g, :c], pv[b, g, :c])):
                return False
        return True

    def fast_gather(self, ids, q):
        if ids:
            S.sfi_fast_step(self.kv, self.sp, ids, q, self.sel, self.cnt, self.out, self.ws)

    def state(self):
        return [x.clone() for x in (self.out, self.mass, self.sel, self.cnt, self.pk, self.pv)]

    def gpu_sel(self, b):
        cnt = self.cnt[b].cpu().numpy()
        sel = self.sel[b].cpu().numpy()
        return [sel[g, :cnt[g]].astype(np.int64) for g in range(self.w.n_kv_heads)]


def _check_slow(r, b, q_b, K64, V64, T):
    w = r.w
    o_ref, P = O.dense_attention(q_b, K64[:, :T], V64[:, :T])
    f_ref = O.group_mass(P, w.n_kv_heads)
    assert np.max(np.abs(np64(r.out[b]) - o_ref)) < OUT_TOL
    assert np.max(np.abs(np64(r.out[b]) - o_ref)) < TRIPWIRE
    check_mass(np64(r.mass[b, :, :T]), f_ref, b)
    kinds = [check_support(s, f_ref[g], T, w.n_sink, w.n_recent, w.top_k, w.lam, f"b{b} g{g}")
             for g, s in enumerate(r.gpu_sel(b))]
    return f_ref, kinds


def _check_properties(r, b, T):
    """Any-size properties of a slow step + select for rows not recomputed."""
    w = r.w
    f = r.mass[b, :, :T].double()
    assert torch.max(torch.abs(f.sum(dim=1) - 1.0)).item() < MASS_SUM_TOL
    assert torch.isfinite(r.out[b]).all()
    n = max(0, T - w.n_sink - w.n_recent)
    for g, s in enumerate(r.gpu_sel(b)):
        assert len(s) == min(w.top_k, n)
        assert np.all(np.diff(s) > 0) and (len(s) == 0 or (s[0] >= w.n_sink and s[-1] < T - w.n_recent))


def test_tiny_fp32_full_loop():
    """All 64 steps of the tiny case: slow steps against the oracle's dense step
    and Selector, fast steps against the oracle fed with the GPU's support; the
    planted positions of each span are reported as recall."""
    w = synth.C1
    dev = torch.device("cuda:0")
    flags = _schedules(w, w.n_steps)
    span_ids = [gen.span_ids_from_flags(flags[0])]
    c = gen.build_cache(w, dev, n_spans=span_ids[0][-1] + 1)
    q = gen.build_queries(w, dev, span_ids, c)
    kv = S.KVDesc(c["K"], c["V"], c["ctx_len"], w.n_q_heads)
    r = Runner(w, kv)
    T = w.ctx
    K64, V64 = np64(c["K"][0]), np64(c["V"][0])
    recalls, exact = [], 0
    for t in range(w.n_steps):
        if flags[0][t]:
            r.slow_separate([0], q[t])
            torch.cuda.synchronize()
            separate = r.state()
            r.slow_packing([0], q[t])
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip(r.state(), separate))   # fused == separate calls
            # the bench's refresh packs nothing: the span's first fast step does
            r.pk.fill_(float("nan"))
            r.pv.fill_(float("nan"))
            r.slow([0], q[t])
            torch.cuda.synchronize()
            assert all(torch.equal(a, b) for a, b in zip(r.state()[:4], separate[:4]))
            _, kinds = _check_slow(r, 0, np64(q[t, 0]), K64, V64, T)
            exact += kinds.count("exact")
            s_idx = span_ids[0][t]
            for g, s in enumerate(r.gpu_sel(0)):
                planted = set(c["planted"][0][g][s_idx].tolist())
                recalls.append(len(planted & set(s.tolist())) / len(planted))
        else:
            if r.fast([0], q[t]):
                assert r.packed_rows_ok(0)
            torch.cuda.synchronize()
            ref = O.fast_step(np64(q[t, 0]), K64, V64, T, w.n_sink, w.n_recent, r.gpu_sel(0))
            assert np.max(np.abs(np64(r.out[0]) - ref)) < OUT_TOL
            packed_out = r.out.clone()
            r.fast_gather([0], q[t])
            torch.cuda.synchronize()
            assert torch.equal(r.out, packed_out)
    assert exact >= 1                       # supports with clear gaps match bit for bit
    assert np.mean(recalls) > 0.9


@pytest.mark.parametrize("wname,n_fast", [("C2", 3), ("C3", 2)])
def test_8b_layer_sampled_steps(wname, n_fast):
    """The 32K and 128K layers at full size: the first slow step and the next
    fast steps, every output against the oracle."""
    w = getattr(synth, wname)
    dev = torch.device("cuda:0")
    n_steps = 1 + n_fast
    flags = _schedules(w, 64)
    span_ids = [gen.span_ids_from_flags(flags[0])]
    c = gen.build_cache(w, dev)
    q = gen.build_queries(w, dev, span_ids, c)
    kv = S.KVDesc(c["K"], c["V"], c["ctx_len"], w.n_q_heads)
    r = Runner(w, kv)
    T = w.ctx
    K64, V64 = np64(c["K"][0]), np64(c["V"][0])
    ora_sels = None
    for t in range(n_steps):
        if flags[0][t]:
            r.slow([0], q[t])
            torch.cuda.synchronize()
            f_ref, kinds = _check_slow(r, 0, np64(q[t, 0]), K64, V64, T)
            ora_sels = [O.select(f_ref[g], T, w.n_sink, w.n_recent, w.top_k, w.lam)[0]
                        for g in range(w.n_kv_heads)]
        else:
            if r.fast([0], q[t]):
                assert r.packed_rows_ok(0)
            torch.cuda.synchronize()
            gpu = np64(r.out[0])
            packed_out = r.out.clone()
            r.fast_gather([0], q[t])
            torch.cuda.synchronize()
            assert torch.equal(r.out, packed_out)
            ref = O.fast_step(np64(q[t, 0]), K64, V64, T, w.n_sink, w.n_recent, r.gpu_sel(0))
            assert np.max(np.abs(gpu - ref)) < OUT_TOL
            assert np.max(np.abs(gpu - ref)) < TRIPWIRE
            # with the oracle's own support (differs only at near-ties)
            ref2 = O.fast_step(np64(q[t, 0]), K64, V64, T, w.n_sink, w.n_recent, ora_sels)
            assert np.max(np.abs(gpu - ref2)) < OUT_TOL


def test_batch16_mixed_steps():
    """Batch 16 with contexts in [8192, 65536]: step 0 (all slow) and the first
    steps in which slow and fast sequences mix.  Four sequences are checked
    against the oracle element by element, the rest through properties."""
    w = synth.C4
    dev = torch.device("cuda:0")
    flags = _schedules(w, 40)
    span_ids = [gen.span_ids_from_flags(f) for f in flags]
    c = gen.build_cache(w, dev)
    q = gen.build_queries(w, dev, span_ids, c)
    kv = S.KVDesc(c["K"], c["V"], c["ctx_len"], w.n_q_heads)
    r = Runner(w, kv)
    ctx = c["ctx_len"]
    check = [int(np.argmin(ctx)), int(np.argmax(ctx)), 3, 11]
    mixed = next(t for t in range(1, 40) if 0 < sum(f[t] for f in flags) < w.batch)
    for t in (0, mixed):
        slow = [b for b in range(w.batch) if flags[b][t]]
        fast = [b for b in range(w.batch) if not flags[b][t]]
        r.slow(slow, q[t])
        r.fast(fast, q[t])
        torch.cuda.synchronize()
        for b in range(w.batch):
            T = ctx[b]
            if b in check:
                K64, V64 = np64(c["K"][b, :, :T]), np64(c["V"][b, :, :T])
                if b in slow:
                    _check_slow(r, b, np64(q[t, b]), K64, V64, T)
                else:
                    ref = O.fast_step(np64(q[t, b]), K64, V64, T, w.n_sink, w.n_recent, r.gpu_sel(b))
                    assert np.max(np.abs(np64(r.out[b]) - ref)) < OUT_TOL
            elif b in slow:
                _check_properties(r, b, T)


def test_growing_history_one_layer():
    """One layer of the 32-layer loop (batch 4, 128K context, k = 4096, window
    512) with a KV append before every step; sequence 0 is checked against the
    oracle, the others through properties."""
    w = synth.C5
    dev = torch.device("cuda:0")
    n_steps = 3
    flags = _schedules(w, n_steps)
    span_ids = [gen.span_ids_from_flags(f) for f in flags]
    c = gen.build_cache(w, dev, layer=0)
    q = gen.build_queries(w, dev, span_ids, c, layer=0)
    kn, vn = gen.append_rows(w, dev, layer=0, n_steps=n_steps)
    kv = S.KVDesc(c["K"], c["V"], c["ctx_len"], w.n_q_heads)
    r = Runner(w, kv)
    ids = list(range(w.batch))
    for t in range(n_steps):
        S.sfi_kv_append(kv, ids, kn[t], vn[t])
        kv.ctx += 1
        slow = [b for b in ids if flags[b][t]]
        fast = [b for b in ids if not flags[b][t]]
        r.slow(slow, q[t])
        r.fast(fast, q[t])
        torch.cuda.synchronize()
        T = int(kv.ctx[0])
        assert torch.equal(c["K"][0, :, T - 1], kn[t, 0])
        K64, V64 = np64(c["K"][0, :, :T]), np64(c["V"][0, :, :T])
        if 0 in slow:
            _check_slow(r, 0, np64(q[t, 0]), K64, V64, T)
        else:
            ref = O.fast_step(np64(q[t, 0]), K64, V64, T, w.n_sink, w.n_recent, r.gpu_sel(0))
            assert np.max(np.abs(np64(r.out[0]) - ref)) < OUT_TOL
        for b in slow:
            if b != 0:
                _check_properties(r, b, int(kv.ctx[b]))


def test_graph_replay_matches_eager():
    """Slow+select and fast steps captured in HIP graphs and replayed several
    times with new queries, eager work and synchronisation between replays;
    every replay equals the eager result bit for bit."""
    dev = torch.device("cuda:0")
    B, Hq, Hkv, D, T = 2, 32, 8, 128, 9000
    g = torch.Generator(device=dev)
    g.manual_seed(77)
    K = torch.randn(B, Hkv, T, D, generator=g, device=dev).to(torch.bfloat16)
    V = torch.randn(B, Hkv, T, D, generator=g, device=dev).to(torch.bfloat16)
    kv = S.KVDesc(K, V, [T, T - 1000], Hq)
    sp = S.support_params(16, 256, 512, 0.1)
    ws = S.alloc_workspace(kv, sp)
    q_buf = torch.empty(B, Hq, D, dtype=torch.bfloat16, device=dev)
    out = torch.empty(B, Hq, D, device=dev)
    mass = torch.empty(B, Hkv, T, device=dev)
    sel = torch.empty(B, Hkv, 512, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, Hkv, dtype=torch.int32, device=dev)

    pk = torch.empty(B, Hkv, 512, D, dtype=torch.bfloat16, device=dev)
    pv = torch.empty_like(pk)

    def slow():
        S.sfi_slow_step_select(kv, sp, [0, 1], q_buf, out, mass, sel, cnt, pk, pv, ws)

    def fast():
        S.sfi_fast_step(kv, sp, [0, 1], q_buf, sel, cnt, out, ws)

    def pack_fast():
        S.sfi_pack_support(kv, sp, [0, 1], sel, cnt, pk, pv)
        S.sfi_fast_step_packed(kv, sp, [0, 1], q_buf, pk, pv, cnt, out, ws)

    qs = [(2 * torch.randn(B, Hq, D, generator=g, device=dev)).to(torch.bfloat16) for _ in range(4)]
    q_buf.copy_(qs[0])
    slow()
    fast()
    torch.cuda.synchronize()
    graphs = []
    for fn in (slow, fast, pack_fast):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            fn()
        graphs.append(gr)
    for rep in range(3):
        for qi in qs:
            q_buf.copy_(qi)
            slow()
            torch.cuda.synchronize()
            ref = (out.clone(), mass.clone(), sel.clone(), cnt.clone())
            fast()
            torch.cuda.synchronize()
            ref_fast = out.clone()
            out.fill_(float("nan"))
            sel.fill_(-5)
            torch.cuda.synchronize()
            graphs[0].replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref[0]) and torch.equal(mass, ref[1])
            assert torch.equal(sel, ref[2]) and torch.equal(cnt, ref[3])
            graphs[1].replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_fast), rep
            out.fill_(float("nan"))
            graphs[2].replay()
            torch.cuda.synchronize()
            assert torch.equal(out, ref_fast), rep
