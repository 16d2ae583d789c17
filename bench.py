#!/usr/bin/env python3
"""Decode-attention throughput of the SFI path on one MI355X.

Workload (default): the 8B-shaped layer at 128K context, batch 1, bf16 KV,
32 query / 8 KV heads, head_dim 128, 16 sinks + 256 recent + top-2048,
lambda 0.1, spans geometric with mean 18 drawn by the boundary scheduler.
Every decode step runs that layer shape over ``--layers`` independent
caches (128 by default: four 32-layer stacks' worth), so none of a layer's KV
rows or support (9.5 MB per fast step) is still in L2 or the 256 MB
last-level cache at its next step; a timed cold-cache check (each call after
a 1 GiB read) confirms the kernel times.

A "step" is one decode step over all layers: for every layer either the slow
path (dense split-K attention + mass + Selector) or the fast path (sparse
attention over the support), as the scheduler says; the first fast step of a
span gathers the selected rows by index and packs them, the later ones read
the packed rows (``--pack refresh`` packs in the refresh instead;
``--slow async`` runs each layer's Selector on a second stream under the next
layer's slow attention, the pages' asynchronous layer pipeline, slower than
one stream on this attention-only loop).  ``value`` = K * layers / wall time
of K steps (decode steps per second per layer), with inputs resident in HBM.
Each step's queries are staged into fixed buffers and the step is replayed as
a HIP graph (one each for slow steps, first fast steps and other fast steps).

Also reported: the blended rate over the workload's whole span schedule
(``full_schedule``, at the schedule's own slow fraction, beside
``slow_fraction_timed`` of the --steps window), per-kernel average durations
from HIP events recorded by the library around its launches (eager pass over
the same steps), the roofline of the dominant kernel, the dense-every-step
baseline, the CPU oracle's per-operation medians on the same workload, and
(``configs``) SFI against dense decode over the whole schedule of every other
workload: the 32K layer, the batch of 16 mixed contexts and the 32-layer
growing-history loop, each replayed from graphs captured per slow/fast row
pattern.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "c3_128k_layer_traffic.json")


def csrc_digest():
    """Digest of the library's code (comments and whitespace left out);
    counter readings apply only to kernels built from the code they were
    taken on."""
    import hashlib
    import re
    d = os.path.join(ROOT, "sparse_kv_attention_sfi_amd", "csrc")
    h = hashlib.sha256()
    for f in sorted(os.listdir(d)):
        if f.endswith((".hip", ".hpp", ".cpp")):
            with open(os.path.join(d, f)) as fh:
                text = fh.read()
            text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
            text = re.sub(r"//[^\n]*", " ", text)
            h.update(f.encode())
            h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def kernel_group(name):
    """Bench kernel name of a device kernel (the Selector's kernels form one group)."""
    if "fast_partial_kernel<" in name and name.split(">")[0].rsplit(",", 1)[-1].strip() not in ("0", "false"):
        return "fast_pack"  # the gather step's packing variants (last template argument: when it packs)
    for key, group in (("slow_partial", "slow_partial"), ("slow_combine", "slow_combine"), ("select_", "select"),
                       ("pack_kernel", "pack"), ("fast_packed", "fast_partial"), ("fast_partial", "fast_partial"),
                       ("fast_merge", "fast_merge")):
        if key in name:
            return group
    return None


def measured_traffic(group, workload_name):
    """Scaled FETCH_SIZE + WRITE_SIZE bytes per launch of a kernel group, if
    the committed counter summary matches the current kernel sources."""
    if workload_name != "C3-8B-layer-128K" or not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as fh:
        t = json.load(fh)
    if t.get("csrc_digest") != csrc_digest():
        return None
    ks = [k for k in t["kernels"].values() if k.get("group") == group]
    if not ks:
        return None
    return sum(k.get("fetch_bytes", 0.0) + k.get("write_bytes", 0.0) for k in ks)
METRIC = "decode-attn steps/sec/layer (slow, fast, blended) + HBM GB/s frac @128K ctx"


def traffic_rate(traffic, avg_us):
    """Measured HBM bytes per launch over the launch's average duration (the
    DRAM-side rate, beside the algorithmic-byte rate), or nothing."""
    if traffic is None or not avg_us:
        return {}
    gbps = traffic / (avg_us * 1e-6) / 1e9
    return {"traffic_GBps": gbps, "traffic_frac": gbps / HBM_PEAK_GBS}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=1024)
    p.add_argument("--warmup", type=int, default=64)
    p.add_argument("--workload", default="C3")
    p.add_argument("--layers", type=int, default=128,
                   help="independent layer caches cycled per decode step (128: a layer's fast-step data, "
                        "9.5 MB, is never still in the 256 MB last-level cache at its next step)")
    p.add_argument("--dense-steps", type=int, default=64)
    p.add_argument("--eager-steps", type=int, default=128)
    p.add_argument("--mode", choices=["graph", "eager"], default="graph")
    p.add_argument("--fast", choices=["packed", "gather"], default="packed",
                   help="fast step over the packed support (default) or gathering rows by index")
    p.add_argument("--pack", choices=["deferred", "refresh"], default="deferred",
                   help="where the selected rows are packed: by the first fast step of each span "
                        "(sfi_fast_step_pack, default), which reads them anyway, or in the refresh's emission pass")
    p.add_argument("--slow", choices=["fused", "async", "separate"], default="fused",
                   help="slow step + Selector (+ pack): fused on one stream (default), fused with the Selector on a "
                        "second stream under the next layer's slow step, or as separate calls")
    p.add_argument("--async-depth", type=int, default=4,
                   help="layers whose Selector may still run when a later layer's slow step starts (--slow async)")
    p.add_argument("--cold-checks", type=int, default=16,
                   help="calls of the slow and the fast path timed after a 1 GiB cache flush (0: skip)")
    p.add_argument("--batched-caches", type=int, default=8,
                   help="independent layer caches cycled per step for single-layer batched workloads (C4)")
    p.add_argument("--batch-check", type=int, default=16, metavar="B",
                   help="also time the fast step for B sequences in one launch (0: skip)")
    p.add_argument("--graph-reps", type=int, default=16,
                   help="replays of each step kind's graph timed alone (per-layer cost of each kind; 0: skip)")
    p.add_argument("--no-cpu", action="store_true")
    p.add_argument("--no-full-schedule", action="store_true",
                   help="skip the replay of the whole span schedule (its blended rate is then null)")
    p.add_argument("--no-configs", action="store_true",
                   help="skip the per-workload block (32K layer, batch 16, 32-layer growing history)")
    p.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                   help="end with one device copy of MIB MiB (calibrates memory-traffic counters)")
    p.add_argument("--stream-probe", type=int, default=2048, metavar="MIB",
                   help="time a device copy of MIB MiB on the same GPU, for the slow partial's bandwidth as a "
                        "fraction of a plain streaming copy (0: skip)")
    p.add_argument("--traffic-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                   help="no GPU work: turn the counter CSVs of two rocprofv3 --pmc runs (FETCH_SIZE, then "
                        "WRITE_SIZE, each ending with --copy-probe) into the traffic summary bench.py reads")
    return p.parse_args()


def traffic_summary(fetch_dir, write_dir, copy_mib, out_json):
    """Per-dispatch HBM bytes of every library kernel from two rocprofv3
    counter runs: the median reading over each kernel's dispatches, scaled by
    the factor that maps the run's last dispatch (the --copy-probe copy of
    copy_mib MiB) to its known size.  Writes out_json and returns it."""
    import csv
    import glob
    import statistics

    def read(d, counter):
        files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
        if not files:
            raise FileNotFoundError(f"no counter_collection.csv under {d}")
        rows = []
        for f in files:
            with open(f) as fh:
                for r in csv.DictReader(fh):
                    if r.get("Counter_Name") == counter:
                        rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
        rows.sort()
        last = rows[-1]
        factor = copy_mib * float(1 << 20) / (last[2] * 1024.0)
        per = {}
        for _, name, val in rows[:-1]:
            name = name[5:] if name.startswith("void ") else name
            if name.startswith("sfi::"):
                per.setdefault(name, []).append(val * 1024.0 * factor)
        return per, factor, last[2] / 1024.0

    fetch, f_fac, f_copy = read(fetch_dir, "FETCH_SIZE")
    write, w_fac, w_copy = read(write_dir, "WRITE_SIZE")
    kernels = {}
    for name in sorted(set(fetch) | set(write)):
        kernels[name] = {"group": kernel_group(name),
                         "dispatches_fetch": len(fetch.get(name, [])),
                         "fetch_bytes": statistics.median(fetch[name]) if name in fetch else 0.0,
                         "dispatches_write": len(write.get(name, [])),
                         "write_bytes": statistics.median(write[name]) if name in write else 0.0}
    out = {"about": "HBM traffic per dispatch from rocprofv3 --pmc FETCH_SIZE and WRITE_SIZE (two runs): median "
                    "over dispatches of each kernel, scaled by the factor that maps the reading of a "
                    f"{copy_mib} MiB device copy made at the end of the same run to {copy_mib} MiB",
           "calibration": {"copy_mib": copy_mib, "fetch_reading_mib": f_copy, "fetch_factor": f_fac,
                           "write_reading_mib": w_copy, "write_factor": w_fac},
           "csrc_digest": csrc_digest(), "kernels": kernels}
    with open(out_json, "w") as fh:
        json.dump(out, fh, indent=1)
    return out


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.traffic_summary:
        t = traffic_summary(*args.traffic_summary, args.copy_probe or 256, TRAFFIC_FILE)
        print(json.dumps(t["calibration"]))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; the path shards by KV head or "
                          "sequence with no per-step communication, but no multi-GPU run is built",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import numpy as np
    import torch

    import sparse_kv_attention_sfi_amd as S
    import synth
    from synth import gen

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a GPU")
    S.lib()  # fail loudly when the library is missing
    dev = torch.device("cuda:0")
    w = {"C1": synth.C1, "C2": synth.C2, "C3": synth.C3, "C4": synth.C4, "C5": synth.C5}[args.workload]
    if w.batch != 1 or w.append:
        run_batched(args, w, dev)
        return
    L, K, W = args.layers, args.steps, args.warmup
    n_steps = max(W + K, w.n_steps)  # the timed window and the workload's whole schedule

    # schedule (host scheduler) and the span index of every step
    sched = S.Scheduler(1, w.seed, w.span_mode, w.span_param)
    flags = [bool(sched.step()[0]) for _ in range(n_steps)]
    sched.close()
    span_ids = [gen.span_ids_from_flags(flags)]
    n_spans = span_ids[0][-1] + 1

    # inputs: L layer caches, per-step queries, all resident in HBM
    t0 = time.time()
    kvs, q_steps = [], torch.empty(n_steps, L, 1, w.n_q_heads, w.head_dim, dtype=gen.torch_dtype(w.dtype),
                                   device=dev)
    for l in range(L):
        c = gen.build_cache(w, dev, layer=l, n_spans=n_spans)
        kvs.append(S.KVDesc(c["K"], c["V"], c["ctx_len"], w.n_q_heads))
        q_steps[:, l].copy_(gen.build_queries(w, dev, span_ids, c, layer=l))
        del c
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s: {L} layers x {w.ctx} ctx")

    sp = S.support_params(w.n_sink, w.n_recent, w.top_k, w.lam)
    ws = S.alloc_workspace(kvs[0], sp)
    q_buf = torch.empty(L, 1, w.n_q_heads, w.head_dim, dtype=q_steps.dtype, device=dev)
    out_buf = torch.empty(L, 1, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    mass = torch.empty(1, w.n_kv_heads, kvs[0].capacity, dtype=torch.float32, device=dev)
    sel = torch.empty(L, 1, w.n_kv_heads, w.top_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(L, 1, w.n_kv_heads, dtype=torch.int32, device=dev)
    packed = args.fast == "packed"
    # deferred packing: the refresh only selects; the first fast step of the
    # span gathers the selected rows and packs them for the packed steps after it
    deferred = packed and args.pack == "deferred"
    refresh_pk = packed and not deferred
    if packed:
        pk = torch.empty(L, 1, w.n_kv_heads, w.top_k, w.head_dim, dtype=q_steps.dtype, device=dev)
        pv = torch.empty_like(pk)

    fused = args.slow in ("fused", "async")
    if args.slow == "async":
        # up to `depth` layers in flight: layer l + depth reuses layer l's
        # workspace and mass buffer, so it waits for layer l's Selector
        depth = args.async_depth
        side = torch.cuda.Stream()
        wsd = [ws] + [S.alloc_workspace(kvs[0], sp) for _ in range(depth - 1)]
        massd = [mass] + [torch.empty_like(mass) for _ in range(depth - 1)]
        sel_done = [torch.cuda.Event() for _ in range(L)]

    def slow_layer(l):
        S.sfi_slow_step_select(kvs[l], sp, [0], q_buf[l], out_buf[l], mass, sel[l], cnt[l],
                               pk[l] if refresh_pk else None, pv[l] if refresh_pk else None, ws)

    def fast_layer(l):
        if packed:
            S.sfi_fast_step_packed(kvs[l], sp, [0], q_buf[l], pk[l], pv[l], cnt[l], out_buf[l], ws)
        else:
            S.sfi_fast_step(kvs[l], sp, [0], q_buf[l], sel[l], cnt[l], out_buf[l], ws)

    def slow_layers():
        if args.slow == "async":
            main = torch.cuda.current_stream()
            for l in range(L):
                if l >= depth:
                    main.wait_event(sel_done[l - depth])
                S.sfi_slow_step_select_async(kvs[l], sp, [0], q_buf[l], out_buf[l], massd[l % depth], sel[l], cnt[l],
                                             pk[l] if refresh_pk else None, pv[l] if refresh_pk else None,
                                             wsd[l % depth],
                                             main, side)
                sel_done[l].record(side)
            main.wait_stream(side)
            return
        for l in range(L):
            if fused:
                slow_layer(l)
                continue
            S.sfi_slow_step(kvs[l], [0], q_buf[l], out_buf[l], mass, ws)
            S.sfi_select(kvs[l], sp, [0], mass, sel[l], cnt[l], ws)
            if refresh_pk:
                S.sfi_pack_support(kvs[l], sp, [0], sel[l], cnt[l], pk[l], pv[l])

    def fast_layers():
        for l in range(L):
            fast_layer(l)

    def first_layer(l):
        S.sfi_fast_step_pack(kvs[l], sp, [0], q_buf[l], sel[l], cnt[l], out_buf[l], pk[l], pv[l], ws)

    def first_layers():
        for l in range(L):
            first_layer(l)

    def kind_of(t):
        """slow (refresh), first (the span's first fast step: packs when
        deferred) or fast."""
        if flags[t]:
            return "slow"
        return "first" if deferred and (t == 0 or flags[t - 1]) else "fast"

    def dense_layers():
        for l in range(L):
            S.sfi_slow_step(kvs[l], [0], q_buf[l], out_buf[l], None, ws)

    # eager warm-up (also primes the selection used by the first fast step)
    q_buf.copy_(q_steps[0])
    slow_layers()
    if deferred:
        first_layers()
    fast_layers()
    dense_layers()
    torch.cuda.synchronize()

    graphs = None
    if args.mode == "graph":
        graphs = {}
        for name, fn in (("slow", slow_layers), ("first", first_layers), ("fast", fast_layers),
                         ("dense", dense_layers)):
            if name == "first" and not deferred:
                continue
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs[name] = g
        run = {name: g.replay for name, g in graphs.items()}
    else:
        run = {"slow": slow_layers, "first": first_layers, "fast": fast_layers, "dense": dense_layers}

    def step(t, kind=None):
        q_buf.copy_(q_steps[t])
        run[kind or kind_of(t)]()

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(W, W + K):
        step(t)
    torch.cuda.synchronize()
    t_blend = time.perf_counter() - t_start
    n_slow_timed = sum(flags[W:W + K])
    n_first_timed = sum(kind_of(t) == "first" for t in range(W, W + K))
    log(f"blended: {K} steps ({n_slow_timed} slow) x {L} layers in {t_blend * 1e3:.1f} ms")

    # The whole span schedule of the workload (its w.n_steps steps), replayed
    # the same way: the blended rate at the schedule's own slow fraction,
    # whatever share of slow steps the --steps window above happened to hold.
    full_schedule = None
    if not args.no_full_schedule:
        full_flags = flags[:w.n_steps]
        torch.cuda.synchronize()
        t_start = time.perf_counter()
        for t in range(w.n_steps):
            q_buf.copy_(q_steps[t])
            run[kind_of(t)]()
        torch.cuda.synchronize()
        t_full = time.perf_counter() - t_start
        full_schedule = {"steps": w.n_steps, "slow_steps": sum(full_flags),
                         "slow_fraction": sum(full_flags) / w.n_steps,
                         "blended_steps_per_s_layer": w.n_steps * L / t_full}

    # Each kind of step alone, as the decode loop runs it (its graph replayed
    # back to back, one query): the per-layer cost of a refresh, of the span's
    # first fast step and of the other fast steps, kernel gaps included.
    graph_us = None
    if graphs is not None and args.graph_reps:
        graph_us = {}
        q_buf.copy_(q_steps[0])
        for name in ("slow", "first", "fast", "dense"):
            if name not in graphs:
                continue
            graphs[name].replay()
            torch.cuda.synchronize()
            t_start = time.perf_counter()
            for _ in range(args.graph_reps):
                graphs[name].replay()
            torch.cuda.synchronize()
            graph_us[name] = (time.perf_counter() - t_start) * 1e6 / (args.graph_reps * L)

    # dense-every-step baseline (same queries)
    kd = min(args.dense_steps, n_steps)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(kd):
        step(t, "dense")
    torch.cuda.synchronize()
    t_dense = time.perf_counter() - t_start

    # Per-kernel durations: with timing on, the library launches each kernel
    # with a HIP event pair stamped by the kernel's own dispatch packet (on the
    # launch stream), over the same schedule steps, eager.
    S.sfi_profile_reset()
    S.sfi_profile_enable(True)
    ke = min(args.eager_steps, n_steps)
    for t in range(ke):
        q_buf.copy_(q_steps[t])
        {"slow": slow_layers, "first": first_layers, "fast": fast_layers}[kind_of(t)]()
    torch.cuda.synchronize()
    S.sfi_profile_enable(False)
    kern = {}
    for kid, name in S.KERNEL_NAMES.items():
        ms, n = S.sfi_profile_read(kid)
        if n:
            kern[name] = {"launches": n, "avg_us": 1e3 * ms / n}

    # The dense slow step alone (the baseline's kernels, no mass, no Selector):
    # its partial kernel's bandwidth is the figure the dense decode reaches.
    dense_kern = {}
    if kd:
        S.sfi_profile_reset()
        S.sfi_profile_enable(True)
        for t in range(min(8, kd)):
            q_buf.copy_(q_steps[t])
            dense_layers()
        torch.cuda.synchronize()
        S.sfi_profile_enable(False)
        for kid, name in S.KERNEL_NAMES.items():
            ms, n = S.sfi_profile_read(kid)
            if n:
                dense_kern[name] = {"launches": n, "avg_us": 1e3 * ms / n}

    # Cold-cache check: the same kernels, each call preceded by a 1 GiB read
    # that evicts L2 and the 256 MB last-level cache.  (A read, not a write: a
    # written flush would leave the caches full of dirty lines whose write-back
    # the next kernel pays for, which the decode loop never does.)  Close
    # agreement with the averages above shows the 32-layer loop runs cold.
    cold = None
    if args.cold_checks:
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        sink = torch.empty((), dtype=torch.float32, device=dev)
        S.sfi_profile_reset()
        for i in range(args.cold_checks):
            l = i % L
            for fn in (lambda: slow_layer(l), lambda: fast_layer(l)) + ((lambda: first_layer(l),) if deferred else ()):
                # the timed call follows the flush in stream order, with the GPU busy
                # in between (after an idle wait a short kernel also pays to wake up)
                torch.sum(flush, dim=0, out=sink)
                S.sfi_profile_enable(True)
                fn()
                S.sfi_profile_enable(False)
                torch.cuda.synchronize()
        cold = {}
        for kid, name in S.KERNEL_NAMES.items():
            ms, n = S.sfi_profile_read(kid)
            if n:
                cold[name + "_us"] = 1e3 * ms / n
        cold["calls"] = args.cold_checks
        del flush
    T = w.ctx
    esz = 2 if w.dtype == "bf16" else 4
    n_cand = T - w.n_sink - w.n_recent
    kk = min(w.top_k, n_cand)
    supp = min(w.n_sink, T) + min(w.n_recent, T) + kk
    kv_row = w.head_dim * esz
    nsplit = S.sfi_slow_plan(kvs[0], [0])[0]
    nchunk = S.sfi_fast_plan(kvs[0], sp, [0])[0]
    q_bytes = w.n_q_heads * w.head_dim * esz
    # algorithmic bytes per launch (what the method has to move)
    alg = {
        "slow_partial": 2 * w.n_kv_heads * T * kv_row + q_bytes,
        # the combine reads the partial kernel's logits and split partials and
        # writes the mass and the output
        "slow_combine": 4 * w.n_q_heads * T + 4 * w.n_q_heads * nsplit * (w.head_dim + 2)
                        + 4 * w.n_kv_heads * T + 4 * w.n_q_heads * w.head_dim,
        "select": 4 * w.n_kv_heads * n_cand + 4 * w.n_kv_heads * w.top_k
                  + (2 * 2 * w.n_kv_heads * kk * kv_row if fused and refresh_pk else 0),
        "pack": 2 * 2 * w.n_kv_heads * kk * kv_row + 4 * w.n_kv_heads * w.top_k,
        "fast_partial": 2 * w.n_kv_heads * supp * kv_row + q_bytes + (0 if packed else 4 * w.n_kv_heads * w.top_k),
        # the gather step reads the indices and the rows, and writes the selected rows again
        "fast_pack": 2 * w.n_kv_heads * supp * kv_row + q_bytes + 4 * w.n_kv_heads * w.top_k
                     + 2 * w.n_kv_heads * kk * kv_row,
        # the merge reads every chunk's (max, sum) and output partial
        "fast_merge": 4 * w.n_q_heads * nchunk * (w.head_dim + 2) + 4 * w.n_q_heads * w.head_dim,
    }
    for name, k in kern.items():
        if name in alg:
            k["alg_bytes"] = alg[name]
            k["GBps"] = alg[name] / (k["avg_us"] * 1e-6) / 1e9
            k["frac"] = k["GBps"] / HBM_PEAK_GBS
    # GPU time of each kernel over the timed steps = launches there x average
    n_fast_timed = K - n_slow_timed
    per_step = {"slow_partial": n_slow_timed, "slow_combine": n_slow_timed, "select": n_slow_timed,
                "pack": n_slow_timed if refresh_pk else 0, "fast_partial": n_fast_timed - n_first_timed,
                "fast_pack": n_first_timed, "fast_merge": n_fast_timed}
    total_time = {n: kern[n]["avg_us"] * per_step[n] * L for n in kern if n in per_step}
    dominant = max(total_time, key=total_time.get)

    def us(name):
        return kern.get(name, {}).get("avg_us", 0.0)

    # what one launch of each kernel group does on this workload
    scope = {"slow_partial": "split-K dense attention over the whole context, writing the logits for the mass",
             "slow_combine": "merge of the split partials, the mass and the Selector's first histogram",
             "select": ("Selector: threshold-bin gather and emission of the kept positions"
                        + (" with their packed rows" if refresh_pk and fused else "")),
             "fast_pack": "the span's first fast step over the gathered support, packing the selected rows it reads",
             "fast_partial": ("the whole fast step: sparse attention over the support in chunks, and, when the "
                              "launch fits the CUs, the merge of the chunk states in the same kernel"
                              if "fast_merge" not in kern else "sparse attention over the support in chunks"),
             "fast_merge": "merge of the fast step's chunk states (separate kernel)"}

    slow_us = us("slow_partial") + us("slow_combine") + us("select") + us("pack")
    fast_us = us("fast_partial") + us("fast_merge")
    first_us = us("fast_pack") + us("fast_merge") if deferred else None
    value = K * L / t_blend
    dense_rate = kd * L / t_dense if kd else None
    d = kern[dominant]
    result = {
        "metric": METRIC,
        "value": value,
        "unit": "decode steps/s/layer",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": 1e3 * t_blend / K,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: B=1, {w.n_q_heads}q/{w.n_kv_heads}kv heads, D={w.head_dim}, "
                               f"ctx {w.ctx}, {w.dtype} KV, sinks {w.n_sink}, recent {w.n_recent}, "
                               f"top-k {w.top_k}, lambda {w.lam}, geometric spans mean {w.span_param}; "
                               f"{L} independent layer caches per decode step",
                   "layers": L, "ctx": w.ctx, "batch": 1, "mode": args.mode, "fast_path": args.fast,
                   "slow_path": args.slow, "packing": args.pack if packed else None,
                   "slow_steps_timed": n_slow_timed},
        "slow_fraction_timed": n_slow_timed / K,
        "full_schedule": full_schedule,
        "slow_step_us": slow_us or None,
        "fast_step_us": fast_us or None,
        "first_fast_step_us": first_us or None,
        "slow_steps_per_s_layer": 1e6 / slow_us if slow_us else None,
        "fast_steps_per_s_layer": 1e6 / fast_us if fast_us else None,
        "blended_steps_per_s_layer": value,
        "dense_steps_per_s_layer": dense_rate,
        "speedup_vs_dense": value / dense_rate if dense_rate else None,
        "graph_step_us": graph_us,
        "kernels": kern,
        "kernel_time_share": {n: t / sum(total_time.values()) for n, t in total_time.items()},
        "cold_cache_check": cold,
        "roofline": {"bound": "hbm", "kernel": dominant, "scope": scope.get(dominant), "achieved": d.get("GBps"),
                     "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": d.get("frac"), "traffic": measured_traffic(dominant, w.name),
                     "alg_bytes_per_launch": d.get("alg_bytes"), "avg_launch_us": d["avg_us"],
                     **traffic_rate(measured_traffic(dominant, w.name), d["avg_us"])},
        "roofline_dense_slow_partial": ({"bound": "hbm", "achieved": alg["slow_partial"] / (dense_kern["slow_partial"]["avg_us"] * 1e-6) / 1e9,
                                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                         "frac": alg["slow_partial"] / (dense_kern["slow_partial"]["avg_us"] * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                         "alg_bytes_per_launch": alg["slow_partial"],
                                         "avg_launch_us": dense_kern["slow_partial"]["avg_us"],
                                         "dense_combine_us": dense_kern.get("slow_combine", {}).get("avg_us")}
                                        if "slow_partial" in dense_kern else None),
        **{f"roofline_{n}": {"bound": "hbm", "achieved": kern[n]["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                             "frac": kern[n]["frac"], "traffic": measured_traffic(n, w.name),
                             "alg_bytes_per_launch": kern[n]["alg_bytes"], "avg_launch_us": kern[n]["avg_us"],
                             **traffic_rate(measured_traffic(n, w.name), kern[n]["avg_us"])}
           for n in ("slow_partial", "fast_partial") if n in kern and n != dominant},
    }
    if args.batch_check:
        result["fast_step_batch"] = fast_batch_check(w, sp, args.batch_check, dev)
    if args.stream_probe:
        sc = stream_copy_probe(args.stream_probe, dev)
        for key, k in (("slow_partial", kern.get("slow_partial")), ("dense_slow_partial", dense_kern.get("slow_partial"))):
            if k:
                sc[f"{key}_vs_copy"] = alg["slow_partial"] / (k["avg_us"] * 1e-6) / 1e9 / sc["GBps"]
        result["stream_copy"] = sc
    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline(w, kvs[0], q_steps[:, 0], flags, n_slow_timed / K)
    if not args.no_configs:
        del kvs, q_steps, graphs, run
        torch.cuda.synchronize()
        torch.cuda.empty_cache()
        result["configs"] = config_block(dev, result, args.workload, args.pack)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result))


def measure_loop(w, dev, layers, dense_steps, warmup=8, n_steps=None, log_name=None, pack="deferred"):
    """Decode-loop throughput of workload ``w`` over ``layers`` layer caches
    (the workload's own layers, or independent caches cycled so that no
    layer's data is still cached at its next step), over the whole span
    schedule (``n_steps`` steps, the workload's count by default).

    Each decode step runs, for every layer: the KV append (growing-history
    workloads), the fused refresh for the rows that open a span, and one fast
    launch for the others.  With ``pack="deferred"`` the refresh only
    selects, and in the fast launch (sfi_fast_step_pack with per-row flags)
    the rows on their span's first fast step gather and pack their support
    while the others read their packed rows; with ``pack="refresh"`` the
    refresh packs and the fast launch reads packed rows only.  Every distinct
    row pattern of the schedule is captured once as a HIP graph and replayed; with
    appends the context lengths live in device memory (advanced by the
    append kernel), so a captured step stays valid as the history grows.
    The dense baseline replays a graph of the same loop with every row
    dense.  Inputs are resident in HBM; only the query (and appended-row)
    staging copies run beside the replays."""
    import numpy as np
    import torch

    import sparse_kv_attention_sfi_amd as S
    from synth import gen

    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    L = layers
    n_steps = n_steps or w.n_steps
    sched = S.Scheduler(B, w.seed, w.span_mode, w.span_param)
    plan = [tuple(tuple(x) for x in sched.step()) for _ in range(n_steps)]
    sched.close()
    flags = [[b in slow for slow, _ in plan] for b in range(B)]
    deferred = pack == "deferred"
    if deferred:
        # (slow rows, rows on their span's first fast step, other fast rows)
        plan = [(slow, tuple(b for b in fast if t > 0 and b in plan[t - 1][0]),
                 tuple(b for b in fast if not (t > 0 and b in plan[t - 1][0])))
                for t, (slow, fast) in enumerate(plan)]
    else:
        plan = [(slow, (), fast) for slow, fast in plan]
    span_ids = [gen.span_ids_from_flags(f) for f in flags]
    t0 = time.time()
    kvs, ctx_devs = [], []
    q_all = torch.empty(n_steps, L, B, Hq, D, dtype=gen.torch_dtype(w.dtype), device=dev)
    if w.append:
        kn_all = torch.empty(n_steps, L, B, Hkv, D, dtype=q_all.dtype, device=dev)
        vn_all = torch.empty_like(kn_all)
    for l in range(L):
        c = gen.build_cache(w, dev, layer=l, n_spans=span_ids[0][-1] + 1)
        T0 = list(c["ctx_len"])
        if w.append:
            # device lengths advanced by the append kernel; the host values are
            # the bound every launch is planned for (the schedule's last length)
            ctx_dev = torch.tensor(T0, dtype=torch.int32, device=dev)
            kvs.append(S.KVDesc(c["K"], c["V"], [t + n_steps for t in T0], Hq, ctx_dev=ctx_dev))
            ctx_devs.append((ctx_dev, T0))
            kn, vn = gen.append_rows(w, dev, layer=l, n_steps=n_steps)
            kn_all[:, l].copy_(kn)
            vn_all[:, l].copy_(vn)
            del kn, vn
        else:
            kvs.append(S.KVDesc(c["K"], c["V"], T0, Hq))
        q_all[:, l].copy_(gen.build_queries(w, dev, span_ids, c, layer=l))
        del c
    torch.cuda.synchronize()
    log(f"{log_name or w.name}: inputs ready in {time.time() - t0:.1f}s ({L} layers, batch {B})")
    sp = S.support_params(w.n_sink, w.n_recent, w.top_k, w.lam)
    ws = S.alloc_workspace(kvs[0], sp)
    out = torch.empty(L, B, Hq, D, device=dev)
    mass = torch.empty(B, Hkv, kvs[0].capacity, device=dev)
    sel = torch.empty(L, B, Hkv, w.top_k, dtype=torch.int32, device=dev)
    cnt = torch.zeros(L, B, Hkv, dtype=torch.int32, device=dev)
    pk = torch.empty(L, B, Hkv, w.top_k, D, dtype=q_all.dtype, device=dev)
    pv = torch.empty_like(pk)
    q_buf = torch.empty_like(q_all[0])
    if w.append:
        kn_buf, vn_buf = torch.empty_like(kn_all[0]), torch.empty_like(vn_all[0])
    all_rows = list(range(B))

    def step_calls(slow, first, fast, dense=False):
        for l in range(L):
            if w.append:
                S.sfi_kv_append(kvs[l], all_rows, kn_buf[l], vn_buf[l])
            if dense:
                S.sfi_slow_step(kvs[l], all_rows, q_buf[l], out[l], None, ws)
                continue
            if slow:
                S.sfi_slow_step_select(kvs[l], sp, list(slow), q_buf[l], out[l], mass, sel[l], cnt[l],
                                       None if deferred else pk[l], None if deferred else pv[l], ws)
            if first:
                # one launch for every fast row: the rows on their span's first
                # fast step gather and pack, the others read their packed rows
                rows = sorted(first + fast)
                S.sfi_fast_step_pack(kvs[l], sp, rows, q_buf[l], sel[l], cnt[l], out[l], pk[l], pv[l], ws,
                                     pack_flags=[int(b in first) for b in rows])
            elif fast:
                S.sfi_fast_step_packed(kvs[l], sp, list(fast), q_buf[l], pk[l], pv[l], cnt[l], out[l], ws)

    def stage(t):
        q_buf.copy_(q_all[t])
        if w.append:
            kn_buf.copy_(kn_all[t])
            vn_buf.copy_(vn_all[t])

    def restart():
        for ctx_dev, T0 in ctx_devs:
            ctx_dev.copy_(torch.tensor(T0, dtype=torch.int32))

    graphs = {}
    for key in sorted(set(plan)) + [("dense",)]:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            if key == ("dense",):
                step_calls((), (), (), dense=True)
            else:
                step_calls(*key)
        graphs[key] = g
    for t in range(min(warmup, n_steps)):
        stage(t)
        graphs[plan[t]].replay()
    torch.cuda.synchronize()
    restart()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(n_steps):
        stage(t)
        graphs[plan[t]].replay()
    torch.cuda.synchronize()
    t_sfi = time.perf_counter() - t_start
    slow_rows = sum(len(p[0]) for p in plan)
    kd = min(dense_steps, n_steps)
    restart()
    stage(0)
    graphs[("dense",)].replay()
    torch.cuda.synchronize()
    restart()
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(kd):
        stage(t)
        graphs[("dense",)].replay()
    torch.cuda.synchronize()
    t_dense = time.perf_counter() - t_start
    value = n_steps * L / t_sfi
    dense_rate = kd * L / t_dense
    res = {"workload": f"{w.name}: B={B}, {Hq}q/{Hkv}kv heads, D={D}, ctx {w.ctx_min}..{w.ctx}, {w.dtype} KV, "
                       f"sinks {w.n_sink}, recent {w.n_recent}, top-k {w.top_k}, {w.span_mode} spans {w.span_param}"
                       f"{', KV append every step' if w.append else ''}; {L} layers",
           "steps": n_steps, "layers": L, "batch": B,
           "sfi_steps_per_s_layer": value, "sfi_tokens_per_s_layer": value * B,
           "dense_steps_per_s_layer": dense_rate, "dense_steps_timed": kd,
           "speedup_vs_dense": value / dense_rate, "slow_row_fraction": slow_rows / (n_steps * B),
           "packing": pack,
           "graphs": len(graphs), "mode": "graph replay per slow/fast row pattern"
                                          + (", device context lengths" if w.append else "")}
    del kvs, q_all, graphs
    if w.append:
        del kn_all, vn_all
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def run_batched(args, w, dev):
    """The batched and growing-history workloads as the bench line: their
    whole span schedule (or --steps steps) replayed from captured graphs."""
    L = w.n_layers if w.n_layers > 1 else max(1, args.batched_caches)
    r = measure_loop(w, dev, L, args.dense_steps or 64, warmup=args.warmup,
                     n_steps=args.steps if args.steps < w.n_steps else w.n_steps, pack=args.pack)
    result = {
        "metric": METRIC, "value": r["sfi_steps_per_s_layer"], "unit": "decode steps/s/layer", "n_gpus": 1,
        "steps": r["steps"], "warmup": args.warmup, "ms_per_step": 1e3 * r["layers"] / r["sfi_steps_per_s_layer"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": r["workload"], "layers": r["layers"], "batch": r["batch"], "mode": r["mode"]},
        **{k: v for k, v in r.items() if k not in ("workload", "steps", "layers", "batch", "mode")},
    }
    print(json.dumps(result))


def stream_copy_probe(mib, dev, reps=10):
    """A plain device-to-device copy of `mib` MiB (torch copy_), timed with
    events on the copy's stream: the streaming bandwidth this GPU reaches
    with a read and a write per byte, the practical ceiling the slow step's
    read stream is compared with."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(2):
        dst.copy_(src)
    ts = []
    for _ in range(reps):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        dst.copy_(src)
        b.record()
        b.synchronize()
        ts.append(a.elapsed_time(b) * 1e3)
    ts.sort()
    us = ts[len(ts) // 2]
    gbps = 2.0 * n * 4 / (us * 1e-6) / 1e9
    del src, dst
    return {"mib": mib, "us": us, "GBps": gbps, "frac": gbps / HBM_PEAK_GBS,
            "bytes_per_copy": "read + write"}


def fast_batch_check(w, sp, batch, dev, ctx=32768, calls=20):
    """The fast step of the same layer shape for `batch` sequences in one
    launch (contexts of 32K; the support, 2320 rows per KV head, does not
    depend on the context), each timed launch right after a 1 GiB read so
    that it runs cold: the kernel's bandwidth once a launch moves enough data
    to fill the chip.  Reported beside the batch-1 workload, not part of it."""
    import torch

    import sparse_kv_attention_sfi_amd as S
    from synth import gen

    K, V = gen.random_cache(batch, w.n_kv_heads, ctx, w.head_dim, w.dtype, dev, seed=w.seed + 77)
    kv = S.KVDesc(K, V, [ctx] * batch, w.n_q_heads)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed + 78)
    q = (2 * torch.randn(batch, w.n_q_heads, w.head_dim, generator=g, device=dev)).to(K.dtype)
    ws = S.alloc_workspace(kv, sp)
    out = torch.empty(batch, w.n_q_heads, w.head_dim, device=dev)
    mass = torch.empty(batch, w.n_kv_heads, ctx, device=dev)
    sel = torch.empty(batch, w.n_kv_heads, w.top_k, dtype=torch.int32, device=dev)
    cnt = torch.empty(batch, w.n_kv_heads, dtype=torch.int32, device=dev)
    pk = torch.empty(batch, w.n_kv_heads, w.top_k, w.head_dim, dtype=K.dtype, device=dev)
    pv = torch.empty_like(pk)
    ids = list(range(batch))
    S.sfi_slow_step_select(kv, sp, ids, q, out, mass, sel, cnt, pk, pv, ws)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    sink = torch.empty((), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    supp = w.n_sink + w.n_recent + w.top_k
    esz = 2 if w.dtype == "bf16" else 4
    alg = batch * (2 * w.n_kv_heads * supp * w.head_dim * esz + w.n_q_heads * w.head_dim * esz)
    res = {"batch": batch, "ctx": ctx, "calls": calls}
    for path in ("packed", "gather"):
        S.sfi_profile_reset()
        for _ in range(calls):
            torch.sum(flush, dim=0, out=sink)
            S.sfi_profile_enable(True)
            if path == "packed":
                S.sfi_fast_step_packed(kv, sp, ids, q, pk, pv, cnt, out, ws)
            else:
                S.sfi_fast_step(kv, sp, ids, q, sel, cnt, out, ws)
            S.sfi_profile_enable(False)
            torch.cuda.synchronize()
        r = {}
        for kid, name in S.KERNEL_NAMES.items():
            ms, n = S.sfi_profile_read(kid)
            if n:
                r[name + "_us"] = 1e3 * ms / n
        a = alg + (batch * 4 * w.n_kv_heads * w.top_k if path == "gather" else 0)
        r["fast_partial_alg_bytes"] = a
        r["fast_partial_GBps"] = a / (r["fast_partial_us"] * 1e-6) / 1e9
        r["fast_partial_frac"] = r["fast_partial_GBps"] / HBM_PEAK_GBS
        res[path] = r
    del K, V, kv, flush
    torch.cuda.empty_cache()
    return res


def config_block(dev, headline, name, pack="deferred"):
    """SFI against dense decode on every workload beside the headline: the
    32K layer (128 independent layer caches), the batch of 16 mixed contexts
    (8 cycled caches) and the 32-layer growing-history loop, each over its
    whole span schedule, plus the headline's own full-schedule figures under
    its workload name `name` (which is then not measured a second time)."""
    import synth
    out = {}
    hs = headline.get("full_schedule") or {}
    if hs and headline.get("dense_steps_per_s_layer"):
        out[name] = {"workload": headline["config"]["workload"], "steps": hs["steps"],
                     "sfi_steps_per_s_layer": hs["blended_steps_per_s_layer"],
                     "dense_steps_per_s_layer": headline["dense_steps_per_s_layer"],
                     "speedup_vs_dense": hs["blended_steps_per_s_layer"] / headline["dense_steps_per_s_layer"],
                     "slow_row_fraction": hs["slow_fraction"]}
    for wname, w, layers in (("C2", synth.C2, 128), ("C4", synth.C4, 8), ("C5", synth.C5, synth.C5.n_layers)):
        if wname in out:
            continue
        out[wname] = measure_loop(w, dev, layers, dense_steps=64, warmup=8, pack=pack)
        log(f"{wname}: SFI {out[wname]['sfi_steps_per_s_layer']:.0f} decode steps/s/layer, "
            f"dense {out[wname]['dense_steps_per_s_layer']:.0f}, speedup {out[wname]['speedup_vs_dense']:.2f}")
    return out


def cpu_baseline(w, kv, q_steps, flags, slow_frac_window):
    """The CPU oracle, as it stands, on layer 0 of the same workload: median
    times of its three operations (the slow step's dense attention with the
    mass, the Selector, the fast step) with the BLAS threads numpy uses by
    default and with one thread, and the blended decode rate they give at the
    workload's span-schedule slow fraction (and at the timed window's)."""
    import statistics

    import numpy as np
    from threadpoolctl import threadpool_info, threadpool_limits

    import oracle as O
    T = int(kv.ctx[0])
    K = kv.k[0, :, :T].float().cpu().numpy().astype(np.float64)
    V = kv.v[0, :, :T].float().cpu().numpy().astype(np.float64)
    q = q_steps[0, 0].float().cpu().numpy().astype(np.float64)
    Hkv = K.shape[0]
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])

    def ops(reps_slow, reps_fast):
        ts = {"slow": [], "select": [], "fast": []}
        sels = None
        for _ in range(reps_slow):
            t0 = time.perf_counter()
            _, P = O.dense_attention(q, K, V)
            f = O.group_mass(P, Hkv)
            t1 = time.perf_counter()
            sels = [O.select(f[g], T, w.n_sink, w.n_recent, w.top_k, w.lam)[0] for g in range(Hkv)]
            t2 = time.perf_counter()
            ts["slow"].append(t1 - t0)
            ts["select"].append(t2 - t1)
        for _ in range(reps_fast):
            t0 = time.perf_counter()
            O.fast_step(q, K, V, T, w.n_sink, w.n_recent, sels)
            ts["fast"].append(time.perf_counter() - t0)
        return {k: statistics.median(v) for k, v in ts.items()}

    # about ten seconds of CPU work in all (the slow step and the Selector take
    # about 0.1 s each with all threads)
    reps = {"many": (30, 100), "one": (8, 30)}
    t_start = time.perf_counter()
    many = ops(*reps["many"])
    with threadpool_limits(1):
        one = ops(*reps["one"])
    spent = time.perf_counter() - t_start
    f_sched = sum(flags[:w.n_steps]) / w.n_steps

    def blended(m, f):
        return 1.0 / (f * (m["slow"] + m["select"]) + (1.0 - f) * m["fast"])

    return {"value": blended(many, f_sched), "unit": "decode steps/s/layer", "cores": threads,
            "kind": "oracle", "os_cpu_count": os.cpu_count(),
            "sample": f"layer 0 of the same workload (T={T}), numpy float64: medians of {reps['many'][0]} slow steps "
                      f"(dense attention + mass), {reps['many'][0]} Selector runs and {reps['many'][1]} fast steps with "
                      f"{threads} BLAS threads, and of {reps['one'][0]}/{reps['one'][0]}/{reps['one'][1]} with one "
                      f"thread ({spent:.1f}s in all); value = the blended rate at the schedule's slow fraction "
                      f"{f_sched:.4f}",
            "ms_all_threads": {k: 1e3 * v for k, v in many.items()},
            "ms_one_thread": {k: 1e3 * v for k, v in one.items()},
            "steps_per_s_layer_all_threads": {"slow": 1.0 / (many["slow"] + many["select"]), "fast": 1.0 / many["fast"],
                                              "blended_schedule": blended(many, f_sched),
                                              "blended_timed_window": blended(many, slow_frac_window)},
            "steps_per_s_layer_one_thread": {"slow": 1.0 / (one["slow"] + one["select"]), "fast": 1.0 / one["fast"],
                                             "blended_schedule": blended(one, f_sched)}}


if __name__ == "__main__":
    main()
