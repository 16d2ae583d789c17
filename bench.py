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
path (dense split-K attention + mass + Selector + packing of the selected
rows) or the fast path (sparse attention over the packed support), as the
scheduler says (``--slow async`` runs each layer's Selector on a second
stream under the next layer's slow attention, the pages' asynchronous layer
pipeline; on this attention-only loop it is slower than one stream).
``value`` = K * layers / wall time of K steps (decode steps per
second per layer), with inputs resident in HBM.  Each step's queries are
staged into fixed buffers and the step is replayed as a HIP graph (one for
slow steps, one for fast steps).

Also reported: per-kernel average durations from HIP events recorded by the
library around its launches (eager pass over the same steps), the roofline
of the dominant kernel, the dense-every-step baseline, and the CPU oracle on
a bounded sample of the same workload.
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
    p.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work")
    p.add_argument("--no-cpu", action="store_true")
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
    n_steps = W + K

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
                               pk[l] if packed else None, pv[l] if packed else None, ws)

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
                                             pk[l] if packed else None, pv[l] if packed else None, wsd[l % depth],
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
            if packed:
                S.sfi_pack_support(kvs[l], sp, [0], sel[l], cnt[l], pk[l], pv[l])

    def fast_layers():
        for l in range(L):
            fast_layer(l)

    def dense_layers():
        for l in range(L):
            S.sfi_slow_step(kvs[l], [0], q_buf[l], out_buf[l], None, ws)

    # eager warm-up (also primes the selection used by the first fast step)
    q_buf.copy_(q_steps[0])
    slow_layers()
    fast_layers()
    dense_layers()
    torch.cuda.synchronize()

    if args.mode == "graph":
        graphs = {}
        for name, fn in (("slow", slow_layers), ("fast", fast_layers), ("dense", dense_layers)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                fn()
            graphs[name] = g
        run = {"slow": graphs["slow"].replay, "fast": graphs["fast"].replay, "dense": graphs["dense"].replay}
    else:
        run = {"slow": slow_layers, "fast": fast_layers, "dense": dense_layers}

    def step(t, kind=None):
        q_buf.copy_(q_steps[t])
        run[kind or ("slow" if flags[t] else "fast")]()

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(W, W + K):
        step(t)
    torch.cuda.synchronize()
    t_blend = time.perf_counter() - t_start
    n_slow_timed = sum(flags[W:W + K])
    log(f"blended: {K} steps ({n_slow_timed} slow) x {L} layers in {t_blend * 1e3:.1f} ms")

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
        (slow_layers if flags[t] else fast_layers)()
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
            for fn in (lambda: slow_layer(l), lambda: fast_layer(l)):
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
                  + (2 * 2 * w.n_kv_heads * kk * kv_row if fused and packed else 0),
        "pack": 2 * 2 * w.n_kv_heads * kk * kv_row + 4 * w.n_kv_heads * w.top_k,
        "fast_partial": 2 * w.n_kv_heads * supp * kv_row + q_bytes + (0 if packed else 4 * w.n_kv_heads * w.top_k),
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
                "pack": n_slow_timed if packed else 0, "fast_partial": n_fast_timed, "fast_merge": n_fast_timed}
    total_time = {n: kern[n]["avg_us"] * per_step[n] * L for n in kern if n in per_step}
    dominant = max(total_time, key=total_time.get)

    def us(name):
        return kern.get(name, {}).get("avg_us", 0.0)

    slow_us = us("slow_partial") + us("slow_combine") + us("select") + us("pack")
    fast_us = us("fast_partial") + us("fast_merge")
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
                   "slow_path": args.slow,
                   "slow_steps_timed": n_slow_timed},
        "slow_step_us": slow_us or None,
        "fast_step_us": fast_us or None,
        "slow_steps_per_s_layer": 1e6 / slow_us if slow_us else None,
        "fast_steps_per_s_layer": 1e6 / fast_us if fast_us else None,
        "blended_steps_per_s_layer": value,
        "dense_steps_per_s_layer": dense_rate,
        "speedup_vs_dense": value / dense_rate if dense_rate else None,
        "kernels": kern,
        "kernel_time_share": {n: t / sum(total_time.values()) for n, t in total_time.items()},
        "cold_cache_check": cold,
        "roofline": {"bound": "hbm", "kernel": dominant, "achieved": d.get("GBps"), "peak": HBM_PEAK_GBS,
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
        result["cpu_baseline"] = cpu_baseline(w, kvs[0], q_steps[:, 0], flags, sp, args.cpu_budget)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
    print(json.dumps(result))


def run_batched(args, w, dev):
    """Batched and growing-history workloads (16 sequences with mixed slow and
    fast steps; 4 sequences over 32 layers with a KV append every step).  The
    rows that take a slow step change from step to step and, with appends, so
    do the context lengths baked into every launch, so the loop runs eagerly:
    per layer one append, one fused refresh for the rows that start a span and
    one packed fast step for the others, called through the C ABI with
    prepared arguments.  The dense baseline runs the same loop with a dense
    step for every row."""
    import ctypes as C

    import numpy as np
    import torch

    import sparse_kv_attention_sfi_amd as S
    from sparse_kv_attention_sfi_amd import binding as Bd
    from synth import gen

    lib = S.lib()
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    # layers: the workload's own count, or (single-layer workloads) independent
    # caches cycled so that no layer's data is still cached at its next step
    L = w.n_layers if w.n_layers > 1 else max(1, args.batched_caches)
    K, W = args.steps, args.warmup
    n_steps = W + K
    sched = S.Scheduler(B, w.seed, w.span_mode, w.span_param)
    plan = [sched.step() for _ in range(n_steps)]
    sched.close()
    flags = [[b in slow for slow, _ in plan] for b in range(B)]
    span_ids = [gen.span_ids_from_flags(f) for f in flags]
    t0 = time.time()
    kvs, qs, apps = [], [], []
    for l in range(L):
        c = gen.build_cache(w, dev, layer=l, n_spans=None)
        kvs.append(S.KVDesc(c["K"], c["V"], c["ctx_len"], Hq))
        qs.append(gen.build_queries(w, dev, span_ids, c, layer=l))
        if w.append:
            apps.append(gen.append_rows(w, dev, layer=l, n_steps=n_steps))
        del c
    torch.cuda.synchronize()
    log(f"inputs ready in {time.time() - t0:.1f}s: {L} layers, batch {B}, ctx {kvs[0].ctx.min()}..{kvs[0].ctx.max()}")
    ctx0 = [kv.ctx.copy() for kv in kvs]
    sp = S.support_params(w.n_sink, w.n_recent, w.top_k, w.lam)
    ws = S.alloc_workspace(kvs[0], sp)
    ws_ptr, ws_bytes = C.c_void_p(ws.data_ptr()), C.c_size_t(ws.numel())
    out = torch.empty(B, Hq, D, device=dev)
    mass = torch.empty(B, Hkv, kvs[0].capacity, device=dev)
    sel = [torch.empty(B, Hkv, w.top_k, dtype=torch.int32, device=dev) for _ in range(L)]
    cnt = [torch.zeros(B, Hkv, dtype=torch.int32, device=dev) for _ in range(L)]
    pk = [torch.empty(B, Hkv, w.top_k, D, dtype=kvs[0].dtype, device=dev) for _ in range(L)]
    pv = [torch.empty_like(pk[0]) for _ in range(L)]
    esz = kvs[0].k.element_size()
    stream = C.c_void_p(torch.cuda.current_stream().cuda_stream)
    P = lambda t: C.c_void_p(t.data_ptr())  # noqa: E731
    id_cache = {}

    def ids_of(lst):
        key = tuple(lst)
        if key not in id_cache:
            a = np.asarray(lst, dtype=np.int32)
            id_cache[key] = (a, a.ctypes.data_as(C.POINTER(C.c_int32)), len(lst))
        return id_cache[key][1:]

    all_ids = ids_of(list(range(B)))
    lay = [dict(desc=C.byref(kvs[l].desc), q=qs[l].data_ptr(), qstride=qs[l].stride(0) * esz, sel=P(sel[l]),
                cnt=P(cnt[l]), pk=P(pk[l]), pv=P(pv[l]),
                kn=apps[l][0].data_ptr() if w.append else 0, vn=apps[l][1].data_ptr() if w.append else 0,
                astride=apps[l][0].stride(0) * esz if w.append else 0) for l in range(L)]
    spr, outp, massp = C.byref(sp), P(out), P(mass)

    def ok(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {lib.sfi_last_error().decode()}")

    def step(t, dense=False):
        slow, fast = plan[t]
        if dense:
            slow, fast = list(range(B)), []
        for l in range(L):
            d = lay[l]
            qp = C.c_void_p(d["q"] + t * d["qstride"])
            if w.append:
                ok(lib.sfi_kv_append(d["desc"], all_ids[0], all_ids[1], C.c_void_p(d["kn"] + t * d["astride"]),
                                     C.c_void_p(d["vn"] + t * d["astride"]), stream), "append")
                kvs[l].ctx += 1
            if slow:
                ip, n = ids_of(slow)
                if dense:
                    ok(lib.sfi_slow_step(d["desc"], ip, n, qp, outp, None, ws_ptr, ws_bytes, stream), "dense")
                else:
                    ok(lib.sfi_slow_step_select(d["desc"], spr, ip, n, qp, outp, massp, d["sel"], d["cnt"], d["pk"],
                                                d["pv"], ws_ptr, ws_bytes, stream), "slow")
            if fast:
                ip, n = ids_of(fast)
                ok(lib.sfi_fast_step_packed(d["desc"], spr, ip, n, qp, d["pk"], d["pv"], d["cnt"], outp, ws_ptr,
                                            ws_bytes, stream), "fast")

    for t in range(W):
        step(t)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for t in range(W, W + K):
        step(t)
    torch.cuda.synchronize()
    t_sfi = time.perf_counter() - t_start
    slow_rows = sum(len(plan[t][0]) for t in range(W, W + K))
    log(f"SFI: {K} steps x {L} layers in {t_sfi * 1e3:.1f} ms ({slow_rows} slow row-steps of {K * B})")
    # dense baseline: same loop, every row dense (contexts restarted)
    for l in range(L):
        kvs[l].ctx[:] = ctx0[l]
    kd = min(args.dense_steps, n_steps) if args.dense_steps else min(64, n_steps)
    step(0, dense=True)
    torch.cuda.synchronize()
    for l in range(L):
        kvs[l].ctx[:] = ctx0[l]
    t_start = time.perf_counter()
    for t in range(kd):
        step(t, dense=True)
    torch.cuda.synchronize()
    t_dense = time.perf_counter() - t_start
    value = K * L / t_sfi
    dense_rate = kd * L / t_dense
    result = {
        "metric": METRIC, "value": value, "unit": "decode steps/s/layer", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": 1e3 * t_sfi / K, "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{w.name}: B={B}, {Hq}q/{Hkv}kv heads, D={D}, ctx {w.ctx_min}..{w.ctx}, "
                               f"{w.dtype} KV, sinks {w.n_sink}, recent {w.n_recent}, top-k {w.top_k}, "
                               f"{w.span_mode} spans {w.span_param}, append {w.append}; {L} layers",
                   "layers": L, "batch": B, "mode": "eager (C ABI calls with prepared arguments)"},
        "tokens_per_s_layer": value * B,
        "dense_steps_per_s_layer": dense_rate,
        "speedup_vs_dense": value / dense_rate,
        "slow_row_fraction": slow_rows / (K * B),
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


def cpu_baseline(w, kv, q_steps, flags, sp, budget):
    """The CPU oracle, as it stands, on the first steps of layer 0's schedule
    until ``budget`` seconds of oracle work have run."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle as O
    T = int(kv.ctx[0])
    K = kv.k[0, :, :T].float().cpu().numpy().astype(np.float64)
    V = kv.v[0, :, :T].float().cpu().numpy().astype(np.float64)
    qs = q_steps[:, 0].float().cpu().numpy().astype(np.float64)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    done, sels, spent = 0, None, 0.0
    while spent < budget and done < len(flags):
        t0 = time.perf_counter()
        if flags[done] or sels is None:
            _, _, sels = O.slow_step(qs[done], K, V, T, w.n_sink, w.n_recent, w.top_k, w.lam)
        else:
            O.fast_step(qs[done], K, V, T, w.n_sink, w.n_recent, sels)
        spent += time.perf_counter() - t0
        done += 1
    n_slow = sum(flags[:done])
    return {"value": done / spent, "unit": "decode steps/s/layer", "cores": threads, "kind": "oracle",
            "sample": f"first {done} decode steps ({n_slow} slow) of layer 0 of the same workload, "
                      f"numpy float64, {spent:.1f}s"}


if __name__ == "__main__":
    main()
