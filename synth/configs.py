"""The five synthetic workloads, as plain parameter records.

Only shapes, sizes and knobs live here; nothing in this file computes any
part of the attention, the Selector or the schedule.  The workloads stand in
for the long-context and long-chain-of-thought evaluations reported for SFI
(gist.science technical summary, section 5 "Ergebnisse"), whose datasets and
weights are not used.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Workload:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    ctx: int                   # context length (all sequences) or max of ctx range
    ctx_min: int               # == ctx for a fixed context
    n_steps: int
    span_mode: str             # "fixed" or "geometric"
    span_param: float          # fixed length, or geometric mean
    n_sink: int
    n_recent: int
    top_k: int
    lam: float = 0.1
    n_layers: int = 1
    append: bool = False       # KV append each step (growing history)
    plant: str = "none"        # "span_dirs" | "heavy1pct" | "zipf" | "none"
    seed: int = 1000
    notes: str = ""

    @property
    def group(self):
        return self.n_q_heads // self.n_kv_heads

    @property
    def kv_capacity(self):
        return self.ctx + (self.n_steps if self.append else 0)


C1 = Workload(
    name="C1-tiny-fp32", batch=1, n_q_heads=8, n_kv_heads=2, head_dim=64, dtype="f32",
    ctx=2048, ctx_min=2048, n_steps=64, span_mode="fixed", span_param=16,
    n_sink=4, n_recent=64, top_k=256, plant="span_dirs", seed=1001,
    notes="32 planted positions per span and KV head with key 3u; q = 2u + 0.3 noise")

C2 = Workload(
    name="C2-8B-layer-32K", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
    ctx=32768, ctx_min=32768, n_steps=512, span_mode="geometric", span_param=18,
    n_sink=16, n_recent=256, top_k=2048, plant="heavy1pct", seed=1002,
    notes="1% planted heavy positions per KV head; q_t = q_span + 0.2 noise")

C3 = Workload(
    name="C3-8B-layer-128K", batch=1, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
    ctx=131072, ctx_min=131072, n_steps=1024, span_mode="geometric", span_param=18,
    n_sink=16, n_recent=256, top_k=2048, plant="zipf", seed=1003,
    notes="Zipf(1.1) mass over a random permutation of all positions per KV head")

C4 = Workload(
    name="C4-batch16-mixed", batch=16, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
    ctx=65536, ctx_min=8192, n_steps=512, span_mode="geometric", span_param=18,
    n_sink=16, n_recent=256, top_k=2048, plant="heavy1pct", seed=1004,
    notes="per-sequence contexts uniform in [8192, 65536]; independent schedules")

C5 = Workload(
    name="C5-32layer-loop-128K", batch=4, n_q_heads=32, n_kv_heads=8, head_dim=128, dtype="bf16",
    ctx=131072, ctx_min=131072, n_steps=2048, span_mode="geometric", span_param=30,
    n_sink=16, n_recent=512, top_k=4096, n_layers=32, append=True, plant="none", seed=1005,
    notes="random per-layer caches, KV append each step, long-CoT-like spans")

ALL = {w.name: w for w in (C1, C2, C3, C4, C5)}
BY_INDEX = [C1, C2, C3, C4, C5]
