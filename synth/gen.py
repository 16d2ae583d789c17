"""Seeded synthetic inputs for the SFI decode-attention path.

Both the HIP path (through its Python binding) and the CPU oracle receive
tensors made here; the oracle reads back whatever was generated, so parity
never depends on regenerating them on another device.  Nothing here computes
attention, softmax mass, the Selector's scores or the span schedule: span
boundaries come in as an argument (``span_ids``) from whichever scheduler the
caller uses.

Recipes (per KV head g; u is a unit vector N(0, I)/|.|, eps is N(0, I)):

* ``span_dirs`` (tiny fp32 case): for every span s a fresh direction u[s, g]
  and 32 positions, disjoint across spans, whose keys are set to 3 u[s, g];
  queries q = 2 u[s, g] + 0.3 eps.
* ``heavy1pct`` (8B-shaped layer): ceil(1% of T) candidate positions per KV
  head get 2 sqrt(D) u[g] added to their key (a logit offset of about +4 for
  the span query); q_span = 2 u[g] + 0.3 eps, q_t = q_span + 0.2 eps.
* ``zipf`` (128K layer): the key component along u[g] is replaced by
  c_j = -1.1 ln(pi(j)) sqrt(D) / 2 for a random permutation pi of 1..T, so
  the span query's attention mass falls off as pi^-1.1; queries as heavy1pct.
* ``none`` (32-layer loop): K, V ~ N(0, 1); q_span ~ N(0, I) per span,
  q_t = q_span + 0.2 eps; appended rows N(0, 1).

bf16 tensors are produced by rounding float32 values to nearest even.
"""

from __future__ import annotations

import math

import torch

from .configs import Workload

_DT = {"f32": torch.float32, "bf16": torch.bfloat16}

# stream ids within one (workload, layer) seed
S_K, S_V, S_POS, S_DIR, S_SPANQ, S_STEPQ, S_CTX, S_APPEND = 1, 2, 3, 4, 5, 6, 7, 9


def torch_dtype(name):
    return _DT[name]


def generator(device, seed, layer, stream):
    g = torch.Generator(device=device)
    g.manual_seed(((seed * 64 + layer) * 16 + stream) & 0x7FFFFFFFFFFFFFFF)
    return g


def _randn(shape, gen, device):
    return torch.randn(*shape, generator=gen, device=device, dtype=torch.float32)


def _unit(shape, gen, device):
    x = _randn(shape, gen, device)
    return x / x.norm(dim=-1, keepdim=True)


def context_lengths(w: Workload, device="cpu"):
    """Per-sequence context lengths (uniform integers in [ctx_min, ctx])."""
    if w.ctx_min == w.ctx:
        return [w.ctx] * w.batch
    g = generator("cpu", w.seed, 0, S_CTX)
    t = torch.randint(w.ctx_min, w.ctx + 1, (w.batch,), generator=g)
    return [int(x) for x in t]


def random_cache(batch, n_kv, cap, dim, dtype, device, seed, layer=0):
    """K, V ~ N(0, 1) of shape [B, Hkv, cap, D] in ``dtype``."""
    dt = _DT[dtype] if isinstance(dtype, str) else dtype
    K = torch.empty(batch, n_kv, cap, dim, dtype=dt, device=device)
    V = torch.empty_like(K)
    gk = generator(device, seed, layer, S_K)
    gv = generator(device, seed, layer, S_V)
    for b in range(batch):
        for g in range(n_kv):
            K[b, g].copy_(_randn((cap, dim), gk, device))
            V[b, g].copy_(_randn((cap, dim), gv, device))
    return K, V


def build_cache(w: Workload, device, layer=0, n_spans=None, ctx_lens=None):
    """Key/value cache of one layer for workload ``w``.

    Returns a dict with K, V ([B, Hkv, cap, D]), ctx_len (list), and the
    planted structure (directions ``u`` and planted positions) that the query
    generator needs.  ``n_spans`` is needed by the ``span_dirs`` recipe.
    """
    B, Hkv, D = w.batch, w.n_kv_heads, w.head_dim
    cap = w.kv_capacity
    ctx = ctx_lens if ctx_lens is not None else context_lengths(w)
    K = torch.empty(B, Hkv, cap, D, dtype=_DT[w.dtype], device=device)
    V = torch.empty_like(K)
    gk = generator(device, w.seed, layer, S_K)
    gv = generator(device, w.seed, layer, S_V)
    gp = generator(device, w.seed, layer, S_POS)
    gd = generator(device, w.seed, layer, S_DIR)
    info = {"ctx_len": ctx, "u": None, "planted": [[None] * Hkv for _ in range(B)]}
    if w.plant == "span_dirs":
        if n_spans is None:
            raise ValueError("span_dirs needs n_spans")
        info["u"] = _unit((B, n_spans, Hkv, D), gd, device)
    elif w.plant in ("heavy1pct", "zipf"):
        info["u"] = _unit((B, Hkv, D), gd, device)
    for b in range(B):
        T = ctx[b]
        for g in range(Hkv):
            kf = _randn((cap, D), gk, device)
            V[b, g].copy_(_randn((cap, D), gv, device))
            lo, hi = w.n_sink, T - w.n_recent
            if w.plant == "span_dirs":
                per = 32
                perm = torch.randperm(hi - lo, generator=gp, device=device)[: per * n_spans] + lo
                info["planted"][b][g] = perm.view(n_spans, per)
                for s in range(n_spans):
                    kf[perm[s * per:(s + 1) * per]] = 3.0 * info["u"][b, s, g]
            elif w.plant == "heavy1pct":
                cnt = math.ceil(0.01 * T)
                pos = torch.randperm(hi - lo, generator=gp, device=device)[:cnt] + lo
                info["planted"][b][g] = pos
                kf[pos] += 2.0 * math.sqrt(D) * info["u"][b, g]
            elif w.plant == "zipf":
                u = info["u"][b, g]
                rank = torch.randperm(T, generator=gp, device=device).to(torch.float32) + 1.0
                c = -1.1 * torch.log(rank) * (math.sqrt(D) / 2.0)
                e = kf[:T]
                proj = e @ u
                kf[:T] = e - proj[:, None] * u[None, :] + c[:, None] * u[None, :]
                info["planted"][b][g] = rank
            if cap > T:
                kf[T:] = 0.0
                V[b, g, T:] = 0
            K[b, g].copy_(kf)
    return {"K": K, "V": V, **info}


def build_queries(w: Workload, device, span_ids, info, layer=0):
    """Queries for every step: tensor [n_steps, B, Hq, D] in the KV dtype.

    ``span_ids[b][t]`` is the index of the span that step t of sequence b
    belongs to (0 for the first span), as produced by the caller's scheduler.
    """
    B, Hq, Hkv, D = w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim
    G = Hq // Hkv
    n_steps = len(span_ids[0])
    gs = generator(device, w.seed, layer, S_SPANQ)
    gt = generator(device, w.seed, layer, S_STEPQ)
    q = torch.empty(n_steps, B, Hq, D, dtype=_DT[w.dtype], device=device)
    for b in range(B):
        ids = torch.as_tensor(span_ids[b], dtype=torch.long, device=device)
        n_sp = int(ids.max().item()) + 1
        if w.plant == "span_dirs":
            u = info["u"][b]                                  # [n_spans, Hkv, D]
            base = 2.0 * u.repeat_interleave(G, dim=1)        # [n_spans, Hq, D]
            qf = base[ids] + 0.3 * _randn((n_steps, Hq, D), gt, device)
        else:
            if w.plant in ("heavy1pct", "zipf"):
                u = info["u"][b].repeat_interleave(G, dim=0)  # [Hq, D]
                qs = 2.0 * u[None] + 0.3 * _randn((n_sp, Hq, D), gs, device)
            else:
                qs = _randn((n_sp, Hq, D), gs, device)
            qf = qs[ids] + 0.2 * _randn((n_steps, Hq, D), gt, device)
        q[:, b].copy_(qf)
    return q


def append_rows(w: Workload, device, layer=0, n_steps=None):
    """New K and V rows for every step of a growing-history workload:
    two tensors [n_steps, B, Hkv, D] in the KV dtype, N(0, 1)."""
    n = w.n_steps if n_steps is None else n_steps
    g = generator(device, w.seed, layer, S_APPEND)
    shape = (n, w.batch, w.n_kv_heads, w.head_dim)
    k = _randn(shape, g, device).to(_DT[w.dtype])
    v = _randn(shape, g, device).to(_DT[w.dtype])
    return k, v


def span_ids_from_flags(slow_flags):
    """Turn a per-step slow/fast flag list into span indices (a slow step
    opens a new span).  Pure bookkeeping on the caller's schedule."""
    out, s = [], -1
    for f in slow_flags:
        if f:
            s += 1
        out.append(max(s, 0))
    return out
