"""Plain CPU oracle for Slow-Fast Inference (SFI) decode attention.

TEST INFRASTRUCTURE ONLY.  This module is imported by ``tests/``, by
``__graft_entry__.smoke()`` and by the ``cpu_baseline`` leg of ``bench.py``,
and by nothing else.  The product path (``sparse_kv_attention_sfi_amd``) never
imports it and shares no code, header, table or helper with it.

Everything is numpy float64.  Inputs are taken as the exact values the GPU
sees (bf16 or fp32 widened to float64 without rounding).  Each function is
written from the definition on the pages, step by step, with no blocking,
fusion or reordering beyond what that definition states.

Sources (cited by page title and section; the pages print no code):

* [YBC] "Training-Free LLM Inference Acceleration by Exploiting Attention
  Stability Within Sentences" (ybc.sh), sections "How SFI Works: Two Gears
  for Decoding" and "The Key Observation: Attention Support Stays Put".
* [GIST] "Slow-Fast Inference: Training-Free Inference Acceleration via
  Within-Sentence Support Stability" (gist.science, German technical
  summary), section 2.A "Das Slow-Fast Paradigma", 2.B "Der Training-Free
  Selector" (the mixture equation s_lambda = (1 - lambda) f + lambda r),
  2.C "Trigger-Policy", 3 "Systemdesign und Kernel-Optimierung".
* [ABS] the paper's abstract (fugumt.com record of arXiv 2603.12038v1).

Readings taken where the pages are silent (each is listed with its reason in
the design notes of the repository):

* scale of the dot product is 1/sqrt(D); query head h uses KV head h // G;
* the Selector's evidence f is the slow step's softmax probability, averaged
  over the G query heads that share a KV head (so it sums to 1);
* the prior r is a parameter-free positional sink/recency bias over the
  candidate positions: r(a) = (1/a + 1/(n+1-a)) / (2 H_n);
* the fused score is the printed arithmetic mixture, then a top-k with the
  lowest position winning ties;
* optional, all off by default (``select_heads``): a key-norm correction of
  the prior, one round of linear Soft-NMS within a head and a soft
  exclusivity across heads, in readings stated at each function (the pages
  name these steps but give no formula);
* sinks, recent window and selected memory are disjoint; k counts only the
  selected memory;
* the fast step renormalises the softmax over its support;
* the span schedule is drawn from splitmix64 by Bernoulli trials.

Parity pins for every function live in ``tests/test_oracle_*.py``.  The
choices not fixed by the pages or by mathematics are the exact shape of the
prior r and the forms of the key-norm correction, the Soft-NMS round and
the exclusivity: each is pinned by hand-worked examples and invariants of
its own definition, not by the pages ("parity unpinned" against the pages
for those forms).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from fractions import Fraction

import numpy as np

MASK64 = (1 << 64) - 1


# ---------------------------------------------------------------------------
# O1  dense (slow-step) attention over the whole context
# ---------------------------------------------------------------------------
def dense_attention(q, K, V, scale=None):
    """Exact dense GQA decode attention for one sequence.

    The slow step attends to the entire KV history ([YBC] "How SFI Works":
    slow steps perform full dense attention over the entire KV cache; [GIST]
    2.A: slow steps run dense attention over the whole available context).

    q: [Hq, D]; K, V: [Hkv, T, D] (float64).  Query head h reads KV head
    h // (Hq // Hkv).  Returns (out [Hq, D], P [Hq, T]) where P[h] is the
    softmax probability row of head h.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    Hkv, T, _ = K.shape
    if T == 0:
        raise ValueError("dense attention over an empty context is undefined")
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((Hq, D), dtype=np.float64)
    P = np.empty((Hq, T), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        s = (K[g] @ q[h]) * scale            # logits s_hj, j < T
        m = s.max()
        e = np.exp(s - m)
        p = e / e.sum()                      # softmax over all T positions
        P[h] = p
        out[h] = p @ V[g]
    return out, P


# ---------------------------------------------------------------------------
# O2  Selector evidence: per-KV-head softmax mass of the slow step
# ---------------------------------------------------------------------------
def group_mass(P, n_kv_heads):
    """f[g, j] = mean over the G query heads of KV head g of P[h, j].

    The Selector's evidence is the attention of the current slow step
    ([GIST] 2.B); one score row is formed per KV head because the support is
    chosen per head.
    """
    P = np.asarray(P, dtype=np.float64)
    Hq, T = P.shape
    G = Hq // n_kv_heads
    f = np.zeros((n_kv_heads, T), dtype=np.float64)
    for h in range(Hq):
        f[h // G] += P[h]
    return f / G


# ---------------------------------------------------------------------------
# O3  the three parts of the sparse state
# ---------------------------------------------------------------------------
def sink_positions(t, n_sink):
    """Sink tokens: a small fixed anchor set at the start ([GIST] 2.A item 1)."""
    return np.arange(0, min(n_sink, t), dtype=np.int64)


def recent_positions(t, n_sink, n_recent):
    """Recent window: the last n_recent positions before t, never overlapping
    the sinks ([GIST] 2.A item 2)."""
    return np.arange(max(n_sink, t - n_recent), t, dtype=np.int64)


def candidate_positions(t, n_sink, n_recent):
    """Positions eligible for the selected memory ([GIST] 2.A item 3): every
    position that is neither a sink nor in the recent window."""
    lo, hi = n_sink, t - n_recent
    if hi <= lo:
        return np.zeros(0, dtype=np.int64)
    return np.arange(lo, hi, dtype=np.int64)


# ---------------------------------------------------------------------------
# O4  the prior r over the candidates
# ---------------------------------------------------------------------------
def harmonic(n):
    """H_n = sum_{i=1..n} 1/i, correctly rounded sum of the float64 terms."""
    return math.fsum(1.0 / i for i in range(1, n + 1))


def positional_prior(n):
    """Sink/recency prior over n candidates, as a probability vector.

    [GIST] 2.B says the prior is light, cache-based and corrects structural
    biases; it gives no values.  The reading used here is parameter free:
    candidate a (1-based, a = 1 next to the sinks, a = n next to the recent
    window) gets r(a) = (1/a + 1/(n + 1 - a)) / (2 H_n), which sums to one.
    """
    if n == 0:
        return np.zeros(0, dtype=np.float64)
    a = np.arange(1, n + 1, dtype=np.float64)
    return (1.0 / a + 1.0 / (n + 1 - a)) / (2.0 * harmonic(n))


def key_norms(K_rows):
    """Euclidean norm of every key row, nu_j = ||k_j||_2 (float64)."""
    K_rows = np.asarray(K_rows, np.float64)
    return np.sqrt((K_rows * K_rows).sum(axis=-1))


def keynorm_prior(n, nu, beta, c):
    """Prior over n candidates with the key-norm correction.

    [GIST] 2.B: the cache-based prior also corrects structural biases such as
    tokens with extremely high key norms.  The pages give no formula; the
    reading used here: z_j is candidate j's key norm nu_j in standard
    deviations above the mean over the candidates (population statistics;
    z = 0 when all norms are equal), the positional weight of the candidate
    is multiplied by exp(-beta * max(0, z_j - c)), and the weights are
    renormalised to a distribution.  beta >= 0 sets the strength, c the
    number of standard deviations tolerated; beta = 0 is positional_prior(n)
    itself.
    """
    if beta == 0 or n == 0:
        return positional_prior(n)
    nu = np.asarray(nu, np.float64)
    mu = nu.mean()
    sigma = math.sqrt(((nu - mu) ** 2).mean())
    z = (nu - mu) / sigma if sigma > 0 else np.zeros(n)
    penalty = np.exp(-beta * np.maximum(0.0, z - c))
    a = np.arange(1, n + 1, dtype=np.float64)
    w = (1.0 / a + 1.0 / (n + 1 - a)) * penalty
    return w / w.sum()


# ---------------------------------------------------------------------------
# O5  fusion of evidence and prior
# ---------------------------------------------------------------------------
def fused_score(f_cand, r, lam):
    """s_lambda = (1 - lambda) f + lambda r ([GIST] 2.B, the closed-form
    mixture that the reverse-KL fusion reduces to)."""
    return (1.0 - lam) * np.asarray(f_cand, np.float64) + lam * np.asarray(r, np.float64)


# ---------------------------------------------------------------------------
# O5b  discretisation: Soft-NMS within a head, exclusivity across heads
# ---------------------------------------------------------------------------
def soft_nms(score, radius, decay):
    """Soft non-maximum suppression along the candidates of one head.

    [GIST] 2.B, discretisation step 1: within a head, neighbouring tokens
    with similar scores are suppressed to spread the selection over the
    context.  The pages give no formula; the reading used here is one
    parallel round of linear Soft-NMS (each score decayed once, by its
    strongest suppressor, all decays computed from the undecayed scores)
    with the overlap of two positions d apart, 0 < d <= radius, taken as
    1 - d / (radius + 1).  A neighbour suppresses candidate j when it ranks
    above j: a higher score, or the same score at a lower position (the
    top-k order).  Candidate j keeps s_j * (1 - decay * overlap) for its
    nearest suppressor, s_j when it has none.  radius = 0 or decay = 0
    leaves the scores unchanged.  score: the fused scores of consecutive
    candidate positions.
    """
    s = np.asarray(score, np.float64)
    n = s.shape[0]
    if radius <= 0 or decay == 0 or n == 0:
        return s.copy()
    fac = np.ones(n)
    for d in range(1, radius + 1):
        f_d = 1.0 - decay * (1.0 - d / (radius + 1))
        # neighbour d below j ranks above j on a tie; neighbour d above j only when strictly higher
        below = np.zeros(n, dtype=bool)
        below[d:] = s[:-d] >= s[d:]
        above = np.zeros(n, dtype=bool)
        above[:-d] = s[d:] > s[:-d]
        fac = np.where(below | above, np.minimum(fac, f_d), fac)
    return s * fac


def cross_head_exclusivity(S, eps):
    """Soft competition between the KV heads of a sequence.

    [GIST] 2.B, discretisation step 2: heads compete softly so that they do
    not all select the same tokens.  Reading: head g's score of position j
    is multiplied by its share of the heads' total score there, raised to
    eps: S''[g, j] = S[g, j] * (S[g, j] / sum_h S[h, j]) ** eps.  eps = 0, a
    single head, or a zero total leave the scores unchanged.  S: [Hkv, n].
    """
    S = np.asarray(S, np.float64)
    if eps == 0 or S.shape[0] <= 1:
        return S.copy()
    tot = S.sum(axis=0)
    share = np.divide(S, tot, out=np.ones_like(S), where=tot > 0)
    return S * share ** eps


# ---------------------------------------------------------------------------
# O6  top-k of the fused score
# ---------------------------------------------------------------------------
def topk_select(score, positions, k):
    """Top-min(k, n) positions by (score descending, position ascending).

    [GIST] 2.B ends the Selector with a top-k step that yields the token
    indices of the sparse cache.  Ties go to the lowest position.  Returned in
    ascending position order.
    """
    score = np.asarray(score, np.float64)
    positions = np.asarray(positions, np.int64)
    n = positions.shape[0]
    m = min(k, n)
    if m == 0:
        return np.zeros(0, dtype=np.int64)
    order = np.lexsort((positions, -score))   # primary -score, then position
    return np.sort(positions[order[:m]])


def select(f_row, t, n_sink, n_recent, top_k, lam):
    """Selector for one KV head at context length t: O3 -> O4 -> O5 -> O6.

    Returns (sel ascending int64 array, score over the candidates, candidate
    positions)."""
    cand = candidate_positions(t, n_sink, n_recent)
    n = cand.shape[0]
    r = positional_prior(n)
    s = fused_score(np.asarray(f_row, np.float64)[cand], r, lam) if n else np.zeros(0)
    return topk_select(s, cand, top_k), s, cand


def select_heads(f, K, t, n_sink, n_recent, top_k, lam, knorm_beta=0.0, knorm_c=0.0, nms_radius=0,
                 nms_decay=0.0, excl=0.0):
    """Selector of one sequence over all of its KV heads, in [GIST] 2.B's
    order: the prior (positional, with the key-norm correction), its mixture
    with the evidence, Soft-NMS within each head, exclusivity across the
    heads, then top-k.  With every option at zero it is ``select`` applied
    to each head.

    f: [Hkv, >= t] evidence; K: [Hkv, >= t, D] keys (read only when
    knorm_beta != 0).  Returns (sels, final scores [Hkv, n], candidates).
    """
    cand = candidate_positions(t, n_sink, n_recent)
    n = cand.shape[0]
    Hkv = np.asarray(f).shape[0]
    if n == 0:
        return [np.zeros(0, dtype=np.int64) for _ in range(Hkv)], np.zeros((Hkv, 0)), cand
    S = np.empty((Hkv, n))
    for g in range(Hkv):
        nu = key_norms(np.asarray(K[g])[cand]) if knorm_beta != 0 else None
        r = keynorm_prior(n, nu, knorm_beta, knorm_c)
        s = fused_score(np.asarray(f[g], np.float64)[cand], r, lam)
        S[g] = soft_nms(s, nms_radius, nms_decay)
    S = cross_head_exclusivity(S, excl)
    return [topk_select(S[g], cand, top_k) for g in range(Hkv)], S, cand


# ---------------------------------------------------------------------------
# O7  fast step: attention restricted to the support
# ---------------------------------------------------------------------------
def support(t, n_sink, n_recent, sel):
    """S(t) = sinks u recent window u selected memory ([GIST] 2.A), ascending."""
    parts = [sink_positions(t, n_sink), np.asarray(sel, np.int64),
             recent_positions(t, n_sink, n_recent)]
    return np.sort(np.concatenate(parts))


def sparse_attention(q, K, V, supports, scale=None):
    """Fast step: softmax attention over only the support of each KV head
    ([YBC] "How SFI Works": fast steps restrict attention to the subset found
    by the last slow step; [GIST] 2.A).  The softmax is renormalised over the
    support.

    supports: list of Hkv int arrays of positions.
    """
    q = np.asarray(q, dtype=np.float64)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    Hq, D = q.shape
    Hkv = K.shape[0]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.empty((Hq, D), dtype=np.float64)
    for h in range(Hq):
        g = h // G
        S = np.asarray(supports[g], np.int64)
        if S.shape[0] == 0:
            raise ValueError("empty support")
        s = (K[g][S] @ q[h]) * scale
        m = s.max()
        e = np.exp(s - m)
        out[h] = (e / e.sum()) @ V[g][S]
    return out


# ---------------------------------------------------------------------------
# O8  boundary schedule
# ---------------------------------------------------------------------------
def splitmix64_next(state):
    """One step of splitmix64 (Steele, Lea, Flood, "Fast splittable
    pseudorandom number generators", OOPSLA 2014; the 64-bit finaliser
    constants are Stafford's "Mix13").  Returns (new_state, output)."""
    state = (state + 0x9E3779B97F4A7C15) & MASK64
    z = state
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return state, z ^ (z >> 31)


@dataclass
class SpanSchedule:
    """Per-sequence slow/fast schedule.

    A slow step opens every span and refreshes the support for the rest of it
    ([YBC] "How SFI Works": a slow step at each span boundary, fast steps
    inside the span).  With t_max > 0 a slow step is also forced after t_max
    consecutive fast steps ([GIST] 2.C), and that forced step opens a new
    span.  The trigger-token test of [GIST] 2.C needs generated text; span
    lengths drawn here stand in for it.

    mode 'fixed': every span has length ``param``.
    mode 'geometric': span length is the 1-based index of the first
    splitmix64 draw x with x < floor(2**64 / param)  (Bernoulli trials).
    """
    mode: str
    param: float
    seed: int
    t_max: int = 0
    state: int = field(init=False)
    remaining: int = field(init=False, default=0)
    fast_run: int = field(init=False, default=0)
    forced: bool = field(init=False, default=False)

    def __post_init__(self):
        self.state = self.seed & MASK64
        if self.mode == "fixed":
            if int(self.param) != self.param or self.param < 1:
                raise ValueError("fixed span length must be a positive integer")
        elif self.mode == "geometric":
            mu = Fraction(float(self.param))      # exact value of the double
            if mu < 1 or mu >= 2 ** 52:
                raise ValueError("geometric mean span must be in [1, 2**52)")
            # success when a uniform 64-bit draw is below floor(2**64 / mu)
            self.threshold = (2 ** 64 * mu.denominator) // mu.numerator
        else:
            raise ValueError(self.mode)

    def _draw_span(self):
        if self.mode == "fixed":
            return int(self.param)
        n = 0
        while True:
            n += 1
            self.state, x = splitmix64_next(self.state)
            if x < self.threshold:
                return n

    def force_slow(self):
        self.forced = True

    def step(self):
        """Return True for a slow step, False for a fast step."""
        slow = self.remaining == 0 or self.forced or (self.t_max > 0 and self.fast_run >= self.t_max)
        if slow:
            self.forced = False
            self.remaining = self._draw_span() - 1
            self.fast_run = 0
        else:
            self.remaining -= 1
            self.fast_run += 1
        return slow


def schedule(mode, param, seed, n_steps, t_max=0):
    """List of booleans (True = slow) for one sequence."""
    s = SpanSchedule(mode, param, seed, t_max)
    return [s.step() for _ in range(n_steps)]


# ---------------------------------------------------------------------------
# O9  slow step with Selector, and the decode loop
# ---------------------------------------------------------------------------
def slow_step(q, K, V, t, n_sink, n_recent, top_k, lam, scale=None):
    """One slow step for one sequence at context length t: dense output,
    evidence f and the refreshed selected memory per KV head ([GIST] 2.A:
    the slow step re-evaluates the support and refreshes the selected memory
    for the following fast steps)."""
    Hkv = K.shape[0]
    out, P = dense_attention(q, K[:, :t], V[:, :t], scale)
    f = group_mass(P, Hkv)
    sels = [select(f[g], t, n_sink, n_recent, top_k, lam)[0] for g in range(Hkv)]
    return out, f, sels


def fast_step(q, K, V, t, n_sink, n_recent, sels, scale=None):
    """One fast step at context length t reusing the last slow step's
    selected memory."""
    Hkv = K.shape[0]
    sup = [support(t, n_sink, n_recent, sels[g]) for g in range(Hkv)]
    return sparse_attention(q, K, V, sup, scale)


def kv_append(K, V, t, k_new, v_new):
    """Write the new token's key and value at position t (the history grows
    by one each decode step, [ABS]).  K, V: [Hkv, T_cap, D] arrays, in place."""
    K[:, t] = k_new
    V[:, t] = v_new
