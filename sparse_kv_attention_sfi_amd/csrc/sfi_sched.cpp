// Host-side boundary scheduler of the SFI decode loop.
//
// Every span opens with a slow step, which refreshes the support for the
// fast steps of the rest of the span ("Training-Free LLM Inference
// Acceleration by Exploiting Attention Stability Within Sentences", section
// "How SFI Works: Two Gears for Decoding").  A slow step is also forced after
// t_max consecutive fast steps, and then opens a new span ("Slow-Fast
// Inference ...", gist.science technical summary, 2.C "Trigger-Policy").
// Span lengths stand in for the trigger-token test, which needs generated
// text: fixed, or geometric drawn by Bernoulli trials from splitmix64
// (Steele, Lea and Flood, OOPSLA 2014), integer arithmetic only.
#include <cmath>
#include <cstdint>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "../../include/sfi.h"

namespace sfi {
// Records the message for sfi_last_error() and returns the status (host runtime).
int32_t fail(int32_t status, const char* fmt, ...);
}  // namespace sfi

namespace {

struct SeqState {
  uint64_t rng;
  int64_t remaining;  // steps left in the current span after the current one
  int64_t fast_run;   // consecutive fast steps since the last slow step
  bool forced;
};

uint64_t splitmix64(uint64_t* state) {
  *state += 0x9E3779B97F4A7C15ull;
  uint64_t z = *state;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// floor(2^64 / mu) for a double mu in [1, 2^52), exactly: mu = m * 2^ex with
// an integer mantissa m, so the quotient is floor(2^(64 - ex) / m).
bool geometric_threshold(double mu, unsigned __int128* out) {
  if (!(mu >= 1.0 && mu < 4503599627370496.0)) return false;
  int ex = 0;
  const double fr = std::frexp(mu, &ex);          // mu = fr * 2^ex, fr in [0.5, 1)
  const uint64_t m = static_cast<uint64_t>(std::ldexp(fr, 53));  // exact
  const int sh = 64 - (ex - 53);                  // 2^64 / (m * 2^(ex-53))
  // sh <= 116 for mu >= 1 and >= 65 for mu < 2^52
  const unsigned __int128 num = static_cast<unsigned __int128>(1) << sh;
  *out = num / m;
  return true;
}

}  // namespace

struct sfi_sched {
  int32_t mode;
  int64_t fixed_len;
  unsigned __int128 threshold;  // success iff draw < threshold (may equal 2^64)
  int32_t t_max;
  std::vector<SeqState> seqs;

  int64_t draw_span(SeqState& s) const {
    if (mode == SFI_SPAN_FIXED) return fixed_len;
    int64_t n = 0;
    for (;;) {
      ++n;
      const uint64_t x = splitmix64(&s.rng);
      if (static_cast<unsigned __int128>(x) < threshold) return n;
    }
  }
};

extern "C" {

int32_t sfi_sched_create(int32_t batch, uint64_t seed, int32_t mode, double span_param, int32_t t_max,
                         sfi_sched** out) {
  using sfi::fail;
  if (out == nullptr) return fail(SFI_ERR_INVALID_ARG, "sfi_sched_create: out is NULL");
  *out = nullptr;
  if (batch < 1) return fail(SFI_ERR_INVALID_ARG, "sfi_sched_create: batch must be >= 1 (got %d)", batch);
  if (t_max < 0) return fail(SFI_ERR_INVALID_ARG, "sfi_sched_create: t_max must be >= 0 (got %d)", t_max);
  int64_t fixed_len = 0;
  unsigned __int128 threshold = 0;
  if (mode == SFI_SPAN_FIXED) {
    if (!(span_param >= 1.0) || span_param != std::floor(span_param) || span_param > 1e15)
      return fail(SFI_ERR_INVALID_ARG, "sfi_sched_create: a fixed span length must be an integer in [1, 1e15]");
    fixed_len = static_cast<int64_t>(span_param);
  } else if (mode == SFI_SPAN_GEOMETRIC) {
    if (!geometric_threshold(span_param, &threshold))
      return fail(SFI_ERR_INVALID_ARG, "sfi_sched_create: the geometric mean span must lie in [1, 2^52)");
  } else {
    return fail(SFI_ERR_INVALID_ARG, "sfi_sched_create: unknown span mode %d", mode);
  }
  sfi_sched* s = new (std::nothrow) sfi_sched();
  if (s == nullptr) return fail(SFI_ERR_NO_MEMORY, "sfi_sched_create: out of host memory");
  s->mode = mode;
  s->t_max = t_max;
  s->fixed_len = fixed_len;
  s->threshold = threshold;
  try {
    s->seqs.resize(static_cast<size_t>(batch));
  } catch (const std::bad_alloc&) {
    delete s;
    return fail(SFI_ERR_NO_MEMORY, "sfi_sched_create: out of host memory for %d sequences", batch);
  }
  for (int32_t b = 0; b < batch; ++b) {
    s->seqs[b].rng = seed + static_cast<uint64_t>(b);
    s->seqs[b].remaining = 0;
    s->seqs[b].fast_run = 0;
    s->seqs[b].forced = false;
  }
  *out = s;
  return SFI_OK;
}

int32_t sfi_sched_step(sfi_sched* s, int32_t* slow_ids, int32_t* n_slow, int32_t* fast_ids, int32_t* n_fast) {
  if (s == nullptr || slow_ids == nullptr || n_slow == nullptr || fast_ids == nullptr || n_fast == nullptr)
    return sfi::fail(SFI_ERR_INVALID_ARG, "sfi_sched_step: NULL argument");
  int32_t ns = 0, nf = 0;
  for (size_t b = 0; b < s->seqs.size(); ++b) {
    SeqState& q = s->seqs[b];
    const bool slow = q.remaining == 0 || q.forced || (s->t_max > 0 && q.fast_run >= s->t_max);
    if (slow) {
      q.forced = false;
      q.remaining = s->draw_span(q) - 1;
      q.fast_run = 0;
      slow_ids[ns++] = static_cast<int32_t>(b);
    } else {
      q.remaining -= 1;
      q.fast_run += 1;
      fast_ids[nf++] = static_cast<int32_t>(b);
    }
  }
  *n_slow = ns;
  *n_fast = nf;
  return SFI_OK;
}

int32_t sfi_sched_force_slow(sfi_sched* s, int32_t seq) {
  if (s == nullptr) return sfi::fail(SFI_ERR_INVALID_ARG, "sfi_sched_force_slow: scheduler is NULL");
  if (seq < 0 || static_cast<size_t>(seq) >= s->seqs.size())
    return sfi::fail(SFI_ERR_INVALID_ARG, "sfi_sched_force_slow: sequence %d out of range [0, %zu)", seq,
                     s->seqs.size());
  s->seqs[seq].forced = true;
  return SFI_OK;
}

void sfi_sched_destroy(sfi_sched* s) { delete s; }

}  // extern "C"
