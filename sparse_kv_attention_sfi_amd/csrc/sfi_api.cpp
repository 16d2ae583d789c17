// Host runtime and C ABI of the SFI decode-attention library: argument
// validation, launch planning (split-K sizes, workgroup tables), workspace
// layout, error reporting and optional per-kernel event timing.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <initializer_list>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "sfi_internal.hpp"

namespace sfi {
namespace {
thread_local std::string g_last_error;
}  // namespace

// Records the message for sfi_last_error() (per calling thread) and returns
// the status.
int32_t fail(int32_t status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return status;
}

namespace {

int32_t hip_fail(hipError_t e, const char* what) {
  return fail(SFI_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int env_int(const char* name, int dflt) {
  const char* s = std::getenv(name);
  if (s == nullptr || *s == '\0') return dflt;
  return std::atoi(s);
}

bool fault_injected(const char* op) {
  const char* s = std::getenv("SFI_FAULT_INJECT");
  return s != nullptr && std::strcmp(s, op) == 0;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

int elem_bytes(int dtype) { return dtype == SFI_BF16 ? 2 : 4; }

// ---- validation -------------------------------------------------------------
int32_t check_desc(const sfi_kv_desc* d) {
  if (d == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc is NULL");
  if (d->batch < 1) return fail(SFI_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", d->batch);
  if (d->n_q_heads < 1 || d->n_kv_heads < 1)
    return fail(SFI_ERR_INVALID_ARG, "head counts must be >= 1 (Hq=%d, Hkv=%d)", d->n_q_heads, d->n_kv_heads);
  // bounds that keep every workspace size and launch-grid count in range
  if (d->batch > kMaxBatch) return fail(SFI_ERR_INVALID_ARG, "batch %d exceeds %d", d->batch, kMaxBatch);
  if (d->n_kv_heads > kMaxKvHeads)
    return fail(SFI_ERR_UNSUPPORTED, "n_kv_heads %d exceeds %d", d->n_kv_heads, kMaxKvHeads);
  if (d->n_q_heads % d->n_kv_heads != 0)
    return fail(SFI_ERR_INVALID_ARG, "n_q_heads (%d) is not a multiple of n_kv_heads (%d)", d->n_q_heads,
                d->n_kv_heads);
  const int G = d->n_q_heads / d->n_kv_heads;
  if (G != 1 && G != 2 && G != 4 && G != 8)
    return fail(SFI_ERR_UNSUPPORTED, "query group size %d not supported (1, 2, 4 or 8)", G);
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(SFI_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->kv_dtype != SFI_F32 && d->kv_dtype != SFI_BF16)
    return fail(SFI_ERR_UNSUPPORTED, "kv_dtype %d not supported", d->kv_dtype);
  if (d->kv_capacity < 1 || d->kv_capacity > (int64_t{1} << 30))
    return fail(SFI_ERR_INVALID_ARG, "kv_capacity %lld out of range [1, 2^30]",
                static_cast<long long>(d->kv_capacity));
  if (!(std::isfinite(d->scale)) || d->scale < 0.f)
    return fail(SFI_ERR_INVALID_ARG, "scale must be finite and >= 0");
  return SFI_OK;
}

// The kernels move K, V, q, the float outputs, the packed rows and the
// workspace in 16-byte vectors and the int32 arrays in 4-byte words, so each
// buffer must start on that boundary (NULL entries are not checked here).
constexpr size_t kVecAlign = 16;
constexpr size_t kIntAlign = 4;

int32_t check_aligned(std::initializer_list<std::pair<const void*, const char*>> bufs, size_t align) {
  for (const auto& [p, name] : bufs)
    if (p != nullptr && reinterpret_cast<uintptr_t>(p) % align != 0)
      return fail(SFI_ERR_INVALID_ARG, "%s is not %zu-byte aligned", name, align);
  return SFI_OK;
}

int32_t check_kv(const sfi_kv_desc* d) {
  if (d->k == nullptr || d->v == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc->k / desc->v is NULL");
  if (d->ctx_len_host == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc->ctx_len_host is NULL");
  if (const int32_t st = check_aligned({{d->ctx_len, "desc->ctx_len"}}, kIntAlign); st != SFI_OK) return st;
  return check_aligned({{d->k, "desc->k"}, {d->v, "desc->v"}}, kVecAlign);
}

int32_t check_seqs(const sfi_kv_desc* d, const int32_t* ids, int32_t n, bool need_ctx, int32_t min_ctx,
                   int64_t max_ctx) {
  if (n < 0) return fail(SFI_ERR_INVALID_ARG, "n_seq must be >= 0 (got %d)", n);
  if (n == 0) return SFI_OK;
  if (ids == nullptr) return fail(SFI_ERR_INVALID_ARG, "seq_ids_host is NULL");
  std::vector<char> seen(static_cast<size_t>(d->batch), 0);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || b >= d->batch) return fail(SFI_ERR_INVALID_ARG, "seq id %d out of range [0, %d)", b, d->batch);
    if (seen[b]) return fail(SFI_ERR_INVALID_ARG, "seq id %d listed twice", b);
    seen[b] = 1;
    if (need_ctx) {
      const int32_t t = d->ctx_len_host[b];
      if (t < min_ctx || t > max_ctx)
        return fail(SFI_ERR_INVALID_ARG, "ctx_len[%d] = %d out of range [%d, %lld]", b, t, min_ctx,
                    static_cast<long long>(max_ctx));
    }
  }
  return SFI_OK;
}

// check_seqs for at most kMaxSeqPerLaunch ids, with the context lengths
// required, without allocating (pairwise duplicate test).
int32_t check_seqs_small(const sfi_kv_desc* d, const int32_t* ids, int32_t n, int32_t min_ctx, int64_t max_ctx) {
  if (n < 0) return fail(SFI_ERR_INVALID_ARG, "n_seq must be >= 0 (got %d)", n);
  if (n > kMaxSeqPerLaunch) return fail(SFI_ERR_UNSUPPORTED, "n_seq %d exceeds %d", n, kMaxSeqPerLaunch);
  if (n == 0) return SFI_OK;
  if (ids == nullptr) return fail(SFI_ERR_INVALID_ARG, "seq_ids_host is NULL");
  for (int32_t i = 0; i < n; ++i) {
    const int32_t b = ids[i];
    if (b < 0 || b >= d->batch) return fail(SFI_ERR_INVALID_ARG, "seq id %d out of range [0, %d)", b, d->batch);
    for (int32_t j = 0; j < i; ++j)
      if (ids[j] == b) return fail(SFI_ERR_INVALID_ARG, "seq id %d listed twice", b);
    const int32_t t = d->ctx_len_host[b];
    if (t < min_ctx || t > max_ctx)
      return fail(SFI_ERR_INVALID_ARG, "ctx_len[%d] = %d out of range [%d, %lld]", b, t, min_ctx,
                  static_cast<long long>(max_ctx));
  }
  return SFI_OK;
}

int32_t check_params(const sfi_support_params* sp) {
  if (sp == nullptr) return fail(SFI_ERR_INVALID_ARG, "support params are NULL");
  if (sp->n_sink < 0 || sp->n_recent < 0 || sp->top_k < 0)
    return fail(SFI_ERR_INVALID_ARG, "n_sink, n_recent and top_k must be >= 0");
  if (sp->top_k > (1 << 24)) return fail(SFI_ERR_INVALID_ARG, "top_k %d too large", sp->top_k);
  if (sp->n_sink > (1 << 30) || sp->n_recent > (1 << 30))
    return fail(SFI_ERR_INVALID_ARG, "n_sink and n_recent must be <= 2^30");
  if (!(sp->lambda >= 0.f && sp->lambda <= 1.f))
    return fail(SFI_ERR_INVALID_ARG, "lambda must lie in [0, 1]");
  if (!(std::isfinite(sp->knorm_beta) && sp->knorm_beta >= 0.f) || !std::isfinite(sp->knorm_c))
    return fail(SFI_ERR_INVALID_ARG, "knorm_beta must be finite and >= 0, knorm_c finite");
  if (sp->nms_radius < 0 || sp->nms_radius > 32) return fail(SFI_ERR_INVALID_ARG, "nms_radius must lie in [0, 32]");
  if (!(sp->nms_decay >= 0.f && sp->nms_decay <= 1.f)) return fail(SFI_ERR_INVALID_ARG, "nms_decay must lie in [0, 1]");
  if (!(std::isfinite(sp->excl) && sp->excl >= 0.f)) return fail(SFI_ERR_INVALID_ARG, "excl must be finite and >= 0");
  return SFI_OK;
}

// Whether the optional Selector steps (key-norm prior, Soft-NMS, exclusivity)
// are on: the Selector then scores the candidates in a pass of its own.
bool sel_options(const sfi_support_params* sp) {
  return sp->knorm_beta > 0.f || (sp->nms_radius > 0 && sp->nms_decay > 0.f) || sp->excl > 0.f;
}

// Candidate positions one score workgroup handles for all KV heads: its
// mixture window (chunk + 2 radius), Soft-NMS results (chunk) and column
// totals (chunk) fit kScoreLds floats; a multiple of 32, at most 1024;
// 0 when even 32 do not fit.
int score_chunk(const sfi_kv_desc* d, const sfi_support_params* sp) {
  const int64_t room = kScoreLds - 2LL * sp->nms_radius * d->n_kv_heads;
  const int64_t c = room / (2LL * d->n_kv_heads + 1) / 32 * 32;
  return static_cast<int>(std::min<int64_t>(1024, std::max<int64_t>(0, c)));
}

float logit_scale(const sfi_kv_desc* d) {
  const float s = d->scale > 0.f ? d->scale : 1.0f / std::sqrt(static_cast<float>(d->head_dim));
  return s * 1.4426950408889634f;  // log2(e): the kernels use exp2
}

// ---- workspace layout -----------------------------------------------------
// [ header | op scratch ].  The header holds the Selector's per-head
// bookkeeping (top-digit histogram, list counter), cleared by the first kernel
// of every call that builds a histogram, and the fast step's per-head chunk
// counters, zero from sfi_workspace_init and left at zero by every fast step;
// it sits at a fixed offset so slow, select and fast calls may share one
// workspace.
// Rows whose fast-step chunk states a workspace holds at once: one launch group.
size_t fast_rows(const sfi_kv_desc* d) { return static_cast<size_t>(std::min(d->batch, kMaxSeqPerLaunch)); }

struct Header {
  size_t sel_hist, sel_list_n, fast_ticket, end;
};
Header header_layout(const sfi_kv_desc* d) {
  const size_t bh = static_cast<size_t>(d->batch) * d->n_kv_heads;
  Header H;
  H.sel_hist = 0;
  H.sel_list_n = H.sel_hist + align_up(bh * 4096 * sizeof(uint32_t));
  H.fast_ticket = H.sel_list_n + align_up(bh * sizeof(int32_t));
  H.end = H.fast_ticket + align_up(fast_rows(d) * d->n_kv_heads * kTicketStride * sizeof(int32_t));
  return H;
}
size_t header_bytes(const sfi_kv_desc* d) { return header_layout(d).end; }

struct SelectLayout {
  size_t list, chunk_above, head_info, above_pos, end;
};
SelectLayout select_layout(const sfi_kv_desc* d) {
  const size_t bh = static_cast<size_t>(d->batch) * d->n_kv_heads;
  SelectLayout L;
  L.list = header_bytes(d);
  L.chunk_above = L.list + align_up(bh * kSelListCap * sizeof(uint64_t));
  L.head_info = L.chunk_above + align_up(bh * kSelMaxChunks * sizeof(int32_t));
  L.above_pos = L.head_info + align_up(bh * 2 * sizeof(int32_t));
  L.end = L.above_pos + align_up(bh * static_cast<size_t>(d->kv_capacity) * sizeof(int32_t));
  return L;
}

// Buffers of the optional Selector steps, placed after every other scratch
// so that the slow step's kernels may write the key norms while its logits
// and partials are in use: final scores and key norms [B][Hkv][T_cap], per
// split norm sums, per head norm statistics, per mass block normaliser sums.
struct ExtLayout {
  size_t score, knorm, knorm_part, knorm_stat, zpart, end;
  int zpart_stride;
};
int slow_part_stride(const sfi_kv_desc* d);
ExtLayout ext_layout(const sfi_kv_desc* d, size_t start) {
  const size_t bh = static_cast<size_t>(d->batch) * d->n_kv_heads;
  const size_t rows = bh * static_cast<size_t>(d->kv_capacity);
  ExtLayout E;
  E.zpart_stride = static_cast<int>(ceil_div(d->kv_capacity, kMassChunk));
  E.score = align_up(start);
  E.knorm = E.score + align_up(rows * sizeof(float));
  E.knorm_part = E.knorm + align_up(rows * sizeof(float));
  E.knorm_stat = E.knorm_part + align_up(bh * slow_part_stride(d) * 2 * sizeof(double));
  E.zpart = E.knorm_stat + align_up(bh * 2 * sizeof(double));
  E.end = E.zpart + align_up(bh * E.zpart_stride * sizeof(double));
  return E;
}

int slow_unit_rows(const sfi_kv_desc* d) {
  return (kSlowThreads / 64) * block_rows(d->head_dim * elem_bytes(d->kv_dtype));
}

int slow_part_stride(const sfi_kv_desc* d) {
  return static_cast<int>(ceil_div(d->kv_capacity, slow_unit_rows(d)));
}

int64_t logit_pitch(const sfi_kv_desc* d) { return (d->kv_capacity + 63) / 64 * 64; }

struct SlowLayout {
  size_t logits, part_ml, part_o, end;
};
SlowLayout slow_layout(const sfi_kv_desc* d) {
  SlowLayout L;
  const size_t heads = static_cast<size_t>(d->batch) * d->n_q_heads;
  const size_t stride = static_cast<size_t>(slow_part_stride(d));
  L.logits = header_bytes(d);
  L.part_ml = L.logits + align_up(heads * static_cast<size_t>(logit_pitch(d)) * sizeof(float));
  L.part_o = L.part_ml + align_up(heads * stride * 2 * sizeof(float));
  L.end = L.part_o + align_up(heads * stride * d->head_dim * sizeof(float));
  return L;
}

int fast_part_stride(const sfi_support_params* sp) {
  const int64_t rows = static_cast<int64_t>(sp->n_sink) + sp->n_recent + sp->top_k;
  return static_cast<int>(std::max<int64_t>(1, ceil_div(rows, fast_chunk_rows())));
}

// Fast-step workgroups per KV head at context t: the support's largest
// possible size in chunks of crow rows.
int32_t fast_chunks(const sfi_support_params* sp, int64_t t, int crow) {
  const int64_t ns_eff = std::min<int64_t>(sp->n_sink, t);
  const int64_t w_lo = std::max<int64_t>(sp->n_sink, t - sp->n_recent);
  const int64_t w_eff = std::max<int64_t>(0, t - w_lo);
  const int64_t n = std::max<int64_t>(0, t - sp->n_sink - sp->n_recent);
  const int64_t smax = ns_eff + w_eff + std::min<int64_t>(sp->top_k, n);
  return static_cast<int32_t>(std::max<int64_t>(1, ceil_div(smax, crow)));
}

struct FastLayout {
  size_t part_ml, part_o, end;
};
FastLayout fast_layout(const sfi_kv_desc* d, const sfi_support_params* sp) {
  FastLayout L;
  const size_t heads = fast_rows(d) * d->n_q_heads;
  const size_t stride = static_cast<size_t>(fast_part_stride(sp));
  L.part_ml = header_bytes(d);
  L.part_o = L.part_ml + align_up(heads * stride * 2 * sizeof(float));
  L.end = L.part_o + align_up(heads * stride * d->head_dim * sizeof(float));
  return L;
}

int32_t check_ws(void* ws, size_t have, size_t need) {
  if (need == 0) return SFI_OK;
  if (ws == nullptr) return fail(SFI_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if (have < need) return fail(SFI_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", have, need);
  return check_aligned({{ws, "workspace"}}, kVecAlign);
}

// ---- event timing ---------------------------------------------------------
struct Prof {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> pending[SFI_K_COUNT];
  std::vector<hipEvent_t> pool;
  double ms[SFI_K_COUNT] = {};
  int64_t launches[SFI_K_COUNT] = {};
};
Prof& prof() {
  static Prof p;
  return p;
}

hipEvent_t take_event(Prof& p) {
  if (!p.pool.empty()) {
    hipEvent_t e = p.pool.back();
    p.pool.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}

thread_local LaunchTiming* g_timing = nullptr;

// Per-thread, per-device events that order work across two streams (timing
// disabled; an event is created on the device current at the call, the device
// of the caller's streams).  A wait binds to the record that precedes it, so
// one event per role can be re-recorded by every call.  They live until the
// process ends: destroying them from a thread-exit destructor could run after
// the HIP runtime has shut down.

bool stream_event(int role, hipEvent_t* out) {
  thread_local hipEvent_t ev[kMaxDevices][2] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  hipEvent_t& e = ev[dev][role];
  if (e == nullptr && hipEventCreateWithFlags(&e, hipEventDisableTiming) != hipSuccess) {
    e = nullptr;
    return false;
  }
  *out = e;
  return true;
}

// Compute units of the current device (queried once per device).
bool compute_units(int* out) {
  static std::atomic<int> cus[kMaxDevices] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return false;
  int n = cus[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return false;
    cus[dev].store(n, std::memory_order_relaxed);
  }
  *out = n;
  return true;
}

// Runs `launch` (returning hipError_t); when timing is on, its kernels stamp a
// fresh event pair from their own dispatch packets.
template <typename F>
hipError_t timed(int kid, hipStream_t s, F&& launch) {
  (void)s;
  Prof& p = prof();
  bool on;
  {
    std::lock_guard<std::mutex> lk(p.mu);
    on = p.on;
  }
  if (!on) return launch();
  LaunchTiming t;
  {
    std::lock_guard<std::mutex> lk(p.mu);
    t.start = take_event(p);
    t.stop = take_event(p);
  }
  if (t.start == nullptr || t.stop == nullptr) return hipErrorOutOfMemory;
  const hipEvent_t a = t.start, b = t.stop;
  g_timing = &t;
  const hipError_t e = launch();
  g_timing = nullptr;
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lk(p.mu);
  p.pending[kid].emplace_back(a, b);
  return hipSuccess;
}

// ---- launch tables --------------------------------------------------------
// Splits the id list into groups of at most kMaxSeqPerLaunch.
template <typename F>
int32_t for_each_group(const int32_t* ids, int32_t n, F&& f) {
  for (int32_t i0 = 0; i0 < n; i0 += kMaxSeqPerLaunch) {
    const int32_t cnt = std::min<int32_t>(kMaxSeqPerLaunch, n - i0);
    const int32_t st = f(ids + i0, cnt);
    if (st != SFI_OK) return st;
  }
  return SFI_OK;
}

// ---- launch planning ------------------------------------------------------
// Slow step: split-K partial over the whole history, then the combine
// (output merge + mass).  Fills the launch arguments of one id group.
// with_mass: the step writes mass (its partial kernel stores logits); mass
// may still be NULL when only the launch table is wanted.
void plan_slow(const sfi_kv_desc* desc, const int32_t* ids, int32_t cnt, const void* q, float* out, float* mass,
               bool with_mass, char* w, SlowArgs& a, CombineArgs& c) {
  const SlowLayout L = slow_layout(desc);
  const int G = desc->n_q_heads / desc->n_kv_heads;
  const int unit = slow_unit_rows(desc);
  // workgroups the split-K partial aims at; SFI_SLOW_TARGET_WGS overrides it
  // for tuning (read once per process)
  static const int target = std::max(64, env_int("SFI_SLOW_TARGET_WGS", kSlowTargetWgs));
  a.k = desc->k;
  a.v = desc->v;
  a.q = q;
  // w is NULL when only the launch table is wanted (sfi_slow_plan)
  a.logits = (mass && w) ? reinterpret_cast<float*>(w + L.logits) : nullptr;
  a.part_ml = w ? reinterpret_cast<float*>(w + L.part_ml) : nullptr;
  a.part_o = w ? reinterpret_cast<float*>(w + L.part_o) : nullptr;
  a.out = out;
  a.mass = mass;
  a.t_cap = desc->kv_capacity;
  a.n_q_heads = desc->n_q_heads;
  a.n_kv_heads = desc->n_kv_heads;
  a.part_stride = slow_part_stride(desc);
  a.scale_log2 = logit_scale(desc);
  a.logit_pitch = logit_pitch(desc);
  int64_t rows = 0, t_max = 1;
  for (int i = 0; i < cnt; ++i) {
    rows += static_cast<int64_t>(desc->ctx_len_host[ids[i]]) * desc->n_kv_heads;
    t_max = std::max<int64_t>(t_max, desc->ctx_len_host[ids[i]]);
  }
  // at most kMaxMergeSlots splits per head (the merge stages them in LDS);
  // splits of at least kSlowMinRows rows: shorter ones (a 32K row aimed at
  // 1024 workgroups gets 256) cost more per row than they gain in workgroups
  // (28.7 against 31.6 us with mass on a 32K layer, 30.9 against 33.2 us
  // without); with mass at most kLogitBufRows where that limit allows, so
  // that the partial kernel can buffer each split's logits
  int64_t want = std::max<int64_t>(ceil_div(rows, target), kSlowMinRows);
  if (with_mass) want = std::min<int64_t>(want, kLogitBufRows);
  const int64_t per = std::max(want, ceil_div(t_max, kMaxMergeSlots));
  a.split_rows = static_cast<int32_t>(std::max<int64_t>(unit, ceil_div(per, unit) * unit));
  a.tab.n = cnt;
  a.tab.ctx_dev = desc->ctx_len;
  a.tab.wg_begin[0] = 0;
  c.tab.n = cnt;
  c.tab.ctx_dev = desc->ctx_len;
  c.tab.wg_begin[0] = 0;
  for (int i = 0; i < cnt; ++i) {
    const int b = ids[i];
    const int T = desc->ctx_len_host[b];
    a.tab.ent[i].seq = b;
    a.tab.ent[i].ctx = T;
    a.tab.ent[i].nsplit = static_cast<int32_t>(ceil_div(T, a.split_rows));
    a.tab.wg_begin[i + 1] = a.tab.wg_begin[i] + desc->n_kv_heads * a.tab.ent[i].nsplit;
    c.mass_blocks[i] = with_mass ? static_cast<int32_t>(ceil_div(T, kMassChunk)) : 0;
    c.tab.ent[i].seq = b;
    c.tab.ent[i].ctx = T;
    c.tab.ent[i].nsplit = a.tab.ent[i].nsplit;
    c.tab.wg_begin[i + 1] = c.tab.wg_begin[i] + desc->n_kv_heads * (c.mass_blocks[i] + G);
  }
  c.logits = a.logits;
  c.part_ml = a.part_ml;
  c.part_o = a.part_o;
  c.out = out;
  c.mass = mass;
  c.t_cap = a.t_cap;
  c.n_q_heads = a.n_q_heads;
  c.n_kv_heads = a.n_kv_heads;
  c.part_stride = a.part_stride;
  c.logit_pitch = a.logit_pitch;
}

int32_t run_slow(const sfi_kv_desc* desc, const SlowArgs& a, const CombineArgs& c, int32_t cnt, hipStream_t s) {
  const int G = desc->n_q_heads / desc->n_kv_heads;
  hipError_t e = timed(SFI_K_SLOW_PARTIAL, s, [&] {
    return launch_slow_partial(a, desc->kv_dtype, desc->head_dim, G, a.tab.wg_begin[cnt], s);
  });
  if (e != hipSuccess) return hip_fail(e, "slow partial launch");
  e = timed(SFI_K_SLOW_COMBINE, s, [&] { return launch_slow_combine(c, desc->head_dim, G, c.tab.wg_begin[cnt], s); });
  if (e != hipSuccess) return hip_fail(e, "slow combine launch");
  return SFI_OK;
}

// Selector: candidates of each (sequence, KV head) cut into chunks of at
// least kSelMinChunk, at most kSelMaxChunks chunks per head.
void plan_select(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* ids, int32_t cnt,
                 const float* mass, int32_t* sel_idx, int32_t* sel_cnt, char* w, SelectArgs& a) {
  const SelectLayout L = select_layout(desc);
  const Header H = header_layout(desc);
  a.mass = mass;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.hist = reinterpret_cast<uint32_t*>(w + H.sel_hist);
  a.list_n = reinterpret_cast<int32_t*>(w + H.sel_list_n);
  a.list = reinterpret_cast<uint64_t*>(w + L.list);
  a.chunk_above = reinterpret_cast<int32_t*>(w + L.chunk_above);
  a.head_info = reinterpret_cast<int32_t*>(w + L.head_info);
  a.above_pos = reinterpret_cast<int32_t*>(w + L.above_pos);
  a.t_cap = desc->kv_capacity;
  a.n_kv_heads = desc->n_kv_heads;
  a.n_sink = sp->n_sink;
  a.n_recent = sp->n_recent;
  a.top_k = sp->top_k;
  a.lambda = sp->lambda;
  int64_t n_max = 0;
  for (int i = 0; i < cnt; ++i)
    n_max = std::max<int64_t>(n_max, desc->ctx_len_host[ids[i]] - static_cast<int64_t>(sp->n_sink) - sp->n_recent);
  const int64_t chunk = std::max<int64_t>(kSelMinChunk, ceil_div(ceil_div(n_max, kSelMaxChunks), 512) * 512);
  a.chunk = static_cast<int32_t>(chunk);
  a.tab.n = cnt;
  a.tab.ctx_dev = desc->ctx_len;
  a.tab.wg_begin[0] = 0;
  for (int i = 0; i < cnt; ++i) {
    const int64_t T = desc->ctx_len_host[ids[i]];
    const int64_t n = std::max<int64_t>(0, T - sp->n_sink - sp->n_recent);
    const bool keep_all = n <= sp->top_k || sp->top_k == 0;
    const int64_t m_keep = std::max<int64_t>(1, ceil_div(sp->top_k, chunk));
    // device context lengths may be shorter than the bound n was taken from:
    // the grid then covers both the keep-all emission and the bound's chunks
    const int64_t M = desc->ctx_len != nullptr ? std::max(m_keep, ceil_div(n, chunk))
                      : keep_all              ? m_keep
                                              : ceil_div(n, chunk);
    a.tab.ent[i].seq = ids[i];
    a.tab.ent[i].ctx = static_cast<int32_t>(T);
    a.tab.ent[i].nsplit = static_cast<int32_t>(M);
    a.tab.wg_begin[i + 1] = a.tab.wg_begin[i] + desc->n_kv_heads * a.tab.ent[i].nsplit;
  }
}

int32_t run_select(const SelectArgs& a, int32_t cnt, hipStream_t s) {
  const int grid = a.tab.wg_begin[cnt];
  const hipError_t e = timed(SFI_K_SELECT, s, [&] { return launch_select(a, grid, s); });
  return e == hipSuccess ? SFI_OK : hip_fail(e, "select launch");
}

// The optional Selector steps: the final scores of every listed row's
// candidates into the extension's score buffer (key-norm correction when
// knorm is given, with the combine's statistics), then the radix top-k over
// those scores.  Timed with the Selector.
int32_t run_scored_select(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* ids, int32_t cnt,
                          const float* mass, const ExtLayout& E, char* w, bool knorm, SelectArgs& sa,
                          hipStream_t s) {
  ScoreArgs a{};
  a.mass = mass;
  a.knorm = knorm ? reinterpret_cast<const float*>(w + E.knorm) : nullptr;
  a.knorm_stat = reinterpret_cast<const double*>(w + E.knorm_stat);
  a.zpart = reinterpret_cast<const double*>(w + E.zpart);
  a.score = reinterpret_cast<float*>(w + E.score);
  a.t_cap = desc->kv_capacity;
  a.n_kv_heads = desc->n_kv_heads;
  a.n_sink = sp->n_sink;
  a.n_recent = sp->n_recent;
  a.zpart_stride = E.zpart_stride;
  a.chunk = score_chunk(desc, sp);
  a.lambda = sp->lambda;
  a.knorm_beta = sp->knorm_beta;
  a.knorm_c = sp->knorm_c;
  a.nms_radius = sp->nms_radius;
  a.nms_decay = sp->nms_decay;
  a.excl = sp->excl;
  a.tab.n = cnt;
  a.tab.ctx_dev = desc->ctx_len;
  a.tab.wg_begin[0] = 0;
  for (int i = 0; i < cnt; ++i) {
    const int64_t n = std::max<int64_t>(0, desc->ctx_len_host[ids[i]] - static_cast<int64_t>(sp->n_sink) - sp->n_recent);
    a.tab.ent[i].seq = ids[i];
    a.tab.ent[i].ctx = desc->ctx_len_host[ids[i]];
    a.tab.ent[i].nsplit = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(n, a.chunk)));
    a.tab.wg_begin[i + 1] = a.tab.wg_begin[i] + a.tab.ent[i].nsplit;
  }
  sa.mass = a.score;
  sa.pre_scores = true;
  sa.hist_ready = false;
  const int grid = a.tab.wg_begin[cnt];
  const hipError_t e = timed(SFI_K_SELECT, s, [&] {
    hipError_t x = launch_score(a, grid, s);
    return x == hipSuccess ? launch_select(sa, sa.tab.wg_begin[cnt], s) : x;
  });
  return e == hipSuccess ? SFI_OK : hip_fail(e, "select launch");
}

// The optional steps' constraints a call checks before it enqueues anything.
int32_t check_options(const sfi_kv_desc* desc, const sfi_support_params* sp) {
  if (sel_options(sp) && score_chunk(desc, sp) < 32)
    return fail(SFI_ERR_UNSUPPORTED, "n_kv_heads %d with nms_radius %d exceeds the score pass's LDS (n_kv_heads * "
                "(64 + 2 * nms_radius) + 32 <= 16384)", desc->n_kv_heads, sp->nms_radius);
  return SFI_OK;
}

}  // namespace

LaunchTiming* launch_timing() { return g_timing; }

}  // namespace sfi

using namespace sfi;

extern "C" {

int32_t sfi_version(void) { return SFI_VERSION_MAJOR * 100 + SFI_VERSION_MINOR; }

const char* sfi_status_str(int32_t st) {
  switch (st) {
    case SFI_OK: return "SFI_OK";
    case SFI_ERR_INVALID_ARG: return "SFI_ERR_INVALID_ARG";
    case SFI_ERR_UNSUPPORTED: return "SFI_ERR_UNSUPPORTED";
    case SFI_ERR_WORKSPACE: return "SFI_ERR_WORKSPACE";
    case SFI_ERR_HIP: return "SFI_ERR_HIP";
    case SFI_ERR_INJECTED: return "SFI_ERR_INJECTED";
    case SFI_ERR_NO_MEMORY: return "SFI_ERR_NO_MEMORY";
    default: return "SFI_ERR_UNKNOWN";
  }
}

const char* sfi_last_error(void) { return g_last_error.c_str(); }

size_t sfi_workspace_bytes(const sfi_kv_desc* desc, const sfi_support_params* sp, int32_t op) {
  if (check_desc(desc) != SFI_OK) return 0;
  switch (op) {
    case SFI_OP_SLOW: return slow_layout(desc).end;
    case SFI_OP_SELECT:
      if (check_params(sp) != SFI_OK) return 0;
      return sel_options(sp) ? ext_layout(desc, select_layout(desc).end).end : select_layout(desc).end;
    case SFI_OP_FAST:
      if (check_params(sp) != SFI_OK) return 0;
      return fast_layout(desc, sp).end;
    case SFI_OP_SLOW_SELECT: {
      if (check_params(sp) != SFI_OK) return 0;
      const size_t base = std::max(slow_layout(desc).end, select_layout(desc).end);
      return sel_options(sp) ? ext_layout(desc, base).end : base;
    }
    default: fail(SFI_ERR_INVALID_ARG, "unknown op %d", op); return 0;
  }
}

int32_t sfi_workspace_init(void* ws, size_t ws_bytes, void* stream) {
  if (ws == nullptr || ws_bytes == 0) return SFI_OK;
  if (const int32_t st = check_aligned({{ws, "workspace"}}, kVecAlign); st != SFI_OK) return st;
  const hipError_t e = launch_fill_zero(ws, ws_bytes, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SFI_OK : hip_fail(e, "workspace init");
}

int32_t sfi_slow_step(const sfi_kv_desc* desc, const int32_t* seq_ids, int32_t n_seq, const void* q, float* out,
                      float* mass, void* ws, size_t ws_bytes, void* stream) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_kv(desc)) != SFI_OK) return st;
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (n_seq == 0) return SFI_OK;
  if (q == nullptr || out == nullptr) return fail(SFI_ERR_INVALID_ARG, "q / out is NULL");
  if ((st = check_aligned({{q, "q"}, {out, "out"}, {mass, "mass"}}, kVecAlign)) != SFI_OK) return st;
  if ((st = check_ws(ws, ws_bytes, slow_layout(desc).end)) != SFI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    SlowArgs a{};
    CombineArgs c{};
    plan_slow(desc, ids, cnt, q, out, mass, mass != nullptr, w, a, c);
    return run_slow(desc, a, c, cnt, s);
  });
}

int32_t sfi_slow_plan(const sfi_kv_desc* desc, const int32_t* seq_ids, int32_t n_seq, int32_t with_mass,
                      int32_t* splits) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if (desc->ctx_len_host == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc->ctx_len_host is NULL");
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (n_seq == 0) return SFI_OK;
  if (splits == nullptr) return fail(SFI_ERR_INVALID_ARG, "splits is NULL");
  int32_t done = 0;
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    SlowArgs a{};
    CombineArgs c{};
    plan_slow(desc, ids, cnt, nullptr, nullptr, nullptr, with_mass != 0, nullptr, a, c);
    for (int i = 0; i < cnt; ++i) splits[done + i] = a.tab.ent[i].nsplit;
    done += cnt;
    return SFI_OK;
  });
}

int32_t sfi_fast_plan(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                      int32_t n_seq, int32_t* chunks) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_params(sp)) != SFI_OK) return st;
  if (desc->ctx_len_host == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc->ctx_len_host is NULL");
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (n_seq == 0) return SFI_OK;
  if (chunks == nullptr) return fail(SFI_ERR_INVALID_ARG, "chunks is NULL");
  const int crow = fast_chunk_rows();
  for (int32_t i = 0; i < n_seq; ++i) chunks[i] = fast_chunks(sp, desc->ctx_len_host[seq_ids[i]], crow);
  return SFI_OK;
}

int32_t sfi_select(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids, int32_t n_seq,
                   const float* mass, int32_t* sel_idx, int32_t* sel_cnt, void* ws, size_t ws_bytes,
                   void* stream) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_params(sp)) != SFI_OK) return st;
  if (desc->ctx_len_host == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc->ctx_len_host is NULL");
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (fault_injected("select")) return fail(SFI_ERR_INJECTED, "select failure forced by SFI_FAULT_INJECT");
  if (n_seq == 0) return SFI_OK;
  if (mass == nullptr || sel_cnt == nullptr || (sel_idx == nullptr && sp->top_k > 0))
    return fail(SFI_ERR_INVALID_ARG, "mass / sel_idx / sel_cnt is NULL");
  if ((st = check_aligned({{mass, "mass"}}, kVecAlign)) != SFI_OK) return st;
  if ((st = check_aligned({{sel_idx, "sel_idx"}, {sel_cnt, "sel_cnt"}}, kIntAlign)) != SFI_OK) return st;
  if (sp->knorm_beta > 0.f)
    return fail(SFI_ERR_UNSUPPORTED, "the key-norm prior needs the slow step's key norms: use sfi_slow_step_select");
  if ((st = check_options(desc, sp)) != SFI_OK) return st;
  const bool ext = sel_options(sp);
  const ExtLayout E = ext_layout(desc, select_layout(desc).end);
  if ((st = check_ws(ws, ws_bytes, ext ? E.end : select_layout(desc).end)) != SFI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    SelectArgs a{};
    plan_select(desc, sp, ids, cnt, mass, sel_idx, sel_cnt, w, a);
    return ext ? run_scored_select(desc, sp, ids, cnt, mass, E, w, false, a, s) : run_select(a, cnt, s);
  });
}

// Slow step + Selector (+ packing).  The Selector's kernels run on sel_s; when
// that is another stream it waits for the slow step's kernels on s, and with
// several launch groups the next group's slow step (which reuses the
// workspace) waits for the previous group's Selector.
static int32_t slow_step_select_impl(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                                     int32_t n_seq, const void* q, float* out, float* mass, int32_t* sel_idx,
                                     int32_t* sel_cnt, void* packed_k, void* packed_v, void* ws, size_t ws_bytes,
                                     hipStream_t s, hipStream_t sel_s) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_kv(desc)) != SFI_OK) return st;
  if ((st = check_params(sp)) != SFI_OK) return st;
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (fault_injected("select")) return fail(SFI_ERR_INJECTED, "select failure forced by SFI_FAULT_INJECT");
  if (n_seq == 0) return SFI_OK;
  if (q == nullptr || out == nullptr || mass == nullptr || sel_cnt == nullptr ||
      (sel_idx == nullptr && sp->top_k > 0))
    return fail(SFI_ERR_INVALID_ARG, "q / out / mass / sel_idx / sel_cnt is NULL");
  if ((packed_k == nullptr) != (packed_v == nullptr))
    return fail(SFI_ERR_INVALID_ARG, "packed_k and packed_v must both be given or both be NULL");
  if ((st = check_aligned({{q, "q"}, {out, "out"}, {mass, "mass"}, {packed_k, "packed_k"}, {packed_v, "packed_v"}},
                          kVecAlign)) != SFI_OK)
    return st;
  if ((st = check_aligned({{sel_idx, "sel_idx"}, {sel_cnt, "sel_cnt"}}, kIntAlign)) != SFI_OK) return st;
  if ((st = check_options(desc, sp)) != SFI_OK) return st;
  const bool ext = sel_options(sp), knorm = sp->knorm_beta > 0.f;
  const ExtLayout E = ext_layout(desc, std::max(slow_layout(desc).end, select_layout(desc).end));
  if ((st = check_ws(ws, ws_bytes, ext ? E.end : std::max(slow_layout(desc).end, select_layout(desc).end))) != SFI_OK)
    return st;
  const bool split = sel_s != s;
  hipEvent_t ev_slow = nullptr, ev_sel = nullptr;
  if (split && (!stream_event(0, &ev_slow) || !stream_event(1, &ev_sel)))
    return fail(SFI_ERR_HIP, "could not create the events that order the two streams");
  char* w = static_cast<char*>(ws);
  const Header H = header_layout(desc);
  bool first = true;
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    hipError_t e;
    if (split && !first && (e = hipStreamWaitEvent(s, ev_sel, 0)) != hipSuccess)
      return hip_fail(e, "stream wait");
    first = false;
    // the slow scratch and the Selector scratch overlap: the Selector's
    // kernels run after the combine has consumed the logits and partials
    SlowArgs a{};
    CombineArgs c{};
    plan_slow(desc, ids, cnt, q, out, mass, mass != nullptr, w, a, c);
    c.n_sink = sp->n_sink;
    c.n_recent = sp->n_recent;
    c.top_k = sp->top_k;
    c.lambda = sp->lambda;
    if (!ext) {
      // the combine builds the Selector's first histogram next to the mass
      a.clear_hist = reinterpret_cast<uint32_t*>(w + H.sel_hist);
      a.clear_list_n = reinterpret_cast<int32_t*>(w + H.sel_list_n);
      c.sel_hist = reinterpret_cast<uint32_t*>(w + H.sel_hist);
    } else if (knorm) {
      // the slow step emits key norms; the combine their statistics
      a.knorm = reinterpret_cast<float*>(w + E.knorm);
      a.knorm_part = reinterpret_cast<double*>(w + E.knorm_part);
      a.n_sink = sp->n_sink;
      a.n_recent = sp->n_recent;
      c.knorm = a.knorm;
      c.knorm_part = a.knorm_part;
      c.knorm_stat = reinterpret_cast<double*>(w + E.knorm_stat);
      c.zpart = reinterpret_cast<double*>(w + E.zpart);
      c.zpart_stride = E.zpart_stride;
      c.knorm_beta = sp->knorm_beta;
      c.knorm_c = sp->knorm_c;
    }
    int32_t r = run_slow(desc, a, c, cnt, s);
    if (r != SFI_OK) return r;
    if (split) {
      if ((e = hipEventRecord(ev_slow, s)) != hipSuccess) return hip_fail(e, "event record");
      if ((e = hipStreamWaitEvent(sel_s, ev_slow, 0)) != hipSuccess) return hip_fail(e, "stream wait");
    }
    SelectArgs sa{};
    plan_select(desc, sp, ids, cnt, mass, sel_idx, sel_cnt, w, sa);
    sa.hist_ready = true;
    if (packed_k != nullptr) {
      sa.k = desc->k;
      sa.v = desc->v;
      sa.packed_k = packed_k;
      sa.packed_v = packed_v;
      sa.row_bytes = desc->head_dim * elem_bytes(desc->kv_dtype);
      sa.rows32 = static_cast<uint64_t>(desc->kv_capacity) * sa.row_bytes <= kOutOfRange - 15 &&
                  static_cast<uint64_t>(sp->top_k) * sa.row_bytes <= kOutOfRange - 15;
    }
    r = ext ? run_scored_select(desc, sp, ids, cnt, mass, E, w, knorm, sa, sel_s) : run_select(sa, cnt, sel_s);
    if (r != SFI_OK) return r;
    if (split && (e = hipEventRecord(ev_sel, sel_s)) != hipSuccess) return hip_fail(e, "event record");
    return SFI_OK;
  });
}

int32_t sfi_slow_step_select(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                             int32_t n_seq, const void* q, float* out, float* mass, int32_t* sel_idx,
                             int32_t* sel_cnt, void* packed_k, void* packed_v, void* ws, size_t ws_bytes,
                             void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  return slow_step_select_impl(desc, sp, seq_ids, n_seq, q, out, mass, sel_idx, sel_cnt, packed_k, packed_v, ws,
                               ws_bytes, s, s);
}

int32_t sfi_slow_step_select_async(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                                   int32_t n_seq, const void* q, float* out, float* mass, int32_t* sel_idx,
                                   int32_t* sel_cnt, void* packed_k, void* packed_v, void* ws, size_t ws_bytes,
                                   void* stream, void* select_stream) {
  return slow_step_select_impl(desc, sp, seq_ids, n_seq, q, out, mass, sel_idx, sel_cnt, packed_k, packed_v, ws,
                               ws_bytes, static_cast<hipStream_t>(stream), static_cast<hipStream_t>(select_stream));
}

// Arguments of a fast step other than its scratch memory.  small_ids: the
// allocation-free check of at most kMaxSeqPerLaunch ids (no host heap use).
static int32_t check_fast(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                          int32_t n_seq, const void* q, const int32_t* sel_idx, const void* packed_k,
                          const void* packed_v, const int32_t* sel_cnt, const float* out, bool small_ids) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_kv(desc)) != SFI_OK) return st;
  if ((st = check_params(sp)) != SFI_OK) return st;
  if (small_ids) {
    if ((st = check_seqs_small(desc, seq_ids, n_seq, 1, desc->kv_capacity)) != SFI_OK) return st;
  } else if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) {
    return st;
  }
  if (n_seq == 0) return SFI_OK;
  if (q == nullptr || out == nullptr || sel_cnt == nullptr)
    return fail(SFI_ERR_INVALID_ARG, "q / out / sel_cnt is NULL");
  if (sel_idx == nullptr && (packed_k == nullptr || packed_v == nullptr) && sp->top_k > 0)
    return fail(SFI_ERR_INVALID_ARG, "sel_idx (or packed_k / packed_v) is NULL");
  if (sp->n_sink == 0 && sp->n_recent == 0 && sp->top_k == 0)
    return fail(SFI_ERR_INVALID_ARG, "the support is empty (n_sink = n_recent = top_k = 0)");
  if ((st = check_aligned({{q, "q"}, {out, "out"}, {packed_k, "packed_k"}, {packed_v, "packed_v"}}, kVecAlign)) !=
      SFI_OK)
    return st;
  if ((st = check_aligned({{sel_idx, "sel_idx"}, {sel_cnt, "sel_cnt"}}, kIntAlign)) != SFI_OK) return st;
  const int crow = fast_chunk_rows();
  if (static_cast<int64_t>(sp->n_sink) + sp->n_recent + sp->top_k > static_cast<int64_t>(crow) * kMaxMergeSlots)
    return fail(SFI_ERR_UNSUPPORTED, "support of %lld rows exceeds %d",
                static_cast<long long>(sp->n_sink) + sp->n_recent + sp->top_k, crow * kMaxMergeSlots);
  return SFI_OK;
}

// One launch group of a fast step: the sparse-attention kernel, and the merge
// kernel when the launch does not fit the GPU in one pass.  part_ml / part_o /
// ticket: the chunk states and per-head counters (zero) for up to cnt rows.
static int32_t launch_fast_group(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* ids,
                                 int32_t cnt, const void* q, const int32_t* sel_idx, const void* packed_k,
                                 const void* packed_v, const int32_t* sel_cnt, float* out, float* part_ml,
                                 float* part_o, int32_t* ticket, hipStream_t s, bool timing,
                                 void* pack_out_k = nullptr, void* pack_out_v = nullptr, uint64_t pack_mask = ~0ull) {
  const int G = desc->n_q_heads / desc->n_kv_heads;
  const int crow = fast_chunk_rows();
  FastArgs a{};
  a.k = desc->k;
  a.v = desc->v;
  a.packed_k = packed_k;
  a.packed_v = packed_v;
  a.q = q;
  a.sel_idx = sel_idx;
  a.sel_cnt = sel_cnt;
  a.pack_out_k = pack_out_k;
  a.pack_out_v = pack_out_v;
  if (pack_out_k != nullptr) {
    // rows that pack gather through sel_idx; the others read the packed
    // buffers (written by an earlier call); both kinds: one mixed launch
    const uint64_t all = cnt >= 64 ? ~0ull : (1ull << cnt) - 1;
    pack_mask &= all;
    if (pack_mask == 0) {
      a.packed_k = pack_out_k;
      a.packed_v = pack_out_v;
      a.pack_out_k = a.pack_out_v = nullptr;
    } else if (pack_mask != all) {
      a.packed_k = pack_out_k;
      a.packed_v = pack_out_v;
      a.pack_mask = pack_mask;
    }
  }
  a.part_ml = part_ml;
  a.part_o = part_o;
  a.out = out;
  a.t_cap = desc->kv_capacity;
  a.n_q_heads = desc->n_q_heads;
  a.n_kv_heads = desc->n_kv_heads;
  a.n_sink = sp->n_sink;
  a.n_recent = sp->n_recent;
  a.top_k = sp->top_k;
  a.chunk_rows = crow;
  a.part_stride = fast_part_stride(sp);
  a.scale_log2 = logit_scale(desc);
  a.tab.n = cnt;
  a.tab.ctx_dev = desc->ctx_len;
  a.tab.wg_begin[0] = 0;
  for (int i = 0; i < cnt; ++i) {
    const int b = ids[i];
    a.tab.ent[i].seq = b;
    a.tab.ent[i].ctx = desc->ctx_len_host[b];
    a.tab.ent[i].nsplit = fast_chunks(sp, desc->ctx_len_host[b], crow);
    a.tab.wg_begin[i + 1] = a.tab.wg_begin[i] + desc->n_kv_heads * a.tab.ent[i].nsplit;
  }
  // a launch that fits the chip in one pass merges its chunks in the same
  // kernel; a larger one hands them to the merge kernel
  const int grid = a.tab.wg_begin[cnt];
  int cus = 0;
  if (!compute_units(&cus)) return fail(SFI_ERR_HIP, "could not query the device's compute units");
  const bool fused = grid <= cus;
  a.ticket = fused ? ticket : nullptr;
  auto partial = [&] { return launch_fast_partial(a, desc->kv_dtype, desc->head_dim, G, grid, s); };
  auto merge = [&] { return launch_fast_merge(a, desc->head_dim, G, s); };
  hipError_t e = timing ? timed(a.pack_out_k != nullptr ? SFI_K_FAST_PACK : SFI_K_FAST, s, partial) : partial();
  if (e == hipSuccess && !fused) e = timing ? timed(SFI_K_FAST_MERGE, s, merge) : merge();
  return e == hipSuccess ? SFI_OK : hip_fail(e, "fast launch");
}

static int32_t fast_step_impl(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                              int32_t n_seq, const void* q, const int32_t* sel_idx, const void* packed_k,
                              const void* packed_v, const int32_t* sel_cnt, float* out, void* ws, size_t ws_bytes,
                              void* stream, void* pack_out_k = nullptr, void* pack_out_v = nullptr,
                              const int32_t* pack_flags = nullptr) {
  int32_t st = check_fast(desc, sp, seq_ids, n_seq, q, sel_idx, packed_k, packed_v, sel_cnt, out, false);
  if (st != SFI_OK || n_seq == 0) return st;
  const FastLayout L = fast_layout(desc, sp);
  if ((st = check_ws(ws, ws_bytes, L.end)) != SFI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    static_assert(kMaxSeqPerLaunch <= 64, "one pack_mask bit per table entry");
    uint64_t mask = ~0ull;
    if (pack_flags != nullptr) {
      mask = 0;
      for (int32_t i = 0; i < cnt; ++i)
        if (pack_flags[(ids - seq_ids) + i] != 0) mask |= 1ull << i;
    }
    return launch_fast_group(desc, sp, ids, cnt, q, sel_idx, packed_k, packed_v, sel_cnt, out,
                             reinterpret_cast<float*>(w + L.part_ml), reinterpret_cast<float*>(w + L.part_o),
                             reinterpret_cast<int32_t*>(w + header_layout(desc).fast_ticket), s, true, pack_out_k,
                             pack_out_v, mask);
  });
}

int32_t sfi_fast_step(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids, int32_t n_seq,
                      const void* q, const int32_t* sel_idx, const int32_t* sel_cnt, float* out, void* ws,
                      size_t ws_bytes, void* stream) {
  if (sel_idx == nullptr && sp != nullptr && sp->top_k > 0) return fail(SFI_ERR_INVALID_ARG, "sel_idx is NULL");
  return fast_step_impl(desc, sp, seq_ids, n_seq, q, sel_idx, nullptr, nullptr, sel_cnt, out, ws, ws_bytes, stream);
}

int32_t sfi_fast_step_pack(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                           int32_t n_seq, const int32_t* pack_flags, const void* q, const int32_t* sel_idx,
                           const int32_t* sel_cnt, float* out, void* packed_k, void* packed_v, void* ws,
                           size_t ws_bytes, void* stream) {
  if (sp != nullptr && sp->top_k > 0) {
    if (sel_idx == nullptr) return fail(SFI_ERR_INVALID_ARG, "sel_idx is NULL");
    if (packed_k == nullptr || packed_v == nullptr) return fail(SFI_ERR_INVALID_ARG, "packed_k / packed_v is NULL");
    int32_t st;
    if ((st = check_aligned({{packed_k, "packed_k"}, {packed_v, "packed_v"}}, kVecAlign)) != SFI_OK) return st;
  }
  const bool pack = sp != nullptr && sp->top_k > 0;
  return fast_step_impl(desc, sp, seq_ids, n_seq, q, sel_idx, nullptr, nullptr, sel_cnt, out, ws, ws_bytes, stream,
                        pack ? packed_k : nullptr, pack ? packed_v : nullptr, pack_flags);
}

int32_t sfi_fast_step_packed(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                             int32_t n_seq, const void* q, const void* packed_k, const void* packed_v,
                             const int32_t* sel_cnt, float* out, void* ws, size_t ws_bytes, void* stream) {
  if ((packed_k == nullptr || packed_v == nullptr) && sp != nullptr && sp->top_k > 0)
    return fail(SFI_ERR_INVALID_ARG, "packed_k / packed_v is NULL");
  return fast_step_impl(desc, sp, seq_ids, n_seq, q, nullptr, packed_k, packed_v, sel_cnt, out, ws, ws_bytes,
                        stream);
}

int32_t sfi_fast_step_packed_noalloc(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                                     int32_t n_seq, const void* q, const void* packed_k, const void* packed_v,
                                     const int32_t* sel_cnt, float* out, void* stream) {
  if ((packed_k == nullptr || packed_v == nullptr) && sp != nullptr && sp->top_k > 0)
    return fail(SFI_ERR_INVALID_ARG, "packed_k / packed_v is NULL");
  int32_t st = check_fast(desc, sp, seq_ids, n_seq, q, nullptr, packed_k, packed_v, sel_cnt, out, true);
  if (st != SFI_OK || n_seq == 0) return st;
  // the chunk states of n_seq rows, after the counter block
  const size_t heads = static_cast<size_t>(n_seq) * desc->n_q_heads;
  const size_t stride = static_cast<size_t>(fast_part_stride(sp));
  const size_t ml_bytes = align_up(heads * stride * 2 * sizeof(float));
  const size_t o_bytes = align_up(heads * stride * desc->head_dim * sizeof(float));
  if (static_cast<size_t>(n_seq) * desc->n_kv_heads > kNoAllocCounters)
    return fail(SFI_ERR_UNSUPPORTED, "n_seq * n_kv_heads = %zu exceeds %d (the fixed scratch's counters)",
                static_cast<size_t>(n_seq) * desc->n_kv_heads, kNoAllocCounters);
  if (kNoAllocCounterBytes + ml_bytes + o_bytes > SFI_NOALLOC_SCRATCH_BYTES)
    return fail(SFI_ERR_UNSUPPORTED, "the chunk states of this call need %zu bytes; the fixed scratch holds %zu",
                kNoAllocCounterBytes + ml_bytes + o_bytes, static_cast<size_t>(SFI_NOALLOC_SCRATCH_BYTES));
  hipStream_t s = static_cast<hipStream_t>(stream);
  char* w = nullptr;
  if ((st = noalloc_scratch(s, &w)) != SFI_OK) return st;
  return launch_fast_group(desc, sp, seq_ids, n_seq, q, nullptr, packed_k, packed_v, sel_cnt, out,
                           reinterpret_cast<float*>(w + kNoAllocCounterBytes),
                           reinterpret_cast<float*>(w + kNoAllocCounterBytes + ml_bytes),
                           reinterpret_cast<int32_t*>(w), s, false);
}

int32_t sfi_pack_support(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                         int32_t n_seq, const int32_t* sel_idx, const int32_t* sel_cnt, void* packed_k,
                         void* packed_v, void* stream) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_kv(desc)) != SFI_OK) return st;
  if ((st = check_params(sp)) != SFI_OK) return st;
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (n_seq == 0 || sp->top_k == 0) return SFI_OK;
  if (sel_idx == nullptr || sel_cnt == nullptr || packed_k == nullptr || packed_v == nullptr)
    return fail(SFI_ERR_INVALID_ARG, "sel_idx / sel_cnt / packed_k / packed_v is NULL");
  if ((st = check_aligned({{packed_k, "packed_k"}, {packed_v, "packed_v"}}, kVecAlign)) != SFI_OK) return st;
  if ((st = check_aligned({{sel_idx, "sel_idx"}, {sel_cnt, "sel_cnt"}}, kIntAlign)) != SFI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    PackArgs a{};
    a.k = desc->k;
    a.v = desc->v;
    a.packed_k = packed_k;
    a.packed_v = packed_v;
    a.sel_idx = sel_idx;
    a.sel_cnt = sel_cnt;
    a.t_cap = desc->kv_capacity;
    a.n_kv_heads = desc->n_kv_heads;
    a.n_sink = sp->n_sink;
    a.n_recent = sp->n_recent;
    a.top_k = sp->top_k;
    a.tab.n = cnt;
    a.tab.ctx_dev = desc->ctx_len;
    a.tab.wg_begin[0] = 0;
    for (int i = 0; i < cnt; ++i) {
      const int64_t t = desc->ctx_len_host[ids[i]];
      const int64_t kmax = std::min<int64_t>(sp->top_k, std::max<int64_t>(0, t - sp->n_sink - sp->n_recent));
      a.tab.ent[i].seq = ids[i];
      a.tab.ent[i].ctx = static_cast<int32_t>(t);
      a.tab.ent[i].nsplit = static_cast<int32_t>(std::max<int64_t>(1, ceil_div(kmax, kPackRows)));
      a.tab.wg_begin[i + 1] = a.tab.wg_begin[i] + desc->n_kv_heads * a.tab.ent[i].nsplit;
    }
    const hipError_t e = timed(SFI_K_PACK, s, [&] {
      return launch_pack(a, desc->kv_dtype, desc->head_dim, a.tab.wg_begin[cnt], s);
    });
    return e == hipSuccess ? SFI_OK : hip_fail(e, "pack launch");
  });
}

int32_t sfi_kv_append(const sfi_kv_desc* desc, const int32_t* seq_ids, int32_t n_seq, const void* k_new,
                      const void* v_new, void* stream) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_kv(desc)) != SFI_OK) return st;
  // with device context lengths the host values are only bounds: the kernel
  // skips a row whose device length has reached the capacity
  const int64_t max_t = desc->ctx_len != nullptr ? desc->kv_capacity : desc->kv_capacity - 1;
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 0, max_t)) != SFI_OK) return st;
  if (n_seq == 0) return SFI_OK;
  if (k_new == nullptr || v_new == nullptr) return fail(SFI_ERR_INVALID_ARG, "k_new / v_new is NULL");
  if ((st = check_aligned({{k_new, "k_new"}, {v_new, "v_new"}}, kVecAlign)) != SFI_OK) return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    AppendArgs a{};
    a.k = desc->k;
    a.v = desc->v;
    a.k_new = k_new;
    a.v_new = v_new;
    a.t_cap = desc->kv_capacity;
    a.n_kv_heads = desc->n_kv_heads;
    a.tab.n = cnt;
    a.tab.ctx_dev = desc->ctx_len;
    for (int i = 0; i < cnt; ++i) {
      a.tab.ent[i].seq = ids[i];
      a.tab.ent[i].ctx = desc->ctx_len_host[ids[i]];
      a.tab.ent[i].nsplit = 1;
      a.tab.wg_begin[i] = i;
    }
    a.tab.wg_begin[cnt] = cnt;
    const hipError_t e = timed(SFI_K_APPEND, s, [&] {
      return launch_append(a, desc->kv_dtype, desc->head_dim, cnt, s);
    });
    return e == hipSuccess ? SFI_OK : hip_fail(e, "append launch");
  });
}

int32_t sfi_debug_support(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids,
                          int32_t n_seq, const int32_t* sel_idx, const int32_t* sel_cnt, int32_t* support_out,
                          int32_t* support_cnt, int32_t cap_per_head, void* stream) {
  int32_t st;
  if ((st = check_desc(desc)) != SFI_OK) return st;
  if ((st = check_params(sp)) != SFI_OK) return st;
  if (desc->ctx_len_host == nullptr) return fail(SFI_ERR_INVALID_ARG, "desc->ctx_len_host is NULL");
  if ((st = check_seqs(desc, seq_ids, n_seq, true, 1, desc->kv_capacity)) != SFI_OK) return st;
  if (n_seq == 0) return SFI_OK;
  if (sel_idx == nullptr || sel_cnt == nullptr || support_out == nullptr || support_cnt == nullptr)
    return fail(SFI_ERR_INVALID_ARG, "NULL buffer");
  if (cap_per_head < 1) return fail(SFI_ERR_INVALID_ARG, "cap_per_head must be >= 1");
  if ((st = check_aligned({{sel_idx, "sel_idx"}, {sel_cnt, "sel_cnt"}, {support_out, "support_out"},
                           {support_cnt, "support_cnt"}}, kIntAlign)) != SFI_OK)
    return st;
  hipStream_t s = static_cast<hipStream_t>(stream);
  return for_each_group(seq_ids, n_seq, [&](const int32_t* ids, int32_t cnt) -> int32_t {
    SupportArgs a{};
    a.sel_idx = sel_idx;
    a.sel_cnt = sel_cnt;
    a.support_out = support_out;
    a.support_cnt = support_cnt;
    a.t_cap = desc->kv_capacity;
    a.n_kv_heads = desc->n_kv_heads;
    a.n_sink = sp->n_sink;
    a.n_recent = sp->n_recent;
    a.top_k = sp->top_k;
    a.cap_per_head = cap_per_head;
    a.tab.n = cnt;
    a.tab.ctx_dev = desc->ctx_len;
    for (int i = 0; i < cnt; ++i) {
      a.tab.ent[i].seq = ids[i];
      a.tab.ent[i].ctx = desc->ctx_len_host[ids[i]];
      a.tab.ent[i].nsplit = 1;
      a.tab.wg_begin[i] = i * desc->n_kv_heads;
    }
    a.tab.wg_begin[cnt] = cnt * desc->n_kv_heads;
    const hipError_t e = launch_support(a, cnt * desc->n_kv_heads, s);
    return e == hipSuccess ? SFI_OK : hip_fail(e, "support launch");
  });
}

int32_t sfi_profile_enable(int32_t on) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on = on != 0;
  return SFI_OK;
}

static int32_t drain_profile(Prof& p) {
  for (int k = 0; k < SFI_K_COUNT; ++k) {
    for (auto& pr : p.pending[k]) {
      hipError_t e = hipEventSynchronize(pr.second);
      if (e != hipSuccess) return hip_fail(e, "profile event sync");
      float ms = 0.f;
      e = hipEventElapsedTime(&ms, pr.first, pr.second);
      if (e != hipSuccess) return hip_fail(e, "profile elapsed time");
      p.ms[k] += ms;
      p.launches[k] += 1;
      p.pool.push_back(pr.first);
      p.pool.push_back(pr.second);
    }
    p.pending[k].clear();
  }
  return SFI_OK;
}

int32_t sfi_profile_reset(void) {
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  const int32_t st = drain_profile(p);
  for (int k = 0; k < SFI_K_COUNT; ++k) {
    p.ms[k] = 0.0;
    p.launches[k] = 0;
  }
  return st;
}

int32_t sfi_profile_read(int32_t kernel, double* total_ms, int64_t* launches) {
  if (kernel < 0 || kernel >= SFI_K_COUNT) return fail(SFI_ERR_INVALID_ARG, "unknown kernel id %d", kernel);
  if (total_ms == nullptr || launches == nullptr) return fail(SFI_ERR_INVALID_ARG, "NULL output");
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  const int32_t st = drain_profile(p);
  if (st != SFI_OK) return st;
  *total_ms = p.ms[kernel];
  *launches = p.launches[kernel];
  return SFI_OK;
}

}  // extern "C"
