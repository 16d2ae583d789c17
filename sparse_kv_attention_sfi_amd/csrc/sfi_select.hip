// Selector kernels of the SFI path for gfx950 ("Slow-Fast Inference ...",
// gist.science technical summary, 2.B "Der Training-Free Selector").
//
// For each (sequence, KV head) the n candidate positions [n_sink, T - n_recent)
// get the fused score
//     s = (1 - lambda) * f + lambda * r,   r(a) = (1/a + 1/(n+1-a)) / (2 H_n)
// (the closed-form mixture of the slow step's mass f with the prior r; a is
// the 1-based offset from the sinks), and the k best are kept.  Exact top-k
// uses a 64-bit key that makes every candidate distinct:
//     key = order-preserving bits of s  << 32  |  ~position
// so "larger key" means "higher score, or equal score and lower position";
// the kept set is {key >= K*} with K* the k-th largest key.
//
// The candidates of a head are cut into chunks handled by separate
// workgroups, so the selection of one head spreads over many CUs:
//   0. the head's histogram and list counter start at zero (cleared by
//      select_clear, or by the slow step's partial kernel in the fused call)
//   1. histogram of the top 12 key bits, added into a per-head global
//      histogram (select_hist, or the slow step's combine in the fused call).
//   2. select_gather: every workgroup finds the bin d1 holding K*, lists the
//      positions of its keys above d1 (all of them are kept) with their count,
//      and appends its keys in d1 to a per-head list (one atomic per workgroup
//      reserves its range).
//   3. select_emit: every workgroup resolves K* inside the list in LDS (by
//      direct ranking when the list is short, else 12 bits per level), derives
//      how many kept keys precede its chunk, and writes the kept positions of
//      its chunk (its listed keys above d1 and its list keys at or above K*)
//      in ascending order from there; when the refresh also packs, it copies
//      their K and V rows into the packed buffers at the same slots.  If d1
//      holds more keys than fit in LDS, K* comes from radix passes over all
//      candidates instead.
//  With the optional key-norm prior, Soft-NMS or exclusivity, select_score
//  first writes the final scores, and the steps above rank those.
// Resolving K* redundantly in every emitting workgroup costs less than a
// kernel boundary.  Workgroups never hand data to each other inside a
// kernel: on gfx950 a device-scope fence writes back and invalidates the
// XCD's L2.
#include <math.h>

#include "sfi_device.hpp"
#include "sfi_internal.hpp"
#include "sfi_score.hpp"

namespace sfi {

constexpr int kSelWaves = kSelThreads / 64;

// Exclusive prefix sum over the workgroup in thread order; *total gets the sum.
__device__ __forceinline__ int block_excl_scan(int v, int* s_wave, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave[wave] = incl;
  __syncthreads();
  int before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const int x = s_wave[w];
    before += (w < wave) ? x : 0;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

struct HeadCtx {
  int e, g, c, b, T, n, M;
  int64_t bg;
  bool keep_all;
};

__device__ __forceinline__ HeadCtx head_ctx(const SelectArgs& a) {
  HeadCtx h;
  const int wg = blockIdx.x;
  h.e = find_entry(a.tab, wg);
  const int local = wg - a.tab.wg_begin[h.e];
  h.M = a.tab.ent[h.e].nsplit;
  // consecutive workgroups take the same chunk of consecutive KV heads: with
  // workgroups dealt round-robin to the XCDs, all chunks of one head then
  // share an XCD (when the head count divides by the XCD count), so its
  // histogram, lists and counts are fetched into one L2 only
  h.g = local % a.n_kv_heads;
  h.c = local / a.n_kv_heads;
  h.b = a.tab.ent[h.e].seq;
  h.T = row_ctx(a.tab, h.e);
  h.bg = static_cast<int64_t>(h.b) * a.n_kv_heads + h.g;
  h.n = max(0, h.T - a.n_recent - a.n_sink);
  h.keep_all = h.n <= a.top_k || a.top_k == 0;
  return h;
}

__device__ __forceinline__ ScoreParams score_params(const SelectArgs& a, const HeadCtx& h, float inv2h) {
  ScoreParams sp;
  sp.f = a.mass + h.bg * a.t_cap + a.n_sink;
  sp.pre = a.pre_scores;
  sp.n = h.n;
  sp.lo = a.n_sink;
  sp.lambda = a.lambda;
  sp.one_minus_lambda = 1.0f - a.lambda;
  sp.inv_2h = inv2h;
  return sp;
}

// Digit d of a histogram (highest bins first) with
// (count in higher bins) < need <= (count in higher bins) + hist[d].
// Writes the digit and the count above it to s_res[0], s_res[1].
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nbins, int need, int* s_wave,
                                           int* s_res) {
  const int tid = threadIdx.x;
  const int per = (nbins + kSelThreads - 1) / kSelThreads;
  const int b0 = (kSelThreads - 1 - tid) * per;  // thread 0 owns the highest bins
  int local = 0;
  for (int u = 0; u < per; ++u)
    if (b0 + u < nbins) local += static_cast<int>(hist[b0 + u]);
  int tot;
  const int above_me = block_excl_scan(local, s_wave, &tot);
  if (above_me < need && need <= above_me + local) {
    int run = above_me;
    for (int u = per - 1; u >= 0; --u) {
      const int bin = b0 + u;
      if (bin >= nbins) continue;
      const int c = static_cast<int>(hist[bin]);
      if (run + c >= need) {
        s_res[0] = bin;
        s_res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

// find_digit over the 4096-bin top-digit histogram read straight from global
// memory into registers: thread t holds bins 8 (kSelThreads - 1 - t) ... + 7
// (thread 0 the highest), loaded as two 16-byte pieces.
static_assert(kSelBins == 8 * kSelThreads, "eight top-digit bins per thread");
__device__ __forceinline__ void load_top_bins(const uint32_t* ghist, uint32_t (&hv)[8]) {
  const int b0 = (kSelThreads - 1 - threadIdx.x) * 8;
  const uint4 lo = reinterpret_cast<const uint4*>(ghist + b0)[0];
  const uint4 hi = reinterpret_cast<const uint4*>(ghist + b0)[1];
  hv[0] = lo.x; hv[1] = lo.y; hv[2] = lo.z; hv[3] = lo.w;
  hv[4] = hi.x; hv[5] = hi.y; hv[6] = hi.z; hv[7] = hi.w;
}
__device__ __forceinline__ void find_top_digit(const uint32_t (&hv)[8], int need, int* s_wave, int* s_res) {
  const int tid = threadIdx.x;
  const int b0 = (kSelThreads - 1 - tid) * 8;
  int local = 0;
#pragma unroll
  for (int u = 0; u < 8; ++u) local += static_cast<int>(hv[u]);
  int tot;
  const int above_me = block_excl_scan(local, s_wave, &tot);
  if (above_me < need && need <= above_me + local) {
    int run = above_me;
#pragma unroll
    for (int u = 7; u >= 0; --u) {
      const int c = static_cast<int>(hv[u]);
      if (run + c >= need) {
        s_res[0] = b0 + u;
        s_res[1] = run;
        break;
      }
      run += c;
    }
  }
  __syncthreads();
}

// K* among the m threshold-bin keys in LDS (m <= kSelListCap): the key with
// exactly need - 1 larger keys.  The bits below the top digit are resolved
// 8 at a time: the keys that match the resolved prefix are histogrammed into
// 256 LDS bins and one wave scans them; once at most 64 keys match the
// prefix, they are gathered and one wave ranks them.  s_h: 256 words,
// s_small: 64 keys, s_res: 4 ints.
__device__ uint64_t list_resolve(const uint64_t* keys, int m, int need, uint64_t prefix, uint64_t pmask, int shift,
                                 uint32_t* s_h, uint64_t* s_small, int* s_res, uint64_t* s_key) {
  const int tid = threadIdx.x, lane = tid & 63;
  int match = m;
  while (match > 64 && shift > 0) {
    const int width = shift >= 8 ? 8 : shift;
    shift -= width;
    const uint32_t dmask = (1u << width) - 1u;
    if (tid < 256) s_h[tid] = 0u;
    __syncthreads();
    for (int i = tid; i < m; i += kSelThreads) {
      const uint64_t key = keys[i];
      if ((key & pmask) == prefix) atomicAdd(&s_h[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    if (tid < 64) {
      // lane l: bins 255 - 4 l (first) down to 252 - 4 l
      const uint4 h4 = reinterpret_cast<const uint4*>(s_h)[63 - lane];
      const int hb[4] = {static_cast<int>(h4.w), static_cast<int>(h4.z), static_cast<int>(h4.y),
                         static_cast<int>(h4.x)};
      const int c = hb[0] + hb[1] + hb[2] + hb[3];
      int incl = c;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_up(incl, d, 64);
        if (lane >= d) incl += y;
      }
      int run = incl - c;
      if (run < need && need <= incl) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (run + hb[u] >= need) {
            s_res[0] = 255 - 4 * lane - u;
            s_res[1] = run;
            s_res[2] = hb[u];
            break;
          }
          run += hb[u];
        }
      }
    }
    __syncthreads();
    const int digit = s_res[0];
    need -= s_res[1];
    match = s_res[2];
    prefix |= static_cast<uint64_t>(digit) << shift;
    pmask |= static_cast<uint64_t>(dmask) << shift;
    __syncthreads();
  }
  if (tid == 0) s_res[3] = 0;
  __syncthreads();
  for (int i = tid; i < m; i += kSelThreads) {
    const uint64_t key = keys[i];
    if ((key & pmask) == prefix) {
      const int slot = atomicAdd(&s_res[3], 1);
      if (slot < 64) s_small[slot] = key;
    }
  }
  __syncthreads();
  if (tid < 64) {
    const int cnt = min(s_res[3], 64);
    const uint64_t mine = lane < cnt ? s_small[lane] : 0ull;
    int rank = 0;
    for (int j = 0; j < cnt; ++j) rank += s_small[j] > mine;
    if (lane < cnt && rank == need - 1) *s_key = mine;
  }
  __syncthreads();
  return *s_key;
}

// Exclusive prefix sum over the workgroup of two counters at once (64-bit
// lanes: a in the high word, b in the low word); *total gets both sums.
__device__ __forceinline__ uint64_t block_excl_scan2(uint32_t a, uint32_t b, uint64_t* s_wave2, uint64_t* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint64_t v = (static_cast<uint64_t>(a) << 32) | b;
  uint64_t incl = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const uint64_t y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) s_wave2[wave] = incl;
  __syncthreads();
  uint64_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kSelWaves; ++w) {
    const uint64_t x = s_wave2[w];
    before += (w < wave) ? x : 0ull;
    all += x;
  }
  __syncthreads();
  *total = all;
  return before + incl - v;
}

// Among m <= kSelThreads distinct keys in LDS (16-byte aligned), the one with
// exactly need - 1 larger keys.  The list is cut into P = kSelThreads / m
// parts; thread t counts the keys of part t / m that exceed key t % m (eight
// keys per step, broadcast 16-byte LDS reads), and the P partial ranks are
// summed through LDS.  s_part holds kSelThreads ints.
__device__ __forceinline__ uint64_t rank_select(const uint64_t* keys, int m, int need, int* s_part,
                                                uint64_t* s_out) {
  const int tid = threadIdx.x;
  const int parts = m > 0 ? kSelThreads / m : 1;
  const int span = ((m + parts - 1) / parts + 7) & ~7;  // keys per part, a multiple of 8
  const int i = m > 0 ? tid % m : 0, part = m > 0 ? tid / m : parts;
  if (part < parts) {
    const uint64_t mine = keys[i];
    const int j0 = min(m, part * span), j1 = min(m, j0 + span);
    int rank = 0;
    const int j8 = j0 + ((j1 - j0) & ~7);
    for (int j = j0; j < j8; j += 8) {
      const ulonglong2* p = reinterpret_cast<const ulonglong2*>(keys + j);
      const ulonglong2 a = p[0], b = p[1], c = p[2], d = p[3];
      rank += (a.x > mine) + (a.y > mine) + (b.x > mine) + (b.y > mine) + (c.x > mine) + (c.y > mine) +
              (d.x > mine) + (d.y > mine);
    }
    for (int j = j8; j < j1; ++j) rank += keys[j] > mine;
    s_part[tid] = rank;
  }
  __syncthreads();
  if (tid < m) {
    int rank = 0;
    for (int p = 0; p < parts; ++p) rank += s_part[p * m + tid];
    if (rank == need - 1) *s_out = keys[tid];
  }
  __syncthreads();
  return *s_out;
}

// Resolves the remaining digits of K* (below `shift`) among the `match` keys
// that equal `prefix` on `pmask`; keys come from `src(i)` for i < count.  Each
// level histograms the next (up to) 12 bits; as soon as at most kSelThreads
// keys share the resolved prefix they are gathered into LDS and ranked.
// s_hist must be 16-byte aligned (its first 4 KiB also hold the gathered keys).
template <typename Src>
__device__ uint64_t radix_resolve(Src src, int count, int match, uint64_t prefix, uint64_t pmask, int shift,
                                  int need, uint32_t* s_hist, int* s_wave, int* s_res, uint64_t* s_key) {
  const int tid = threadIdx.x;
  while (shift > 0) {
    if (match <= kSelThreads) {
      uint64_t* small = reinterpret_cast<uint64_t*>(s_hist);
      if (tid == 0) s_res[0] = 0;
      __syncthreads();
      for (int i = tid; i < count; i += kSelThreads) {
        const uint64_t key = src(i);
        if ((key & pmask) == prefix) small[atomicAdd(&s_res[0], 1)] = key;
      }
      __syncthreads();
      // partial ranks after the gathered keys (kSelThreads 64-bit keys = 2 kSelThreads words)
      const uint64_t k = rank_select(small, match, need, reinterpret_cast<int*>(s_hist) + 2 * kSelThreads, s_key);
      __syncthreads();
      return k;
    }
    const int width = shift >= kSelDigitBits ? kSelDigitBits : shift;
    shift -= width;
    const uint32_t dmask = (1u << width) - 1u;
    const int nbins = 1 << width;
    for (int i = tid; i < nbins; i += kSelThreads) s_hist[i] = 0u;
    __syncthreads();
    for (int i = tid; i < count; i += kSelThreads) {
      const uint64_t key = src(i);
      if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dmask], 1u);
    }
    __syncthreads();
    find_digit(s_hist, nbins, need, s_wave, s_res);
    const int digit = s_res[0];
    need -= s_res[1];
    match = static_cast<int>(s_hist[digit]);
    prefix |= static_cast<uint64_t>(digit) << shift;
    pmask |= static_cast<uint64_t>(dmask) << shift;
    __syncthreads();
  }
  return prefix;
}

// ---------------------------------------------------------------------------
// 0. clear the per-head bookkeeping (one workgroup per listed head)
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void select_clear_kernel(SelectArgs a) {
  const int e = blockIdx.x / a.n_kv_heads;
  const int g = blockIdx.x - e * a.n_kv_heads;
  const int64_t bg = static_cast<int64_t>(a.tab.ent[e].seq) * a.n_kv_heads + g;
  uint4* h4 = reinterpret_cast<uint4*>(a.hist + bg * kSelBins);
  for (int i = threadIdx.x; i < kSelBins / 4; i += 256) h4[i] = make_uint4(0u, 0u, 0u, 0u);
  if (threadIdx.x == 0) a.list_n[bg] = 0;
}

// ---------------------------------------------------------------------------
// 1. histogram of the top digit
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kSelThreads) void select_hist_kernel(SelectArgs a) {
  __shared__ uint32_t s_hist[kSelBins];
  __shared__ float s_inv2h;
  const HeadCtx h = head_ctx(a);
  if (h.keep_all) return;
  const int tid = threadIdx.x;
  if (tid == 0) s_inv2h = static_cast<float>(1.0 / (2.0 * harmonic_number(h.n)));
  for (int i = tid; i < kSelBins; i += kSelThreads) s_hist[i] = 0u;
  __syncthreads();
  const ScoreParams sp = score_params(a, h, s_inv2h);
  const int i0 = h.c * a.chunk, i1 = min(h.n, i0 + a.chunk);
  for (int i = i0 + tid; i < i1; i += kSelThreads) atomicAdd(&s_hist[top_digit(cand_key(sp, i))], 1u);
  __syncthreads();
  uint32_t* gh = a.hist + h.bg * kSelBins;
  for (int i = tid; i < kSelBins; i += kSelThreads)
    if (s_hist[i] != 0u) atomicAdd(gh + i, s_hist[i]);
}

// ---------------------------------------------------------------------------
// 2. collect the keys of the threshold bin
// ---------------------------------------------------------------------------
constexpr int kRun = 8;                         // candidates per thread and pass
constexpr int kGatherStep = kRun * kSelThreads;  // candidates per pass

__global__ __launch_bounds__(kSelThreads) void select_gather_kernel(SelectArgs a) {
  __shared__ int s_wave[kSelWaves];
  __shared__ int s_res[2];
  __shared__ int s_base;
  __shared__ float s_inv2h;
  const HeadCtx h = head_ctx(a);
  // chunks past the candidates exist only when the grid was planned for a
  // longer context than the row's device length
  if (h.keep_all || (h.c > 0 && h.c * a.chunk >= h.n)) return;
  const int tid = threadIdx.x;
  const int i0 = h.c * a.chunk, i1 = min(h.n, i0 + a.chunk);
  // the histogram is requested first, then the first pass's evidence, so
  // the threshold bin is found while the evidence is still on its way; each
  // thread owns a contiguous run of kRun candidates per pass, so its keys in
  // d1 are written without per-key atomics
  uint32_t hv[8];
  load_top_bins(a.hist + h.bg * kSelBins, hv);
  const float* frow = a.mass + h.bg * a.t_cap + a.n_sink;
  float fv[kRun];
#pragma unroll
  for (int u = 0; u < kRun; ++u) {
    const int i = i0 + tid * kRun + u;
    fv[u] = i < i1 ? frow[i] : 0.f;
  }
  if (tid == 0) s_inv2h = static_cast<float>(1.0 / (2.0 * harmonic_number(h.n)));
  find_top_digit(hv, a.top_k, s_wave, s_res);
  const uint32_t d1 = static_cast<uint32_t>(s_res[0]);
  if (h.c == 0 && tid == 0) {
    a.head_info[2 * h.bg] = s_res[0];
    a.head_info[2 * h.bg + 1] = s_res[1];
  }
  const ScoreParams sp = score_params(a, h, s_inv2h);
  uint64_t* glist = a.list + h.bg * kSelListCap;
  int32_t* gabove = a.above_pos + h.bg * a.t_cap + i0;
  int gt_all = 0;
  for (int t0 = i0; t0 < i1; t0 += kGatherStep) {
    if (t0 != i0) {
#pragma unroll
      for (int u = 0; u < kRun; ++u) {
        const int i = t0 + tid * kRun + u;
        fv[u] = i < i1 ? frow[i] : 0.f;
      }
    }
    uint64_t key[kRun];
    int gt = 0, eq = 0;
#pragma unroll
    for (int u = 0; u < kRun; ++u) {
      const int i = t0 + tid * kRun + u;
      key[u] = key_of(sp, i, fv[u]);
      const uint32_t dig = top_digit(key[u]);
      const bool in = i < i1;
      gt += in && dig > d1;
      eq += in && dig == d1;
    }
    // one scan of both counts: (gt << 16) | eq, totals below 2^16 per pass
    int tot;
    const int pre = block_excl_scan((gt << 16) | eq, s_wave, &tot);
    // this thread's keys above the bin, in candidate order after those of
    // the threads and passes before it
    if (gt > 0) {
      int slot = gt_all + (pre >> 16);
#pragma unroll
      for (int u = 0; u < kRun; ++u) {
        const int i = t0 + tid * kRun + u;
        if (i < i1 && top_digit(key[u]) > d1) gabove[slot++] = i;
      }
    }
    gt_all += tot >> 16;
    const int eq_tot = tot & 0xffff;
    if (eq_tot > 0) {
      if (tid == 0) s_base = atomicAdd(a.list_n + h.bg, eq_tot);
      __syncthreads();
      if (eq > 0) {
        int slot = s_base + (pre & 0xffff);
#pragma unroll
        for (int u = 0; u < kRun; ++u) {
          const int i = t0 + tid * kRun + u;
          if (i < i1 && top_digit(key[u]) == d1) {
            if (slot < kSelListCap) glist[slot] = key[u];
            ++slot;
          }
        }
      }
      __syncthreads();
    }
  }
  if (tid == 0) a.chunk_above[h.bg * kSelMaxChunks + h.c] = gt_all;
}

// ---------------------------------------------------------------------------
// 3. resolve K* and emit in order
// ---------------------------------------------------------------------------
// Copies rows pos[r] of the cache into slots base + r of the packed buffers
// for r < count; workgroup-wide cooperative 16-byte copies.
__device__ __forceinline__ void copy_rows(const SelectArgs& a, int64_t bg, const int* s_pos, int base, int count) {
  const int np = a.row_bytes >> 4;  // 16-byte pieces per row (8, 16 or 32)
  const int lg = __builtin_ctz(np);
  const int items = count * np;
  const char* K = static_cast<const char*>(a.k) + bg * a.t_cap * a.row_bytes;
  const char* V = static_cast<const char*>(a.v) + bg * a.t_cap * a.row_bytes;
  char* PK = static_cast<char*>(a.packed_k) + (bg * a.top_k + base) * a.row_bytes;
  char* PV = static_cast<char*>(a.packed_v) + (bg * a.top_k + base) * a.row_bytes;
  constexpr int kU = 4;
  for (int i0 = threadIdx.x; i0 < items; i0 += kU * kSelThreads) {
    uint4 kv[kU], vv[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int it = i0 + u * kSelThreads;
      if (it < items) {
        const int r = it >> lg, pc = it & (np - 1);
        const int64_t off = static_cast<int64_t>(s_pos[r]) * a.row_bytes + 16 * pc;
        kv[u] = ld16_stream(K + off);
        vv[u] = ld16_stream(V + off);
      }
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int it = i0 + u * kSelThreads;
      if (it < items) {
        const int r = it >> lg, pc = it & (np - 1);
        const int64_t off = static_cast<int64_t>(r) * a.row_bytes + 16 * pc;
        *reinterpret_cast<uint4*>(PK + off) = kv[u];
        *reinterpret_cast<uint4*>(PV + off) = vv[u];
      }
    }
  }
}

// Writes the kept positions of the workgroup's chunk in ascending order at the
// chunk's output offset.  With PACK it also copies their K and V rows into the
// packed buffers at the same slots, so the fast step reads them contiguously.
//
// Usual case (the threshold bin's list fits in LDS and a chunk is at most
// kStep candidates): the chunk's kept keys are its keys above the bin, listed
// by select_gather, and its list keys at or above K*, so the evidence is not
// read again.  The rows above the bin are certain to be kept: their loads are
// issued before K* is resolved and land in registers while it is, and go to
// their slots once the ranks are known.  A bitmap of the chunk's kept
// candidates gives every kept row its rank.  Otherwise the chunk's keys are
// recomputed from the evidence and compared with K*.
template <bool PACK>
__global__ __launch_bounds__(kSelThreads) void select_emit_kernel(SelectArgs a) {
  constexpr int kStep = kGatherStep;  // candidates per emission pass (kRun per thread)
  constexpr int kWords = kStep / 32;
  constexpr int kPreU = 8;            // prefetched 16-byte pieces of K (and of V) per thread
  __shared__ __attribute__((aligned(16))) uint64_t s_list[kSelListCap];
  __shared__ __attribute__((aligned(16))) uint32_t s_hist[kSelBins];
  __shared__ int s_pos[kStep];
  __shared__ int s_late[PACK ? kStep : 1];
  __shared__ uint32_t s_bits[kWords];
  __shared__ int s_wpre[kWords];
  __shared__ int s_wave[kSelWaves];
  __shared__ uint64_t s_wave2[kSelWaves];
  __shared__ uint64_t s_small[64];
  __shared__ int s_res[4];
  __shared__ int s_nlate;
  __shared__ uint64_t s_kstar;
  const HeadCtx h = head_ctx(a);
  const int tid = threadIdx.x;
  const int K = a.top_k;
  int32_t* out = a.sel_idx + h.bg * K;
  if (h.keep_all) {
    const int i0 = h.c * a.chunk, i1 = min(K, i0 + a.chunk);
    for (int i = i0 + tid; i < i1; i += kSelThreads) out[i] = i < h.n ? a.n_sink + i : -1;
    if (h.c == 0 && tid == 0) a.sel_cnt[h.bg] = min(h.n, K);
    if (PACK) {
      const int i_end = min(i1, h.n);
      for (int r0 = i0; r0 < i_end; r0 += kStep) {
        const int cnt = min(kStep, i_end - r0);
        __syncthreads();
        for (int r = tid; r < cnt; r += kSelThreads) s_pos[r] = a.n_sink + r0 + r;
        __syncthreads();
        copy_rows(a, h.bg, s_pos, r0, cnt);
      }
    }
    return;
  }
  const int i0 = h.c * a.chunk, i1 = min(h.n, i0 + a.chunk);
  if (h.c > 0 && i0 >= h.n) return;  // past the candidates (grid planned for a longer context)
  const int lo = a.n_sink + i0;      // first position of this chunk
  // first round trip: the head's bookkeeping, the head of the threshold bin's
  // list, this chunk's count and first entries of keys above the bin
  const int d1 = a.head_info[2 * h.bg];
  const int above = a.head_info[2 * h.bg + 1];
  const int cnt_d1 = a.list_n[h.bg];
  const int n_ab = a.chunk_above[h.bg * kSelMaxChunks + h.c];
  const uint64_t* glist = a.list + h.bg * kSelListCap;
  const int32_t* gabove = a.above_pos + h.bg * a.t_cap + i0;
  // The first kPre entries of the threshold bin's list and of this chunk's
  // keys above the bin are loaded before their counts are known; more are
  // rare (a 128K row: 120-230 keys in the bin, 40-250 above it per chunk).
  constexpr int kPre = 256;
  const uint64_t first = tid < kPre ? glist[tid] : 0ull;  // inside the list; used if tid < cnt_d1
  const int ab_first = tid < kPre && i0 + tid < i1 ? gabove[tid] : 0;
  // keys above the threshold bin in the chunks before this one (this
  // thread's share)
  int above_before = 0;
  for (int c = tid; c < h.c; c += kSelThreads) above_before += a.chunk_above[h.bg * kSelMaxChunks + c];
  const int need = K - above;  // rank of K* inside bin d1 (1-based)
  const uint64_t pfx = static_cast<uint64_t>(d1) << (64 - kSelDigitBits);
  const uint64_t pmask = static_cast<uint64_t>(kSelBins - 1) << (64 - kSelDigitBits);
  if (h.c == 0 && tid == 0) a.sel_cnt[h.bg] = K;

  if (a.chunk <= kStep && cnt_d1 <= kSelListCap && (!PACK || a.rows32)) {
    const int len = i1 - i0, nw = (len + 31) >> 5;
    if (tid < kPre) s_list[tid] = first;
    for (int i = kPre + tid; i < cnt_d1; i += kSelThreads) s_list[i] = glist[i];
    if (tid < kPre && tid < n_ab) s_pos[tid] = ab_first;
    for (int r = kPre + tid; r < n_ab; r += kSelThreads) s_pos[r] = gabove[r];
    if (tid < kWords) s_bits[tid] = 0u;
    if (tid == 0) s_nlate = 0;
    __syncthreads();
    // rows above the bin: loads issued now, stored once their slots are known.
    // Row accesses go through range-checked buffer descriptors of the head's
    // cache rows and packed slots: an item past the list gets an offset past
    // the buffer, so the loops have no branches.
    const int np = PACK ? a.row_bytes >> 4 : 1;  // 8, 16 or 32 pieces per row
    const int lg = __builtin_ctz(np);
    const uint32_t rb = static_cast<uint32_t>(a.row_bytes);
    const int n_pre = PACK ? min(n_ab, (kPreU * kSelThreads) >> lg) : 0;
    const uint32_t cache_bytes = static_cast<uint32_t>(a.t_cap) * rb;
    const __amdgpu_buffer_rsrc_t rk =
        buf_rsrc_u(static_cast<const char*>(a.k) + h.bg * a.t_cap * a.row_bytes, cache_bytes);
    const __amdgpu_buffer_rsrc_t rv =
        buf_rsrc_u(static_cast<const char*>(a.v) + h.bg * a.t_cap * a.row_bytes, cache_bytes);
    uint4 pk[PACK ? kPreU : 1], pv[PACK ? kPreU : 1];
    if (PACK) {
#pragma unroll
      for (int u = 0; u < kPreU; ++u) {
        const int it = tid + kSelThreads * u;
        const int r = it >> lg, pc = it & (np - 1);
        const uint32_t off =
            r < n_pre ? static_cast<uint32_t>(a.n_sink + s_pos[min(r, kStep - 1)]) * rb + 16 * pc : kOutOfRange;
        pk[u] = buf_ld16_stream(rk, off);
        pv[u] = buf_ld16_stream(rv, off);
      }
    }
    const uint64_t kstar =
        list_resolve(s_list, cnt_d1, need, pfx, pmask, 64 - kSelDigitBits, s_hist, s_small, s_res, &s_kstar);
    // mark the chunk's kept candidates; count the kept list keys before it
    int before = above_before;
    for (int i = tid; i < cnt_d1; i += kSelThreads) {
      const uint64_t key = s_list[i];
      if (key < kstar) continue;
      const int p = key_position(key) - lo;
      if (p < 0) {
        ++before;
      } else if (p < len) {
        atomicOr(&s_bits[p >> 5], 1u << (p & 31));
        if (PACK) s_late[atomicAdd(&s_nlate, 1)] = p;
      }
    }
    for (int r = tid; r < n_ab; r += kSelThreads) {
      const int p = s_pos[r] - i0;
      atomicOr(&s_bits[p >> 5], 1u << (p & 31));
      if (PACK && r >= n_pre) s_late[atomicAdd(&s_nlate, 1)] = p;
    }
    __syncthreads();  // the marking is complete
    const uint32_t wbits = tid < nw ? s_bits[tid] : 0u;
    uint64_t tot2;
    const uint64_t pre2 = block_excl_scan2(static_cast<uint32_t>(before), __popc(wbits), s_wave2, &tot2);
    const int base = static_cast<int>(tot2 >> 32);              // kept keys before the chunk
    const int wpre = static_cast<int>(pre2 & 0xffffffffull);   // kept candidates before word tid
    if (tid < nw) s_wpre[tid] = wpre;
    __syncthreads();
    if (tid < nw) {
      int k = base + wpre;
      for (uint32_t bits = wbits; bits != 0u; bits &= bits - 1u, ++k)
        if (k < K) out[k] = lo + 32 * tid + (__ffs(bits) - 1);
    }
    if (PACK) {
      // slot of kept candidate p of the chunk (p is clamped into the chunk, so
      // the lookups of items past a list stay inside the bitmap)
      auto slot_of = [&](int p) {
        p = min(max(p, 0), len - 1);
        return base + s_wpre[p >> 5] + __popc(s_bits[p >> 5] & ((1u << (p & 31)) - 1u));
      };
      const uint32_t packed_bytes = static_cast<uint32_t>(K) * rb;
      const __amdgpu_buffer_rsrc_t rpk =
          buf_rsrc_u(static_cast<char*>(a.packed_k) + h.bg * K * a.row_bytes, packed_bytes);
      const __amdgpu_buffer_rsrc_t rpv =
          buf_rsrc_u(static_cast<char*>(a.packed_v) + h.bg * K * a.row_bytes, packed_bytes);
      // slot -> byte offset in the packed buffers (out of range past K)
      auto slot_off = [&](int slot, int pc) -> uint32_t {
        return slot < K ? static_cast<uint32_t>(slot) * rb + 16 * pc : kOutOfRange;
      };
#pragma unroll
      for (int u = 0; u < kPreU; ++u) {
        const int it = tid + kSelThreads * u;
        const int r = it >> lg, pc = it & (np - 1);
        const uint32_t off = r < n_pre ? slot_off(slot_of(s_pos[min(r, kStep - 1)] - i0), pc) : kOutOfRange;
        buf_st16_stream(rpk, off, pk[u]);
        buf_st16_stream(rpv, off, pv[u]);
      }
      // the kept rows of the threshold bin and the rows above it past the
      // prefetch: copied now
      const int items = s_nlate * np;
      constexpr int kU = 4;
      for (int j0 = 0; j0 < items; j0 += kU * kSelThreads) {
        uint4 kv[kU], vv[kU];
        uint32_t dst[kU];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int it = j0 + tid + u * kSelThreads;
          const int r = min(it >> lg, kStep - 1), pc = it & (np - 1);
          const int p = s_late[r];
          const bool in = it < items;
          dst[u] = in ? slot_off(slot_of(p), pc) : kOutOfRange;
          const uint32_t src = in ? static_cast<uint32_t>(lo + p) * rb + 16 * pc : kOutOfRange;
          kv[u] = buf_ld16_stream(rk, src);
          vv[u] = buf_ld16_stream(rv, src);
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          buf_st16_stream(rpk, dst[u], kv[u]);
          buf_st16_stream(rpv, dst[u], vv[u]);
        }
      }
    }
    return;
  }

  // general case: keys recomputed from the evidence
  const float* frow = a.mass + h.bg * a.t_cap + a.n_sink;
  float fv[kRun];
#pragma unroll
  for (int u = 0; u < kRun; ++u) {
    const int i = i0 + tid * kRun + u;
    fv[u] = i < i1 ? frow[i] : 0.f;
  }
  const float inv2h = static_cast<float>(1.0 / (2.0 * harmonic_number(h.n)));
  const ScoreParams sp = score_params(a, h, inv2h);
  uint64_t key[kRun];
#pragma unroll
  for (int u = 0; u < kRun; ++u) key[u] = key_of(sp, i0 + tid * kRun + u, fv[u]);
  if (tid < kPre) s_list[tid] = first;
  uint64_t kstar;
  int before;  // kept keys of the chunks before this one (this thread's share)
  if (cnt_d1 <= kSelListCap) {
    before = above_before;  // plus the threshold-bin keys at or above K* before the chunk
    for (int i = kPre + tid; i < cnt_d1; i += kSelThreads) s_list[i] = glist[i];
    __syncthreads();
    kstar = cnt_d1 <= kSelThreads
                ? rank_select(s_list, cnt_d1, need, reinterpret_cast<int*>(s_hist), &s_kstar)
                : radix_resolve([&](int i) { return s_list[i]; }, cnt_d1, cnt_d1, pfx, pmask, 64 - kSelDigitBits,
                                need, s_hist, s_wave, s_res, &s_kstar);
    for (int i = tid; i < cnt_d1; i += kSelThreads) {
      const uint64_t key = s_list[i];
      before += key >= kstar && key_position(key) < lo;
    }
  } else {
    // the threshold bin does not fit in LDS: radix passes over all candidates
    __syncthreads();
    kstar = radix_resolve([&](int i) { return cand_key(sp, i); }, h.n, cnt_d1, pfx, pmask, 64 - kSelDigitBits,
                          need, s_hist, s_wave, s_res, &s_kstar);
    // every kept key before the chunk, those above the threshold bin included
    before = 0;
    for (int i = tid; i < i0; i += kSelThreads) before += cand_key(sp, i) >= kstar;
  }
  int base;
  (void)block_excl_scan(before, s_wave, &base);
  for (int t0 = i0; t0 < i1; t0 += kStep) {
    if (t0 != i0) {
#pragma unroll
      for (int u = 0; u < kRun; ++u) {
        const int i = t0 + tid * kRun + u;
        key[u] = key_of(sp, i, i < i1 ? frow[i] : 0.f);
      }
    }
    int flags = 0, c = 0;
#pragma unroll
    for (int u = 0; u < kRun; ++u) {
      const int i = t0 + tid * kRun + u;
      if (i < i1 && key[u] >= kstar) {
        flags |= 1 << u;
        ++c;
      }
    }
    int total;
    const int mine = block_excl_scan(c, s_wave, &total);  // ends with a barrier
    int pos = base + mine;
#pragma unroll
    for (int u = 0; u < kRun; ++u) {
      if ((flags & (1 << u)) && pos < K) {
        const int j = a.n_sink + t0 + tid * kRun + u;
        out[pos] = j;
        if (PACK) s_pos[pos - base] = j;
        ++pos;
      }
    }
    if (PACK) {
      __syncthreads();
      copy_rows(a, h.bg, s_pos, base, max(0, min(total, K - base)));
      __syncthreads();
    }
    base += total;
  }
}

// ---------------------------------------------------------------------------
// optional Selector steps: the candidates' final scores
// ---------------------------------------------------------------------------
// One workgroup scores candidate positions [c0, c0 + chunk) of one row for all
// of its KV heads, in the order of the gist.science technical summary, 2.B:
//  1. prior r: the positional weight 1/a + 1/(n + 1 - a), times the key-norm
//     factor exp(-beta * max(0, z - c)) when that correction is on, over its
//     normaliser (2 H_n, or the sum of the combine's per-block partials), in
//     double precision;
//  2. mixture s = (1 - lambda) f + lambda r in float, as the plain Selector
//     forms it;
//  3. Soft-NMS: the nearest neighbour within the radius that ranks above the
//     candidate (higher s, or equal s at a lower position) decays it by
//     1 - decay * (1 - d / (radius + 1));
//  4. exclusivity: times its share of the row's heads' total, to the power
//     excl.
// Steps 1-2 also cover `radius` positions on either side, so that step 3
// sees every neighbour.  The final scores go to a.score, where the radix
// top-k reads them.
__global__ __launch_bounds__(kScoreThreads) void select_score_kernel(ScoreArgs a) {
#pragma clang fp contract(off)
  __shared__ float s_lds[kScoreLds];
  __shared__ double s_inv[kMaxKvHeads];
  __shared__ double s_mu[kMaxKvHeads], s_sd[kMaxKvHeads];
  const int tid = threadIdx.x;
  const int e = find_entry(a.tab, blockIdx.x);
  const int cidx = blockIdx.x - a.tab.wg_begin[e];
  const int b = a.tab.ent[e].seq;
  const int T = row_ctx(a.tab, e);
  const int Hkv = a.n_kv_heads;
  const int n = max(0, T - a.n_sink - a.n_recent);
  const int c0 = cidx * a.chunk;
  if (c0 >= n) return;  // past the candidates (grid planned for a longer context)
  const int R = a.nms_radius;
  const int W = a.chunk + 2 * R;  // window scored in steps 1-2
  const int64_t row0 = static_cast<int64_t>(b) * Hkv;
  const bool knorm = a.knorm != nullptr;
  // per head: 1 / normaliser of the prior, and the norms' mean and deviation
  if (tid < Hkv) {
    const int64_t bg = row0 + tid;
    if (knorm) {
      const int nblk = (a.tab.ent[e].ctx + kMassChunk - 1) / kMassChunk;
      double z = 0.0;
      for (int k = 0; k < nblk; ++k) z += a.zpart[bg * a.zpart_stride + k];
      s_inv[tid] = z > 0.0 ? 1.0 / z : 0.0;
      s_mu[tid] = a.knorm_stat[2 * bg];
      s_sd[tid] = a.knorm_stat[2 * bg + 1];
    } else {
      s_inv[tid] = 1.0 / (2.0 * harmonic_number(n));
    }
  }
  __syncthreads();
  const float lam = a.lambda, oml = 1.0f - a.lambda;
  const double beta = a.knorm_beta, kc = a.knorm_c;
  float* s_mix = s_lds;                     // [Hkv][W]
  float* s_nms = s_lds + Hkv * W;           // [Hkv][chunk]
  float* s_tot = s_nms + Hkv * a.chunk;     // [chunk]
  for (int idx = tid; idx < Hkv * W; idx += kScoreThreads) {
    const int g = idx / W, q = idx - g * W;
    const int p = c0 - R + q;
    float v = -1.0f;
    if (p >= 0 && p < n) {
      const int64_t off = (row0 + g) * a.t_cap + a.n_sink + p;
      double w = 1.0 / (p + 1) + 1.0 / (n - p);
      if (knorm) {
        const double sd = s_sd[g];
        const double z = sd > 0.0 ? (static_cast<double>(a.knorm[off]) - s_mu[g]) / sd : 0.0;
        w *= exp(-beta * fmax(0.0, z - kc));
      }
      const float r = static_cast<float>(w * s_inv[g]);
      v = __builtin_fmaf(lam, r, oml * a.mass[off]);
    }
    s_mix[idx] = v;
  }
  __syncthreads();
  const bool nms = R > 0 && a.nms_decay > 0.f;
  const int cend = min(a.chunk, n - c0);
  for (int idx = tid; idx < Hkv * a.chunk; idx += kScoreThreads) {
    const int g = idx / a.chunk, q = idx - g * a.chunk;
    if (q >= cend) continue;
    const int p = c0 + q;
    const float* m = s_mix + g * W + q + R;  // m[0] is candidate p
    const float v = m[0];
    float fac = 1.0f;
    if (nms) {
      for (int d = 1; d <= R; ++d) {
        const bool below = p - d >= 0 && m[-d] >= v;
        const bool above = p + d < n && m[d] > v;
        if (below || above) {
          fac = 1.0f - a.nms_decay * (1.0f - static_cast<float>(d) / static_cast<float>(R + 1));
          break;
        }
      }
    }
    s_nms[idx] = v * fac;
  }
  __syncthreads();
  const bool excl = a.excl > 0.f && Hkv > 1;
  if (excl) {
    for (int q = tid; q < cend; q += kScoreThreads) {
      float t = 0.f;
      for (int g = 0; g < Hkv; ++g) t += s_nms[g * a.chunk + q];
      s_tot[q] = t;
    }
    __syncthreads();
  }
  for (int idx = tid; idx < Hkv * a.chunk; idx += kScoreThreads) {
    const int g = idx / a.chunk, q = idx - g * a.chunk;
    if (q >= cend) continue;
    float v = s_nms[idx];
    if (excl && s_tot[q] > 0.f) v = v * powf(v / s_tot[q], a.excl);
    a.score[(row0 + g) * a.t_cap + a.n_sink + c0 + q] = v;
  }
}

hipError_t launch_score(const ScoreArgs& a, int grid, hipStream_t s) {
  launch(select_score_kernel, grid, kScoreThreads, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const SelectArgs& a, int grid, hipStream_t s) {
  hipError_t e;
  if (!a.hist_ready) {
    launch(select_clear_kernel, a.tab.n * a.n_kv_heads, 256, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    launch(select_hist_kernel, grid, kSelThreads, s, a);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  launch(select_gather_kernel, grid, kSelThreads, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.packed_k != nullptr)
    launch(select_emit_kernel<true>, grid, kSelThreads, s, a);
  else
    launch(select_emit_kernel<false>, grid, kSelThreads, s, a);
  return hipGetLastError();
}

}  // namespace sfi
