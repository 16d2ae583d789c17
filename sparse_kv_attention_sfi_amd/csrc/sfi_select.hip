// Selector kernel of the SFI path for gfx950 ("Slow-Fast Inference ...",
// gist.science technical summary, 2.B "Der Training-Free Selector").
//
// One workgroup of 1024 threads per (sequence, KV head).  For the n
// candidate positions [n_sink, T - n_recent) it forms
//     s = (1 - lambda) * f + lambda * r,   r(a) = (1/a + 1/(n+1-a)) / (2 H_n)
// (the closed-form mixture of evidence f and prior r; a is the 1-based
// offset from the sinks) and keeps the k best.  Exact top-k is found by
// radix selection on a 64-bit key that makes every candidate distinct:
//     key = order-preserving bits of s  << 32  |  ~position
// so "larger key" means "higher score, or equal score and lower position".
// The k-th largest key K* is resolved 12 bits at a time: each level builds an
// LDS histogram of the next digit over the candidates that still match the
// resolved prefix.  As soon as those candidates fit in LDS they are copied
// there and the remaining levels run on the copy.  A final ordered pass
// writes every position with key >= K* in ascending order.
#include <math.h>

#include "sfi_device.hpp"
#include "sfi_internal.hpp"

namespace sfi {

constexpr int kSelDigitBits = 12;
constexpr int kSelBins = 1 << kSelDigitBits;
constexpr int kSelListCap = 4096;  // candidates kept in LDS once few enough
constexpr int kSelWaves = kSelectThreads / 64;

struct ScoreParams {
  const float* f;   // mass row, shifted so that f[i] is candidate i
  int n;
  int lo;           // first candidate position
  float one_minus_lambda;
  float lambda;
  float inv_2h;     // 1 / (2 H_n)
};

// Fused score and key of candidate i.  Evaluated identically in every pass.
__device__ __forceinline__ uint64_t cand_key(const ScoreParams& p, int i) {
#pragma clang fp contract(off)
  const float a = static_cast<float>(i + 1);
  const float b = static_cast<float>(p.n - i);
  const float r = (1.0f / a + 1.0f / b) * p.inv_2h;
  const float s = __builtin_fmaf(p.lambda, r, p.one_minus_lambda * p.f[i]);
  uint32_t u = __float_as_uint(s);
  u ^= (u & 0x80000000u) ? 0xffffffffu : 0x80000000u;  // order-preserving
  const uint32_t pos = static_cast<uint32_t>(p.lo + i);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(~pos);
}

// Exclusive prefix sum over the 1024 threads, in thread order.  Returns the
// exclusive prefix; *total receives the sum.  Contains two barriers.
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

// Harmonic number in double: direct sum for small n, else the asymptotic
// series ln n + gamma + 1/(2n) - 1/(12 n^2) + 1/(120 n^4) (error < 1/(252 n^6)).
__device__ double harmonic_number(int n) {
  if (n <= 256) {
    double h = 0.0;
    for (int i = n; i >= 1; --i) h += 1.0 / i;
    return h;
  }
  const double x = static_cast<double>(n);
  const double x2 = x * x;
  return log(x) + 0.57721566490153286061 + 1.0 / (2.0 * x) - 1.0 / (12.0 * x2) + 1.0 / (120.0 * x2 * x2);
}

__global__ __launch_bounds__(kSelectThreads) void select_kernel(SelectArgs a) {
  __shared__ uint32_t s_hist[kSelBins];
  __shared__ uint64_t s_list[kSelListCap];
  __shared__ int s_wave[kSelWaves];
  __shared__ int s_list_n;
  __shared__ int s_digit, s_above;
  __shared__ float s_inv2h;

  const int tid = threadIdx.x;
  const int e = blockIdx.x / a.n_kv_heads;
  const int g = blockIdx.x - e * a.n_kv_heads;
  const int b = a.tab.seq[e];
  const int T = a.tab.ctx[e];
  const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
  const int lo = a.n_sink;
  const int n = max(0, T - a.n_recent - a.n_sink);
  const int K = a.top_k;
  int32_t* out = a.sel_idx + bg * K;

  if (n <= K) {  // every candidate is kept (also covers n == 0)
    for (int i = tid; i < K; i += kSelectThreads) out[i] = i < n ? lo + i : -1;
    if (tid == 0) a.sel_cnt[bg] = n;
    return;
  }

  if (tid == 0) s_inv2h = static_cast<float>(1.0 / (2.0 * harmonic_number(n)));
  __syncthreads();
  ScoreParams sp;
  sp.f = a.mass + bg * a.t_cap + lo;
  sp.n = n;
  sp.lo = lo;
  sp.lambda = a.lambda;
  sp.one_minus_lambda = 1.0f - a.lambda;
  sp.inv_2h = s_inv2h;

  uint64_t prefix = 0, pmask = 0;
  int need = K;     // rank of K* among the candidates matching the prefix
  int shift = 64;
  bool in_lds = false;
  int list_n = 0;
  while (shift > 0) {
    const int width = shift >= kSelDigitBits ? kSelDigitBits : shift;
    shift -= width;
    const uint32_t dmask = (1u << width) - 1u;
    const int nbins = 1 << width;
    for (int i = tid; i < nbins; i += kSelectThreads) s_hist[i] = 0u;
    __syncthreads();
    if (!in_lds) {
      for (int i = tid; i < n; i += kSelectThreads) {
        const uint64_t key = cand_key(sp, i);
        if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dmask], 1u);
      }
    } else {
      for (int i = tid; i < list_n; i += kSelectThreads) {
        const uint64_t key = s_list[i];
        if ((key & pmask) == prefix) atomicAdd(&s_hist[(key >> shift) & dmask], 1u);
      }
    }
    __syncthreads();
    // digit d with (count above d) < need <= (count above d) + hist[d]
    {
      const int per = (nbins + kSelectThreads - 1) / kSelectThreads;
      const int t_hi = kSelectThreads - 1 - tid;  // scan from the top bins down
      const int b0 = t_hi * per;
      int local = 0;
      for (int u = 0; u < per; ++u)
        if (b0 + u < nbins) local += static_cast<int>(s_hist[b0 + u]);
      int tot;
      // thread 0 owns the highest bins, so the exclusive scan in thread order
      // is the count in higher bins
      const int above_me = block_excl_scan(local, s_wave, &tot);
      (void)tot;
      if (above_me < need && need <= above_me + local) {
        int run = above_me;
        for (int u = per - 1; u >= 0; --u) {
          const int bin = b0 + u;
          if (bin >= nbins) continue;
          const int c = static_cast<int>(s_hist[bin]);
          if (run + c >= need) {
            s_digit = bin;
            s_above = run;
            break;
          }
          run += c;
        }
      }
    }
    __syncthreads();
    const int digit = s_digit;
    const int cnt = static_cast<int>(s_hist[digit]);
    need -= s_above;
    prefix |= static_cast<uint64_t>(digit) << shift;
    pmask |= static_cast<uint64_t>(dmask) << shift;
    __syncthreads();  // s_digit / s_hist reused by the next level
    if (shift > 0 && !in_lds && cnt <= kSelListCap) {
      if (tid == 0) s_list_n = 0;
      __syncthreads();
      for (int i = tid; i < n; i += kSelectThreads) {
        const uint64_t key = cand_key(sp, i);
        if ((key & pmask) == prefix) {
          const int slot = atomicAdd(&s_list_n, 1);
          if (slot < kSelListCap) s_list[slot] = key;
        }
      }
      __syncthreads();
      list_n = min(s_list_n, kSelListCap);
      in_lds = true;
    }
  }
  const uint64_t kstar = prefix;

  // ordered emission: positions with key >= K*, ascending
  int base = 0;
  for (int t0 = 0; t0 < n; t0 += 4 * kSelectThreads) {
    const int i0 = t0 + 4 * tid;
    int flags = 0, c = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = i0 + u;
      if (i < n && cand_key(sp, i) >= kstar) {
        flags |= 1 << u;
        ++c;
      }
    }
    int total;
    int pos = base + block_excl_scan(c, s_wave, &total);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if ((flags & (1 << u)) && pos < K) out[pos++] = lo + i0 + u;
    base += total;
  }
  if (tid == 0) a.sel_cnt[bg] = K;
}

hipError_t launch_select(const SelectArgs& a, int grid, hipStream_t s) {
  select_kernel<<<grid, kSelectThreads, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sfi
