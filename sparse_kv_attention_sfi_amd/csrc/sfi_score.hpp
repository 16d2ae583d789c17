// Fused Selector score and its 64-bit selection key ("Slow-Fast Inference
// ...", gist.science technical summary, 2.B "Der Training-Free Selector":
// s = (1 - lambda) f + lambda r).  Shared by every kernel that computes keys,
// so that the histogram built next to the mass and the Selector's own passes
// agree bit for bit.
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

namespace sfi {

struct ScoreParams {
  const float* f;   // mass row (or final-score row when pre), shifted so that f[i] is candidate i
  bool pre;         // f already holds the final scores (the optional Selector steps ran)
  int n;
  int lo;           // first candidate position
  float one_minus_lambda;
  float lambda;
  float inv_2h;     // 1 / (2 H_n)
};

// Fused score and key of candidate i with evidence f.  Evaluated identically
// in every pass.
__device__ __forceinline__ uint64_t key_of(const ScoreParams& p, int i, float f) {
#pragma clang fp contract(off)
  float s = f;
  if (!p.pre) {
    const float a = static_cast<float>(i + 1);
    const float b = static_cast<float>(p.n - i);
    const float r = (__builtin_amdgcn_rcpf(a) + __builtin_amdgcn_rcpf(b)) * p.inv_2h;
    s = __builtin_fmaf(p.lambda, r, p.one_minus_lambda * f);
  }
  uint32_t u = __float_as_uint(s);
  u ^= (u & 0x80000000u) ? 0xffffffffu : 0x80000000u;  // order-preserving
  const uint32_t pos = static_cast<uint32_t>(p.lo + i);
  return (static_cast<uint64_t>(u) << 32) | static_cast<uint64_t>(~pos);
}

__device__ __forceinline__ uint64_t cand_key(const ScoreParams& p, int i) { return key_of(p, i, p.f[i]); }

// Top 12 bits of a key: the first radix digit of the selection.
constexpr int kSelDigitBits = 12;
constexpr int kSelBins = 1 << kSelDigitBits;
__device__ __forceinline__ uint32_t top_digit(uint64_t key) {
  return static_cast<uint32_t>(key >> (64 - kSelDigitBits));
}

__device__ __forceinline__ int key_position(uint64_t key) {
  return static_cast<int>(~static_cast<uint32_t>(key & 0xffffffffull));
}

// Harmonic number in double: direct sum for small n, else the asymptotic
// series ln n + gamma + 1/(2n) - 1/(12 n^2) + 1/(120 n^4) (error < 1/(252 n^6)).
__device__ inline double harmonic_number(int n) {
  if (n <= 256) {
    double h = 0.0;
    for (int i = n; i >= 1; --i) h += 1.0 / i;
    return h;
  }
  const double x = static_cast<double>(n);
  const double x2 = x * x;
  return log(x) + 0.57721566490153286061 + 1.0 / (2.0 * x) - 1.0 / (12.0 * x2) + 1.0 / (120.0 * x2 * x2);
}

}  // namespace sfi
