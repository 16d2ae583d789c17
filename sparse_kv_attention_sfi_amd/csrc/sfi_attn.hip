// Decode-attention kernels of the SFI path for gfx950 (CDNA4).
//
//  * slow_partial: split-K flash-decode over the whole KV history (the slow
//    step's dense attention: "Slow-Fast Inference ...", gist.science
//    technical summary, 2.A).  Each workgroup streams one contiguous chunk of
//    K and V rows of one KV head exactly once and keeps the online-softmax
//    state (running max, running sum, un-normalised output) of the G query
//    heads that share the KV head.  It also stores the scaled logits so the
//    combine kernel can turn them into per-position softmax mass.
//  * slow_combine: merges the split partials into the output and writes the
//    Selector's evidence, the softmax mass averaged over the query group
//    (2.B "Der Training-Free Selector").
//  * fast_packed / fast_partial / fast_mixed, fast_merge: attention
//    restricted to sinks + recent window + selected memory (2.A, items 1-3)
//    in chunks of the support, reading the selected rows from the packed
//    buffers or gathering them by index (and, for the span's first fast
//    step, packing them), then merging the chunk states of each (sequence,
//    KV head): inside the kernel when the launch fits the CUs in one pass,
//    else in fast_merge.
//
// The in-kernel merge is the only place where workgroups of one kernel hand
// data to each other.  It uses device-coherent (sc1) stores and loads and a
// relaxed ticket, with no device-scope fence: on gfx950 such a fence writes
// back and invalidates the XCD's L2, which costs more than a kernel boundary.
//
// Work layout inside a wave (64 lanes), per 16-row tile of K:
//   logits   S[h][j] = q_h . k_j come from MFMA 16x16 (bf16: 16x16x32,
//            fp32: 16x16x4) with the query heads on M (padded to 16) and the
//            16 rows on N.  Lane l loads 16 bytes of row (l % 16) at byte
//            offset 64 * kk + 16 * (l / 16); lanes 0..15 receive the G <= 4
//            logits of their row (lanes 16..31 heads 4..7 when G = 8).
//   softmax  per-head block max over the tile rows with DPP row reductions,
//            exp2 in the log2 domain, probabilities staged in LDS.
//   P.V      VALU FMAs (the slow partial, fp32 caches and one-tile fast
//            steps): lane l owns one 16-byte piece of V rows
//            (l / PPR) + RPL * i, so every V load instruction reads whole
//            rows contiguously; partial outputs are reduced across lanes once
//            at the end.  The bf16 fast step runs P.V on MFMA instead
//            (consume_pv_mfma).
#include <math.h>

#include <algorithm>
#include <cstdlib>
#include <type_traits>

#include "sfi_device.hpp"
#include "sfi_internal.hpp"
#include "sfi_score.hpp"

namespace sfi {

__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <typename E, int D, int G>
struct Attn {
  static constexpr int kEsz = Elem<E>::kBytes;
  static constexpr int kEpp = Elem<E>::kPerPiece;  // elements per 16-byte piece
  static constexpr int kRowBytes = D * kEsz;
  static constexpr int kNL = kRowBytes / 64;       // K pieces per lane per tile
  static constexpr int kPPR = kRowBytes / 16;      // pieces per row
  static constexpr int kRPL = 64 / kPPR;           // rows per V load instruction
  static constexpr int kGroups = (G + 3) / 4;      // 16-lane groups holding logits
  static_assert(G == 1 || G == 2 || G == 4 || G == 8, "group size");
  static_assert(kNL >= 1 && kRPL >= 1, "row size");

  float m_run[G];     // running max per head (wave-uniform), log2 domain
  float l_lane[4];    // per-lane partial softmax sums, head 4 * (lane / 16) + e
  float acc[G][kEpp]; // per-lane un-normalised output piece

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int h = 0; h < G; ++h) {
      m_run[h] = -INFINITY;
#pragma unroll
      for (int i = 0; i < kEpp; ++i) acc[h][i] = 0.f;
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) l_lane[e] = 0.f;
#pragma unroll
    for (int nb = 0; nb < kNB; ++nb) cacc[nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }

  // Value of per-head array x for the head this lane's item e belongs to.  For
  // G = 8 the two candidates are selected bitwise: a plain select of x[e] and
  // x[4 + e] is turned into one load at a lane-dependent offset, which puts x
  // in scratch memory.
  __device__ __forceinline__ static float for_item(const float (&x)[G], int lane, int e) {
    if constexpr (G <= 4) {
      return x[e < G ? e : 0];
    } else {
      const uint32_t hi = 0u - static_cast<uint32_t>((lane >> 4) & 1);
      return __uint_as_float((__float_as_uint(x[e]) & ~hi) | (__float_as_uint(x[4 + e]) & hi));
    }
  }

  // Logits of TILES 16-row tiles in the log2 domain (-inf for rows outside the
  // support): x[t][e] of lane l is head 4 * (l / 16) + e, row 16 t + l % 16.
  template <int TILES>
  __device__ __forceinline__ void logits(const uint4 (&qa)[kNL], const uint4 (&kb)[TILES][kNL],
                                         const bool (&kvalid)[TILES], float scale_log2,
                                         float (&x)[TILES][4]) const {
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      f32x4_t c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kk = 0; kk < kNL; ++kk) c = mfma_piece(E(), qa[kk], kb[t][kk], c);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[t][e] = kvalid[t] ? c[e] * scale_log2 : -INFINITY;
    }
  }

  // Online-softmax step over the block: new running max, p = exp2(x - max),
  // the lane sums, and the factors alpha that rescale the old state.  Returns
  // whether any alpha differs from 1.  FRESH: the state is still the empty one
  // from init() (one call per wave), so the running max becomes the block max.
  template <int TILES, bool FRESH>
  __device__ __forceinline__ bool softmax_step(const float (&x)[TILES][4], float (&p)[TILES][4],
                                               float (&alpha)[G], int lane) {
    float mx[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      float v = x[0][e];
#pragma unroll
      for (int t = 1; t < TILES; ++t) v = fmaxf(v, x[t][e]);
      mx[e] = row16_max(v);
    }
    float m_new[G];
    bool rescale = false;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float bm = lane_bcast(mx[h & 3], 16 * (h >> 2));
      m_new[h] = FRESH ? bm : fmaxf(m_run[h], bm);
      alpha[h] = (FRESH || m_new[h] == m_run[h]) ? 1.f : fast_exp2(m_run[h] - m_new[h]);
      rescale |= (alpha[h] != 1.f);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float mn = for_item(m_new, lane, e);
      const float al = for_item(alpha, lane, e);
      float s = 0.f;
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        p[t][e] = fast_exp2(x[t][e] - mn);
        s += p[t][e];
      }
      l_lane[e] = l_lane[e] * al + s;
    }
#pragma unroll
    for (int h = 0; h < G; ++h) m_run[h] = m_new[h];
    return rescale;
  }

  // Consume one block of TILES * 16 rows: logits, online softmax, P.V on VALU.
  //   kb[t][kk] : K pieces in MFMA layout (row 16 t + lane % 16)
  //   vb[i]     : V pieces in row layout (row lane / PPR + RPL * i)
  //   kvalid[t] : row 16 t + lane % 16 exists
  //   Pw        : this wave's LDS staging area, TILES * 16 * G floats
  //   logit_base: if non-null, the block's logits go to
  //               logit_base[h * head_stride + r] for rows r < valid_rows,
  //               staged through Pw so that each lane writes four consecutive
  //               rows of one head with a single 16-byte store
  template <int TILES, bool FRESH = false>
  __device__ __forceinline__ void consume(const uint4 (&qa)[kNL], const uint4 (&kb)[TILES][kNL],
                                          const uint4 (&vb)[TILES * 16 / kRPL],
                                          const bool (&kvalid)[TILES], float* Pw, float scale_log2,
                                          float* logit_base, int64_t head_stride, int valid_rows, int lane) {
    constexpr int NV = TILES * 16 / kRPL;
    float x[TILES][4];
    logits<TILES>(qa, kb, kvalid, scale_log2, x);
    const int grp = lane >> 4;
    if (logit_base != nullptr) {
      constexpr int ROWS = TILES * 16;
      wave_sync();
      if (grp < kGroups) {
#pragma unroll
        for (int t = 0; t < TILES; ++t)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int h = 4 * grp + e;
            if (h < G) Pw[h * ROWS + 16 * t + (lane & 15)] = x[t][e];
          }
      }
      wave_sync();
#pragma unroll
      for (int j = 0; j < (G * ROWS + 255) / 256; ++j) {
        const int flat = 4 * (64 * j + lane);
        if (flat < G * ROWS) {
          const int h = flat / ROWS, r = flat - h * ROWS;
          const float4 v = *reinterpret_cast<const float4*>(Pw + flat);
          float* dst = logit_base + h * head_stride + r;
          if (r + 4 <= valid_rows) {
            *reinterpret_cast<float4*>(dst) = v;
          } else {
            if (r < valid_rows) dst[0] = v.x;
            if (r + 1 < valid_rows) dst[1] = v.y;
            if (r + 2 < valid_rows) dst[2] = v.z;
          }
        }
      }
    }
    float p[TILES][4];
    float alpha[G];
    const bool rescale = softmax_step<TILES, FRESH>(x, p, alpha, lane);
    // stage P in LDS: row r, head h at Pw[r * G + h]
    wave_sync();
    if (grp < kGroups) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        float* dst = Pw + (16 * t + (lane & 15)) * G;
        if constexpr (G >= 4) {
          *reinterpret_cast<float4*>(dst + 4 * grp) = make_float4(p[t][0], p[t][1], p[t][2], p[t][3]);
        } else if constexpr (G == 2) {
          *reinterpret_cast<float2*>(dst) = make_float2(p[t][0], p[t][1]);
        } else {
          dst[0] = p[t][0];
        }
      }
    }
    wave_sync();
    if (rescale) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int i = 0; i < kEpp; ++i) acc[h][i] *= alpha[h];
    }
    // P.V
    const int rr = lane / kPPR;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const float* src = Pw + (rr + kRPL * i) * G;
      float pr[G];
      if constexpr (G >= 4) {
#pragma unroll
        for (int h4 = 0; h4 < G; h4 += 4) {
          const float4 v4 = *reinterpret_cast<const float4*>(src + h4);
          pr[h4] = v4.x; pr[h4 + 1] = v4.y; pr[h4 + 2] = v4.z; pr[h4 + 3] = v4.w;
        }
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pr[h] = src[h];
      }
      float vf[kEpp];
      widen(E(), vb[i], vf);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int d = 0; d < kEpp; ++d) acc[h][d] = fmaf(pr[h], vf[d], acc[h][d]);
    }
  }

  // ---- P.V on MFMA (bf16 only; one call per wave, blocks of 32-row groups) --
  // out[h][d] = sum_r P[h][r] V[r][d] as 16x16x32 bf16 MFMAs with heads on M,
  // rows on K and 16 columns on N.  P enters as two bf16 terms (its truncation
  // and the truncated remainder, together within 2^-15 of P); V is exact.  V's
  // rows are staged in LDS and read back with the gfx950 transposing read
  // ds_read_b64_tr_b16: within each 16-lane group, lane 4 s + e receives
  // element e of the 8-byte words read by lanes s, 4 + s, 8 + s and 12 + s, so
  // when lane 16 q + 4 j + s reads columns 16 nb + 4 s .. + 3 of row 8 q + j,
  // lane 16 q + n receives column 16 nb + n of rows 8 q .. 8 q + 3 (the MFMA's
  // B operand layout).  The 32-byte column pair c of row r is stored at pair
  // c ^ swz(r), so the 16 rows of one read fall evenly on the LDS banks.
  static constexpr int kNB = D / 16;  // 16-column blocks
  f32x4_t cacc[kNB];                 // C[4 * (lane / 16) + i][16 nb + lane % 16]

  __device__ __forceinline__ static int swz(int r) {
    if constexpr (kPPR == 16) {
      return (r & 3) + 4 * ((r >> 3) & 1);
    } else {
      return ((r >> 1) & 1) + 2 * ((r >> 3) & 1);
    }
  }

  template <int TILES>
  __device__ __forceinline__ void consume_pv_mfma(const uint4 (&qa)[kNL], const uint4 (&kb)[TILES][kNL],
                                                  const uint4 (&vb)[TILES * 16 / kRPL],
                                                  const bool (&kvalid)[TILES], float* Pw, char* Vw,
                                                  float scale_log2, int lane) {
    static_assert(Elem<E>::kBytes == 2 && TILES % 2 == 0, "bf16, whole 32-row groups");
    constexpr int ROWS = TILES * 16;
    constexpr int NV = ROWS / kRPL;
    constexpr int NKB = ROWS / 32;
    float x[TILES][4], p[TILES][4], alpha[G];
    logits<TILES>(qa, kb, kvalid, scale_log2, x);
    softmax_step<TILES, true>(x, p, alpha, lane);
    const int grp = lane >> 4, n = lane & 15;
    // stage P as [head][row] and V rows (swizzled) in this wave's LDS
    if (grp < kGroups) {
#pragma unroll
      for (int t = 0; t < TILES; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (4 * grp + e < G) Pw[(4 * grp + e) * ROWS + 16 * t + n] = p[t][e];
    }
    {
      const int vr = lane / kPPR, vp = lane % kPPR;
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int r = vr + kRPL * i;
        *reinterpret_cast<uint4*>(Vw + r * kRowBytes + 32 * ((vp >> 1) ^ swz(r)) + 16 * (vp & 1)) = vb[i];
      }
    }
    wave_sync();
    const int q = grp;  // this lane's 8-row group within each 32-row block
#pragma unroll
    for (int kb32 = 0; kb32 < NKB; ++kb32) {
      // A operand: head n, rows 32 kb32 + 8 q .. + 7, as truncation + remainder
      uint32_t ahi[4] = {0u, 0u, 0u, 0u}, alo[4] = {0u, 0u, 0u, 0u};
      if (n < G) {
        const float* src = Pw + n * ROWS + 32 * kb32 + 8 * q;
        const float4 p0 = *reinterpret_cast<const float4*>(src);
        const float4 p1 = *reinterpret_cast<const float4*>(src + 4);
        const float pv[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint32_t b0 = __float_as_uint(pv[2 * k]), b1 = __float_as_uint(pv[2 * k + 1]);
          const uint32_t r0 = __float_as_uint(pv[2 * k] - __uint_as_float(b0 & 0xffff0000u));
          const uint32_t r1 = __float_as_uint(pv[2 * k + 1] - __uint_as_float(b1 & 0xffff0000u));
          ahi[k] = (b0 >> 16) | (b1 & 0xffff0000u);
          alo[k] = (r0 >> 16) | (r1 & 0xffff0000u);
        }
      }
      bf16x8_t a_hi, a_lo;
      __builtin_memcpy(&a_hi, ahi, 16);
      __builtin_memcpy(&a_lo, alo, 16);
      // B operand per column block: column 16 nb + n of rows 32 kb32 + 8 q .. + 7,
      // as two transposing reads of four rows each
      const int jr = (lane >> 2) & 3, sc = lane & 3;
      const int r0 = 32 * kb32 + 8 * q + jr, r1 = r0 + 4;
      const char* row0 = Vw + r0 * kRowBytes + 8 * sc;
      const char* row1 = Vw + r1 * kRowBytes + 8 * sc;
      const int sw0 = swz(r0), sw1 = swz(r1);
#pragma unroll
      for (int nb = 0; nb < kNB; ++nb) {
        const v4i16_t lo4 = lds_read_tr16(row0 + 32 * (nb ^ sw0));
        const v4i16_t hi4 = lds_read_tr16(row1 + 32 * (nb ^ sw1));
        bf16x8_t b;
        __builtin_memcpy(&b, &lo4, 8);
        __builtin_memcpy(reinterpret_cast<char*>(&b) + 8, &hi4, 8);
        cacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_hi, b, cacc[nb], 0, 0, 0);
        cacc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a_lo, b, cacc[nb], 0, 0, 0);
      }
    }
  }

  // The MFMA path's wave state to LDS: sm[w * G + h], sl[w * G + h] and this
  // wave's output slot so_w[h * D + d].
  __device__ __forceinline__ void finish_wave_mfma(float* sm, float* sl, float* so_w, int w, int lane) {
    float lt[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = row16_sum(l_lane[h & 3]);
      lt[h] = lane_bcast(v, 16 * (h >> 2));
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sm[w * G + h] = m_run[h];
        sl[w * G + h] = lt[h];
      }
    }
    const int q = lane >> 4, n = lane & 15;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * q + i;
      if (h < G) {
#pragma unroll
        for (int nb = 0; nb < kNB; ++nb) so_w[h * D + 16 * nb + n] = cacc[nb][i];
      }
    }
  }

  // Reduce this wave's state and store it in LDS slot `w`:
  //   sm[w * G + h], sl[w * G + h], so[(w * G + h) * D + d].
  __device__ __forceinline__ void finish_wave(float* sm, float* sl, float* so, int w, int lane) {
    float lt[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = row16_sum(l_lane[h & 3]);
      lt[h] = lane_bcast(v, 16 * (h >> 2));
    }
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int d = 0; d < kEpp; ++d) {
        float v = acc[h][d];
#pragma unroll
        for (int m = kPPR; m < 64; m <<= 1) v += __shfl_xor(v, m, 64);
        acc[h][d] = v;
      }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sm[w * G + h] = m_run[h];
        sl[w * G + h] = lt[h];
      }
    }
    if (lane < kPPR) {
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int d = 0; d < kEpp; ++d) so[(w * G + h) * D + lane * kEpp + d] = acc[h][d];
    }
  }

  // Row groups: lanes that own the same 16-byte piece of different rows.
  static constexpr int kRowGroups = 64 / kPPR;

  // Like finish_wave, but without the cross-lane reduction of the output:
  // every lane stores its piece to so[((w * kRowGroups + rg) * G + h) * D + col]
  // and the workgroup merge sums the row groups (for short per-wave work the
  // shuffles would dominate).
  __device__ __forceinline__ void finish_wave_lds(float* sm, float* sl, float* so, int w, int lane) {
    float lt[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float v = row16_sum(l_lane[h & 3]);
      lt[h] = lane_bcast(v, 16 * (h >> 2));
    }
    if (lane == 0) {
#pragma unroll
      for (int h = 0; h < G; ++h) {
        sm[w * G + h] = m_run[h];
        sl[w * G + h] = lt[h];
      }
    }
    const int rg = lane / kPPR, pc = lane % kPPR;
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = so + ((w * kRowGroups + rg) * G + h) * D + pc * kEpp;
#pragma unroll
      for (int d = 0; d < kEpp; d += 4)
        *reinterpret_cast<float4*>(dst + d) = make_float4(acc[h][d], acc[h][d + 1], acc[h][d + 2], acc[h][d + 3]);
    }
  }
};

// Merge NW wave states from LDS into one (max, sum, output) per head and store
// it to the global partial slot: ml[h * ml_stride] = (m, l),
// o[h * o_stride + d].  Called by all threads of the workgroup after a barrier.
template <int D, int G, int NW>
__device__ __forceinline__ void merge_waves_to_global(const float* sm, const float* sl, const float* so,
                                                      float* ml, int64_t ml_stride, float* o,
                                                      int64_t o_stride, int tid, int nthreads) {
  for (int idx = tid; idx < G * D; idx += nthreads) {
    const int h = idx / D, d = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * G + h]);
    float acc = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm[w * G + h];
        if (mw != -INFINITY) acc += so[(w * G + h) * D + d] * fast_exp2(mw - M);
      }
    }
    o[h * o_stride + d] = acc;
    if (d == 0) {
      float L = 0.f;
      if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < NW; ++w) {
          const float mw = sm[w * G + h];
          if (mw != -INFINITY) L += sl[w * G + h] * fast_exp2(mw - M);
        }
      }
      ml[h * ml_stride] = M;
      ml[h * ml_stride + 1] = L;
    }
  }
}

// Merge of the NW wave states of a workgroup, each of RG row groups, wave w's
// at so[w * wave_stride + (rg * G + h) * D + d] (finish_wave_lds: wave_stride =
// RG * G * D; finish_wave_mfma: RG = 1).  Each thread owns four consecutive
// columns of one head: it scales the NW wave states once and reads 16-byte
// vectors, then hands emit(h, d, acc, M, L) the merged un-normalised output
// quad at column d, the head's running max and its sum.
template <int D, int G, int NW, int RG, typename Emit>
__device__ __forceinline__ void merge_wave_groups(const float* sm, const float* sl, const float* so,
                                                  int wave_stride, int tid, int nthreads, Emit emit) {
  constexpr int Q = D / 4;  // column quads per head
  for (int idx = tid; idx < G * Q; idx += nthreads) {
    const int h = idx / Q, d = 4 * (idx - h * Q);
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm[w * G + h]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    float L = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float mw = sm[w * G + h];
        if (mw == -INFINITY) continue;
        const float sc = fast_exp2(mw - M);
        float4 part = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
        for (int rg = 0; rg < RG; ++rg) {
          const float4 v = *reinterpret_cast<const float4*>(so + w * wave_stride + (rg * G + h) * D + d);
          part.x += v.x; part.y += v.y; part.z += v.z; part.w += v.w;
        }
        acc.x += part.x * sc; acc.y += part.y * sc; acc.z += part.z * sc; acc.w += part.w * sc;
        L += sl[w * G + h] * sc;
      }
    }
    emit(h, d, acc, M, L);
  }
}

// Load the query pieces of KV head g's query group in MFMA operand-A layout.
template <typename E, int D, int G>
__device__ __forceinline__ void load_q(const void* q, int64_t q_row0, int lane,
                                       uint4 (&qa)[Attn<E, D, G>::kNL]) {
  using A = Attn<E, D, G>;
  const int h = lane & 15;
  const char* base = static_cast<const char*>(q) + (q_row0 + (h < G ? h : 0)) * A::kRowBytes;
#pragma unroll
  for (int kk = 0; kk < A::kNL; ++kk) {
    if (h < G) {
      qa[kk] = ld16(base + 64 * kk + 16 * (lane >> 4));
    } else {
      qa[kk] = make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// ---------------------------------------------------------------------------
// slow step, kernel 1: split-K partials
// ---------------------------------------------------------------------------
// NORMS: also the Euclidean norm of every key row streamed (the key-norm
// prior's input) and, per split, the sums of the candidates' norms and
// squared norms in double precision.  A row's 16-byte pieces sit in lanes
// l, l + 16, l + 32 and l + 48 of the MFMA layout; each lane sums its pieces'
// squares (pairwise in float, then in double) and two lane exchanges complete
// the row.
template <typename E, int D, int G, bool NORMS>
__global__ __launch_bounds__(kSlowThreads) void slow_partial_kernel(SlowArgs a) {
  using A = Attn<E, D, G>;
  constexpr int RB = A::kRowBytes;
  constexpr int ROWS = block_rows(RB);
  constexpr int TILES = ROWS / 16;
  constexpr int NV = ROWS / A::kRPL;
  constexpr int NW = kSlowThreads / 64;

  __shared__ __attribute__((aligned(16))) float s_p[NW * ROWS * G];
  __shared__ __attribute__((aligned(16))) float s_o[NW * G * D];
  __shared__ float s_m[NW * G], s_l[NW * G];
  // the split's logits, [head][row], written out in one pass at the end
  __shared__ __attribute__((aligned(16))) float s_lg[G * kLogitBufRows];
  __shared__ double s_nrm[NORMS ? 2 * NW : 1];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wg = blockIdx.x;
  const int e = find_entry(a.tab, wg);
  const int local = wg - a.tab.wg_begin[e];
  const int nsplit = a.tab.ent[e].nsplit;
  const int g = local / nsplit;
  const int split = local - g * nsplit;
  const int b = a.tab.ent[e].seq;
  const int T = row_ctx(a.tab, e);
  const int r_begin = split * a.split_rows;
  const int r_end = min(T, r_begin + a.split_rows);
  if (a.clear_hist != nullptr && split == 0) {
    // fresh Selector bookkeeping for the histogram the combine builds next
    const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
    uint4* h4 = reinterpret_cast<uint4*>(a.clear_hist + bg * kSelBins);
    for (int i = threadIdx.x; i < kSelBins / 4; i += kSlowThreads) h4[i] = make_uint4(0u, 0u, 0u, 0u);
    if (threadIdx.x == 0) a.clear_list_n[bg] = 0;
  }

  const int64_t kv_row0 = (static_cast<int64_t>(b) * a.n_kv_heads + g) * a.t_cap;
  const char* Kb = static_cast<const char*>(a.k) + kv_row0 * RB;
  const char* Vb = static_cast<const char*>(a.v) + kv_row0 * RB;
  const int64_t qh0 = static_cast<int64_t>(b) * a.n_q_heads + g * G;

  uint4 qa[A::kNL];
  load_q<E, D, G>(a.q, qh0, lane, qa);

  A st;
  st.init();
  float* Pw = s_p + wave * ROWS * G;
  const int kr = lane & 15, kg = lane >> 4;
  const int vr = lane / A::kPPR, vp = lane % A::kPPR;
  // Logits of a split that fits kLogitBufRows collect in LDS and leave in one
  // contiguous pass per head after the loop, written through to memory:
  // stored block by block, or left dirty in L2, they interleave with the K/V
  // read stream and cost HBM time far above their share of bytes.
  const bool buffered = a.logits != nullptr && a.split_rows <= kLogitBufRows;
  double nrm_sum = 0.0, nrm_sq = 0.0;  // NORMS: this lane's candidate rows

  for (int r0 = r_begin + wave * ROWS; r0 < r_end; r0 += NW * ROWS) {
    uint4 kb[TILES][A::kNL];
    uint4 vb[NV];
    bool kvalid[TILES];
#pragma unroll
    for (int t = 0; t < TILES; ++t) {
      const int row = r0 + 16 * t + kr;
      kvalid[t] = row < r_end;
      const char* src = Kb + static_cast<int64_t>(kvalid[t] ? row : r_end - 1) * RB + 16 * kg;
#pragma unroll
      for (int kk = 0; kk < A::kNL; ++kk) kb[t][kk] = ld16_stream(src + 64 * kk);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int row = min(r0 + vr + A::kRPL * i, r_end - 1);
      vb[i] = ld16_stream(Vb + static_cast<int64_t>(row) * RB + 16 * vp);
    }
    if constexpr (NORMS) {
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        double p2 = 0.0;
#pragma unroll
        for (int kk = 0; kk < A::kNL; ++kk) {
          float x[A::kEpp];
          widen(E(), kb[t][kk], x);
#pragma unroll
          for (int e = 0; e < A::kEpp; ++e) x[e] = x[e] * x[e];
#pragma unroll
          for (int w2 = A::kEpp / 2; w2 >= 1; w2 /= 2)
#pragma unroll
            for (int e = 0; e < w2; ++e) x[e] += x[e + w2];
          p2 += static_cast<double>(x[0]);
        }
        p2 += __shfl_xor(p2, 16, 64);
        p2 += __shfl_xor(p2, 32, 64);
        const int row = r0 + 16 * t + kr;
        if (kg == 0 && row < r_end) {
          const double nu = sqrt(p2);
          a.knorm[(static_cast<int64_t>(b) * a.n_kv_heads + g) * a.t_cap + row] = static_cast<float>(nu);
          if (row >= a.n_sink && row < T - a.n_recent) {
            nrm_sum += nu;
            nrm_sq += p2;
          }
        }
      }
    }
    float* lbase = a.logits == nullptr ? nullptr
                   : buffered          ? s_lg + (r0 - r_begin)
                                       : a.logits + qh0 * a.logit_pitch + r0;
    st.template consume<TILES>(qa, kb, vb, kvalid, Pw, a.scale_log2, lbase,
                               buffered ? kLogitBufRows : a.logit_pitch, r_end - r0, lane);
  }
  if (buffered) {
    __syncthreads();
    const int rows = r_end - r_begin;
    // head h is uniform across the workgroup, so the buffer descriptor of its
    // logit row is too (one scalar descriptor per store instruction)
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float* dst = a.logits + (qh0 + h) * a.logit_pitch + r_begin;  // this split's logits of head h
      for (int r = 4 * threadIdx.x; r < rows; r += 4 * kSlowThreads) {
        const float4 v = *reinterpret_cast<const float4*>(s_lg + h * kLogitBufRows + r);
        if (r + 4 <= rows) {
          st16_wt(dst, 4 * rows, 4 * r, v);
        } else {
          st4_wt(dst + r, v.x);
          if (r + 1 < rows) st4_wt(dst + r + 1, v.y);
          if (r + 2 < rows) st4_wt(dst + r + 2, v.z);
        }
      }
    }
  }
  if constexpr (NORMS) {
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {
      nrm_sum += __shfl_xor(nrm_sum, m, 64);
      nrm_sq += __shfl_xor(nrm_sq, m, 64);
    }
    if (lane == 0) {
      s_nrm[2 * wave] = nrm_sum;
      s_nrm[2 * wave + 1] = nrm_sq;
    }
  }
  st.finish_wave(s_m, s_l, s_o, wave, lane);
  __syncthreads();
  if constexpr (NORMS) {
    if (threadIdx.x == 0) {
      double sn = 0.0, sq = 0.0;
#pragma unroll
      for (int w2 = 0; w2 < NW; ++w2) {
        sn += s_nrm[2 * w2];
        sq += s_nrm[2 * w2 + 1];
      }
      double* kp = a.knorm_part + ((static_cast<int64_t>(b) * a.n_kv_heads + g) * a.part_stride + split) * 2;
      kp[0] = sn;
      kp[1] = sq;
    }
  }
  const int64_t slot = qh0 * a.part_stride + split;
  merge_waves_to_global<D, G, NW>(s_m, s_l, s_o, a.part_ml + slot * 2,
                                  static_cast<int64_t>(a.part_stride) * 2, a.part_o + slot * D,
                                  static_cast<int64_t>(a.part_stride) * D, threadIdx.x, kSlowThreads);
}

// ---------------------------------------------------------------------------
// merging partial (max, sum, output) slots
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  v = fmaxf(v, __shfl_xor(v, 32, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  v = row16_sum(v);
  v += __shfl_xor(v, 16, 64);
  v += __shfl_xor(v, 32, 64);
  return v;
}

constexpr int kMaxSlots = kMaxMergeSlots;

// Global max M_h and 1 / L_h of NH heads over n slots; ml of head h is at
// ml + h * ml_hstride as (m, l) pairs.  Ends with a barrier.
// Global max M_h and 1 / L_h of NH heads from n <= kMaxSlots (max, sum)
// partial pairs (one wave per head); every pair is read once, in a single
// round trip.
template <int NH, int NW>
__device__ __forceinline__ void head_max_sum(const float* ml, int64_t ml_hstride, int n, float* sM,
                                             float* sInvL) {
  constexpr int kPer = kMaxSlots / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int h = wave; h < NH; h += NW) {
    const float* p = ml + h * ml_hstride;
    float2 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int s = lane + 64 * u;
      v[u] = s < n ? *reinterpret_cast<const float2*>(p + 2 * s) : make_float2(-INFINITY, 0.f);
    }
    float m = -INFINITY;
#pragma unroll
    for (int u = 0; u < kPer; ++u) m = fmaxf(m, v[u].x);
    m = wave_max(m);
    float l = 0.f;
    if (m != -INFINITY) {
#pragma unroll
      for (int u = 0; u < kPer; ++u)
        if (v[u].x != -INFINITY) l += v[u].y * fast_exp2(v[u].x - m);
    }
    l = wave_sum(l);
    if (lane == 0) {
      sM[h] = m;
      sInvL[h] = l > 0.f ? 1.f / l : 0.f;
    }
  }
  __syncthreads();
}

template <int NH, int NT>
struct MergeSmem {
  float m[NH * kMaxSlots];
  float l[NH * kMaxSlots];
  float M[NH];
  float invL[NH];
  float4 red[NT];
};

// out[h * D + d] = sum_s exp2(m_hs - M_h) / L_h * o_hs[d] for NH heads over
// n <= kMaxSlots partial slots.  Each thread owns one float4 column of one
// head for a strided subset of the slots.  Its first kPrefetch output loads
// are issued together with the (m, l) loads, so a merge of up to
// kPrefetch * NSUB slots costs a single round trip to memory.
template <int D, int NH, int NT>
__device__ __forceinline__ void merge_partials(const float* ml, int64_t ml_hstride, const float* po,
                                               int64_t po_hstride, int n, float* out,
                                               MergeSmem<NH, NT>& sm) {
  constexpr int C4 = D / 4;
  constexpr int NC = NH * C4;
  static_assert(NC <= NT, "one column per thread at least");
  constexpr int NSUB = NT / NC;
  constexpr int NW = NT / 64;
  constexpr int kPrefetch = 8;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = tid % NC, sub = tid / NC;
  const int h = col / C4, c4 = col - h * C4;
  const bool active = sub < NSUB;
  const float* base = po + h * po_hstride + 4 * c4;
  float4 v[kPrefetch];
#pragma unroll
  for (int u = 0; u < kPrefetch; ++u) {
    const int s = sub + u * NSUB;
    v[u] = (active && s < n) ? *reinterpret_cast<const float4*>(base + static_cast<int64_t>(s) * D)
                             : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  for (int i = tid; i < NH * n; i += NT) {
    const int hh = i / n, s = i - hh * n;
    const float2 p = *reinterpret_cast<const float2*>(ml + hh * ml_hstride + 2 * s);
    sm.m[hh * kMaxSlots + s] = p.x;
    sm.l[hh * kMaxSlots + s] = p.y;
  }
  __syncthreads();
  for (int hh = wave; hh < NH; hh += NW) {
    float m = -INFINITY;
    for (int s = lane; s < n; s += 64) m = fmaxf(m, sm.m[hh * kMaxSlots + s]);
    m = wave_max(m);
    float l = 0.f;
    if (m != -INFINITY) {
      for (int s = lane; s < n; s += 64) {
        const float ms = sm.m[hh * kMaxSlots + s];
        if (ms != -INFINITY) l += sm.l[hh * kMaxSlots + s] * fast_exp2(ms - m);
      }
    }
    l = wave_sum(l);
    if (lane == 0) {
      sm.M[hh] = m;
      sm.invL[hh] = l > 0.f ? 1.f / l : 0.f;
    }
  }
  __syncthreads();
  const float M = sm.M[h], il = sm.invL[h];
  const float* mh = sm.m + h * kMaxSlots;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  if (active) {
#pragma unroll
    for (int u = 0; u < kPrefetch; ++u) {
      const int s = sub + u * NSUB;
      if (s < n && mh[s] != -INFINITY) {
        const float w = fast_exp2(mh[s] - M) * il;
        acc.x += w * v[u].x; acc.y += w * v[u].y; acc.z += w * v[u].z; acc.w += w * v[u].w;
      }
    }
    for (int s0 = sub + kPrefetch * NSUB; s0 < n; s0 += kPrefetch * NSUB) {
      float4 x[kPrefetch];
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        const int s = s0 + u * NSUB;
        x[u] = s < n ? *reinterpret_cast<const float4*>(base + static_cast<int64_t>(s) * D)
                     : make_float4(0.f, 0.f, 0.f, 0.f);
      }
#pragma unroll
      for (int u = 0; u < kPrefetch; ++u) {
        const int s = s0 + u * NSUB;
        if (s < n && mh[s] != -INFINITY) {
          const float w = fast_exp2(mh[s] - M) * il;
          acc.x += w * x[u].x; acc.y += w * x[u].y; acc.z += w * x[u].z; acc.w += w * x[u].w;
        }
      }
    }
  }
  if constexpr (NSUB > 1) {
    sm.red[tid] = acc;
    __syncthreads();
    if (sub == 0) {
      float4 t = acc;
#pragma unroll
      for (int u = 1; u < NSUB; ++u) {
        const float4 x = sm.red[u * NC + col];
        t.x += x.x; t.y += x.y; t.z += x.z; t.w += x.w;
      }
      *reinterpret_cast<float4*>(out + h * D + 4 * c4) = t;
    }
  } else {
    if (active) *reinterpret_cast<float4*>(out + h * D + 4 * c4) = acc;
  }
}

// The key-norm prior's statistics of KV head row (b, g): mean and standard
// deviation of the candidates' key norms, from the slow partial's per-split
// sums (the same fixed-order reduction in every workgroup, so all agree bit
// for bit; mass block 0 stores them), and this mass block's share of the
// prior's normaliser: the sum over its candidates of the positional weight
// 1/a + 1/(n + 1 - a) times exp(-beta * max(0, z - c)), z the candidate's
// norm in standard deviations above the mean, in double precision.
__device__ void knorm_prior_block(const CombineArgs& a, int b, int g, int r, int T, int nsplit, int j0, int j1) {
  constexpr int NW = kCombineThreads / 64;
  __shared__ double s_stat[2];
  __shared__ double s_red[NW];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
  const int n = max(0, T - a.n_sink - a.n_recent);
  if (wave == 0) {
    const double* kp = a.knorm_part + bg * a.part_stride * 2;
    double sn = 0.0, sq = 0.0;
    for (int i = lane; i < nsplit; i += 64) {
      sn += kp[2 * i];
      sq += kp[2 * i + 1];
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
      sn += __shfl_xor(sn, m, 64);
      sq += __shfl_xor(sq, m, 64);
    }
    if (lane == 0) {
      const double mu = n > 0 ? sn / n : 0.0;
      const double sd = n > 0 ? sqrt(fmax(0.0, sq / n - mu * mu)) : 0.0;
      s_stat[0] = mu;
      s_stat[1] = sd;
      if (r == 0) {
        a.knorm_stat[2 * bg] = mu;
        a.knorm_stat[2 * bg + 1] = sd;
      }
    }
  }
  __syncthreads();
  const double mu = s_stat[0], sd = s_stat[1];
  const double beta = a.knorm_beta, c = a.knorm_c;
  const float* nrow = a.knorm + bg * a.t_cap;
  double z = 0.0;
  const int lo = max(j0, a.n_sink), hi = min(j1, T - a.n_recent);
  for (int j = lo + tid; j < hi; j += kCombineThreads) {
    const int i = j - a.n_sink;
    const double w = 1.0 / (i + 1) + 1.0 / (n - i);
    const double zz = sd > 0.0 ? (static_cast<double>(nrow[j]) - mu) / sd : 0.0;
    z += w * exp(-beta * fmax(0.0, zz - c));
  }
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) z += __shfl_xor(z, m, 64);
  if (lane == 0) s_red[wave] = z;
  __syncthreads();
  if (tid == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += s_red[w];
    a.zpart[bg * a.zpart_stride + r] = tot;
  }
}

// ---------------------------------------------------------------------------
// slow step, kernel 2: merge partials; per-position softmax mass
// ---------------------------------------------------------------------------
//
// With HIST, the mass workgroups also add every candidate's top key digit to
// the Selector's histogram (the first pass of its radix top-k), using the same
// score function as the Selector on the very value they store as the mass.
template <int D, int G, bool HIST>
__global__ __launch_bounds__(kCombineThreads) void slow_combine_kernel(CombineArgs a) {
  constexpr int NW = kCombineThreads / 64;
  constexpr int PER = kMassChunk / (4 * kCombineThreads);  // float4 groups per thread
  __shared__ float s_M[G], s_invL[G];
  __shared__ MergeSmem<1, kCombineThreads> s_merge;
  __shared__ uint32_t s_hist[HIST ? kSelBins : 1];
  __shared__ float s_inv2h;

  const int tid = threadIdx.x;
  const int wg = blockIdx.x;
  const int e = find_entry(a.tab, wg);
  const int local = wg - a.tab.wg_begin[e];
  const int mblocks = a.mass_blocks[e];
  const int per_g = mblocks + G;
  const int g = local / per_g;
  const int r = local - g * per_g;
  const int b = a.tab.ent[e].seq;
  const int T = row_ctx(a.tab, e);
  const int nsplit = a.tab.ent[e].nsplit;
  const int64_t qh0 = static_cast<int64_t>(b) * a.n_q_heads + g * G;
  const int64_t ml_hstride = static_cast<int64_t>(a.part_stride) * 2;
  const float* ml = a.part_ml + qh0 * ml_hstride;

  if (r < mblocks) {
    // f_j = (1/G) sum_h exp2(x_hj - M_h) / L_h, four positions per thread; the
    // logit loads are issued before the (m, l) loads so both share a round trip
    const int j0 = r * kMassChunk;
    const int j1 = min(T, j0 + kMassChunk);
    const float* lg = a.logits + qh0 * a.logit_pitch;
    float* mrow = a.mass + (static_cast<int64_t>(b) * a.n_kv_heads + g) * a.t_cap;
    float4 x[PER][G];
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int j = j0 + 4 * (it * kCombineThreads + tid);
#pragma unroll
      for (int h = 0; h < G; ++h)
        x[it][h] = j < j1 ? ld16_stream_f(lg + h * a.logit_pitch + j) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // candidates [n_sink, T - n_recent) take part in a top-k only when there
    // are more of them than k (otherwise the Selector keeps all of them)
    const int n_cand = max(0, T - a.n_sink - a.n_recent);
    const bool hist = HIST && n_cand > a.top_k && a.top_k > 0;
    if (hist) {
      for (int i = tid; i < kSelBins; i += kCombineThreads) s_hist[i] = 0u;
      if (tid == 0) s_inv2h = static_cast<float>(1.0 / (2.0 * harmonic_number(n_cand)));
    }
    head_max_sum<G, NW>(ml, ml_hstride, nsplit, s_M, s_invL);  // ends with a barrier
    const float invG = 1.f / static_cast<float>(G);
    ScoreParams sp;
    sp.f = nullptr;
    sp.pre = false;
    sp.n = n_cand;
    sp.lo = a.n_sink;
    sp.lambda = a.lambda;
    sp.one_minus_lambda = 1.0f - a.lambda;
    sp.inv_2h = hist ? s_inv2h : 0.f;
#pragma unroll
    for (int it = 0; it < PER; ++it) {
      const int j = j0 + 4 * (it * kCombineThreads + tid);
      if (j >= j1) continue;
      float f[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float M = s_M[h], il = s_invL[h];
        f[0] += fast_exp2(x[it][h].x - M) * il;
        f[1] += fast_exp2(x[it][h].y - M) * il;
        f[2] += fast_exp2(x[it][h].z - M) * il;
        f[3] += fast_exp2(x[it][h].w - M) * il;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (j + u >= j1) continue;
        const float m = f[u] * invG;
        mrow[j + u] = m;
        if (hist) {
          const int i = j + u - a.n_sink;
          if (i >= 0 && i < n_cand) atomicAdd(&s_hist[top_digit(key_of(sp, i, m))], 1u);
        }
      }
    }
    if (hist) {
      __syncthreads();
      uint32_t* gh = a.sel_hist + (static_cast<int64_t>(b) * a.n_kv_heads + g) * kSelBins;
      for (int i = tid; i < kSelBins; i += kCombineThreads)
        if (s_hist[i] != 0u) atomicAdd(gh + i, s_hist[i]);
    }
    if (a.knorm_part != nullptr) knorm_prior_block(a, b, g, r, T, nsplit, j0, j1);
  } else {
    const int h = r - mblocks;
    merge_partials<D, 1, kCombineThreads>(ml + h * ml_hstride, ml_hstride,
                                          a.part_o + (qh0 + h) * a.part_stride * D,
                                          static_cast<int64_t>(a.part_stride) * D, nsplit,
                                          a.out + (qh0 + h) * D, s_merge);
  }
}

// ---------------------------------------------------------------------------
// fast step: sparse attention over the support in chunks, then the merge of
// the chunk states (in the kernel or in a merge kernel)
// ---------------------------------------------------------------------------
struct SupportGeom {
  int ns_eff, w_lo, w_eff, cnt, size;
};

// Support of KV head row `bg` at context t: [0, ns_eff) sinks, then the window
// [w_lo, w_lo + w_eff), then sel_idx[0 : cnt].
__device__ __forceinline__ SupportGeom support_geom(int t, int n_sink, int n_recent, int top_k,
                                                    const int32_t* sel_cnt, int64_t bg) {
  SupportGeom s;
  s.ns_eff = min(n_sink, t);
  s.w_lo = max(n_sink, t - n_recent);
  s.w_eff = max(0, t - s.w_lo);
  const int n = max(0, t - n_sink - n_recent);
  const int kmax = min(top_k, n);
  s.cnt = min(max(sel_cnt[bg], 0), kmax);
  s.size = s.ns_eff + s.w_eff + s.cnt;
  return s;
}

// Position of support element p, or -1 when the stored index is not a
// position of the current context.
__device__ __forceinline__ int support_pos(const SupportGeom& s, int p, int t,
                                           const int32_t* sel_row) {
  if (p < s.ns_eff) return p;
  if (p < s.ns_eff + s.w_eff) return s.w_lo + (p - s.ns_eff);
  if (p < s.size) {
    const int j = sel_row[p - s.ns_eff - s.w_eff];
    return (j >= 0 && j < t) ? j : -1;
  }
  return -1;
}

// Fast-step P.V runs on MFMA for bf16 caches when every wave covers whole
// 32-row groups, else on VALU.
template <typename E, int TILES>
constexpr bool fast_pv_mfma() {
  return Elem<E>::kBytes == 2 && TILES % 2 == 0;
}

// Shared memory of the fast step's tail: the last workgroup of a head merges
// the chunk states of its kFastThreads / (G * D / 4) slot subsets through it
// (subset 0 stays in registers, so only the other subsets take entries).
template <int D, int G>
struct FastTailSmem {
  static constexpr int kEntries = kFastThreads > G * D / 4 ? kFastThreads - G * D / 4 : 1;
  float m[kEntries];
  float l[kEntries];
  float4 o[kEntries];
  int last;
};

// Shared memory of a fast-step workgroup (gather and packed paths alike): the
// probabilities of each wave's rows, the per-wave output slots (VALU P.V) or
// the V staging rows (MFMA P.V), the per-wave running max and sum, the support
// positions of the chunk (gather path), and the tail's merge buffers.  Each
// is its own LDS variable (one set per instantiation), so the compiler knows
// they do not overlap.
template <typename E, int D, int G, int TILES>
struct FastSmem {
  float* p;
  float* o;
  char* v;
  float* m;
  float* l;
  int* pos;
  FastTailSmem<D, G>* tail;
};
template <typename E, int D, int G, int TILES>
__device__ __forceinline__ FastSmem<E, D, G, TILES> fast_smem() {
  constexpr int kRows = TILES * 16, kWaves = kFastThreads / 64;
  constexpr bool kMfma = fast_pv_mfma<E, TILES>();
  __shared__ __attribute__((aligned(16))) float p[kWaves * kRows * G];
  __shared__ __attribute__((aligned(16))) float o[kMfma ? 4 : kWaves * Attn<E, D, G>::kRowGroups * G * D];
  __shared__ __attribute__((aligned(16))) char v[kMfma ? kWaves * kRows * Attn<E, D, G>::kRowBytes : 16];
  __shared__ float m[kWaves * G], l[kWaves * G];
  __shared__ int pos[kWaves * kRows];
  __shared__ FastTailSmem<D, G> tail;
  return {p, o, v, m, l, pos, &tail};
}

// Merge of the nchunk chunk states of the G query heads of one (sequence, KV
// head) into the output, renormalised over the whole support.  Thread
// (sub, h, c4) merges slots sub, sub + NSUB, ... of head h's column quad c4
// online (running max), in batches whose loads are issued together; the NSUB
// subset states are then combined through LDS.  COHERENT: the states were
// published by other workgroups of the running kernel and are read with
// device-coherent loads; otherwise a previous kernel wrote them.  Both the
// in-kernel merge and the merge kernel run this code with kFastThreads
// threads, so they give the same bits.
template <int D, int G, bool COHERENT>
__device__ __forceinline__ void fast_merge_slots(const FastArgs& a, int64_t eg, int64_t qh0, int nchunk,
                                                 FastTailSmem<D, G>& sh, int tid) {
  constexpr int C4 = D / 4;
  constexpr int NC = G * C4;  // column quads of the group: 16 ... 256
  constexpr int NSUB = kFastThreads / NC;
  static_assert(NSUB >= 1 && NSUB * NC == kFastThreads, "whole column quads per thread");
  constexpr int kBatch = 16;
  const int col = tid % NC, sub = tid / NC;
  const int h = col / C4, c4 = col - h * C4;
  // one buffer descriptor per workgroup (its G heads' rows), so every load
  // takes a scalar descriptor; lanes differ only in their offsets
  const float* mlg = a.part_ml + eg * G * a.part_stride * 2;
  const float* og = a.part_o + eg * G * a.part_stride * D;
  const int ml_bytes = G * a.part_stride * 8, o_bytes = G * a.part_stride * D * 4;
  const int ml_off = h * a.part_stride * 8, o_off = (h * a.part_stride * D + 4 * c4) * 4;
  float M = -INFINITY, L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int s0 = sub; s0 < nchunk; s0 += kBatch * NSUB) {
    float2 ml[kBatch];
    float4 o[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int sl = s0 + u * NSUB;
      if (sl < nchunk) {
        if constexpr (COHERENT) {
          ml[u] = ld8_dev(mlg, ml_bytes, ml_off + sl * 8);
          o[u] = ld16_dev(og, o_bytes, o_off + sl * D * 4);
        } else {
          ml[u] = *reinterpret_cast<const float2*>(reinterpret_cast<const char*>(mlg) + ml_off + sl * 8);
          o[u] = *reinterpret_cast<const float4*>(reinterpret_cast<const char*>(og) + o_off + sl * D * 4);
        }
      } else {
        ml[u] = make_float2(-INFINITY, 0.f);
        o[u] = make_float4(0.f, 0.f, 0.f, 0.f);
      }
    }
    float mb = M;
#pragma unroll
    for (int u = 0; u < kBatch; ++u) mb = fmaxf(mb, ml[u].x);
    if (mb == -INFINITY) continue;
    if (M != mb) {
      const float sc = M == -INFINITY ? 0.f : fast_exp2(M - mb);
      acc.x *= sc; acc.y *= sc; acc.z *= sc; acc.w *= sc;
      L *= sc;
      M = mb;
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (ml[u].x == -INFINITY) continue;
      const float w = fast_exp2(ml[u].x - M);
      acc.x += w * o[u].x; acc.y += w * o[u].y; acc.z += w * o[u].z; acc.w += w * o[u].w;
      L += w * ml[u].y;
    }
  }
  if constexpr (NSUB > 1) {
    static_assert(FastTailSmem<D, G>::kEntries == (NSUB - 1) * NC, "one entry per thread of subsets 1..");
    if (sub != 0) {
      sh.m[tid - NC] = M;
      sh.l[tid - NC] = L;
      sh.o[tid - NC] = acc;
    }
    __syncthreads();
    if (sub != 0) return;
#pragma unroll
    for (int u = 1; u < NSUB; ++u) {
      const float mu = sh.m[(u - 1) * NC + col];
      if (mu == -INFINITY) continue;
      const float mn = fmaxf(M, mu);
      const float s_old = M == -INFINITY ? 0.f : fast_exp2(M - mn), s_new = fast_exp2(mu - mn);
      const float4 ou = sh.o[(u - 1) * NC + col];
      acc.x = acc.x * s_old + ou.x * s_new; acc.y = acc.y * s_old + ou.y * s_new;
      acc.z = acc.z * s_old + ou.z * s_new; acc.w = acc.w * s_old + ou.w * s_new;
      L = L * s_old + sh.l[(u - 1) * NC + col] * s_new;
      M = mn;
    }
  }
  const float il = L > 0.f ? 1.f / L : 0.f;
  *reinterpret_cast<float4*>(a.out + (qh0 + h) * D + 4 * c4) = make_float4(acc.x * il, acc.y * il, acc.z * il, acc.w * il);
}

// Tail of a fast-step workgroup: every wave's state to LDS, then the merge of
// the NW wave states.  A support of one chunk writes the output directly.
// Otherwise the chunk state is published for the merge:
//  * launches that fit the chip in one pass (a.ticket set) merge in the same
//    kernel: the workgroup publishes with device-coherent stores, waits for
//    them to complete and takes a ticket from the head's counter; the one
//    that draws the last ticket merges every chunk state into the output and
//    resets the counter to zero for the next call.  Nothing waits on another
//    workgroup, and no L2 write-back or invalidate is needed.
//  * larger launches store plainly and fast_merge_kernel merges afterwards:
//    there the wait for the stores and the ticket would hold a CU slot that
//    the next workgroup could already use.
// On the MFMA path a wave's output slot reuses its own V staging rows (its
// reads of them are complete).
// `late` issues stores that nothing in the kernel waits for (the packing of
// sfi_fast_step_pack): after the ticket, so that the wait for the chunk-state
// stores does not also wait for them, and in the last workgroup after the
// merge, whose loads would otherwise wait behind them.
template <typename A, int D, int G, int NW, int ROWS, bool MFMA, typename Late>
__device__ __forceinline__ void fast_finish(A& st, float* s_m, float* s_l, float* s_o, char* s_v,
                                            FastTailSmem<D, G>& sh, int wave, int lane, int tid, const FastArgs& a,
                                            int64_t eg, int64_t qh0, int chunk, int nchunk, Late&& late) {
  constexpr int kWaveBytes = ROWS * A::kRowBytes;
  if constexpr (MFMA) {
    wave_sync();
    st.finish_wave_mfma(s_m, s_l, reinterpret_cast<float*>(s_v + wave * kWaveBytes), wave, lane);
  } else {
    st.finish_wave_lds(s_m, s_l, s_o, wave, lane);
  }
  __syncthreads();
  const float* so = MFMA ? reinterpret_cast<const float*>(s_v) : s_o;
  constexpr int kStride = MFMA ? kWaveBytes / 4 : A::kRowGroups * G * D;
  constexpr int RG = MFMA ? 1 : A::kRowGroups;
  if (nchunk == 1) {
    merge_wave_groups<D, G, NW, RG>(s_m, s_l, so, kStride, tid, kFastThreads,
                                    [&](int h, int d, float4 acc, float, float L) {
                                      const float il = L > 0.f ? 1.f / L : 0.f;
                                      *reinterpret_cast<float4*>(a.out + (qh0 + h) * D + d) =
                                          make_float4(acc.x * il, acc.y * il, acc.z * il, acc.w * il);
                                    });
    late();
    return;
  }
  // one buffer descriptor per workgroup (its G heads' rows)
  float* mlg = a.part_ml + eg * G * a.part_stride * 2;
  float* og = a.part_o + eg * G * a.part_stride * D;
  if (a.ticket == nullptr) {
    merge_wave_groups<D, G, NW, RG>(s_m, s_l, so, kStride, tid, kFastThreads,
                                    [&](int h, int d, float4 acc, float M, float L) {
                                      *reinterpret_cast<float4*>(og + (h * a.part_stride + chunk) * D + d) = acc;
                                      if (d == 0)
                                        *reinterpret_cast<float2*>(mlg + (h * a.part_stride + chunk) * 2) =
                                            make_float2(M, L);
                                    });
    late();
    return;
  }
  const int ml_bytes = G * a.part_stride * 8, o_bytes = G * a.part_stride * D * 4;
  merge_wave_groups<D, G, NW, RG>(s_m, s_l, so, kStride, tid, kFastThreads,
                                  [&](int h, int d, float4 acc, float M, float L) {
                                    st16_dev(og, o_bytes, ((h * a.part_stride + chunk) * D + d) * 4, acc);
                                    if (d == 0) st8_dev(mlg, ml_bytes, (h * a.part_stride + chunk) * 8, make_float2(M, L));
                                  });
  wait_vmem();  // this thread's chunk-state stores have completed
  __syncthreads();
  int32_t* ticket = a.ticket + eg * kTicketStride;
  if (tid == 0) sh.last = __hip_atomic_fetch_add(ticket, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == nchunk - 1;
  __syncthreads();
  if (!sh.last) {
    late();
    return;
  }
  fast_merge_slots<D, G, true>(a, eg, qh0, nchunk, sh, tid);
  if (tid == 0) __hip_atomic_store(ticket, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  late();
}

// When the fast step that gathers also packs (sfi_fast_step_pack), the
// selected rows it loaded are stored either after the workgroup's ticket
// (launches that merge in the kernel: neither the wait for the chunk-state
// stores nor the last workgroup's merge waits behind them) or right after the
// attention math (launches that merge in the second kernel: the loaded rows
// then need not stay in registers through the tail, which keeps the register
// count, and so the workgroups per CU, of the plain gather).
constexpr int kPackNone = 0, kPackAfterTicket = 1, kPackAfterMath = 2;

// Fast step over the support gathered through sel_idx: each workgroup first
// resolves its chunk's support positions into LDS, then loads the rows.
// PACK (kPack*): whether and when to write the selected rows it loads to the
// packed buffers.
template <typename E, int D, int G, int TILES, bool ONE, int PACK>
__device__ __forceinline__ void fast_gather_body(const FastArgs& a, const FastSmem<E, D, G, TILES>& sm, int e) {
  using A = Attn<E, D, G>;
  constexpr int RB = A::kRowBytes;
  constexpr int ROWS = TILES * 16;  // rows per wave
  constexpr int NW = kFastThreads / 64;
  constexpr int CH = NW * ROWS;     // rows per workgroup
  constexpr int NV = ROWS / A::kRPL;

  constexpr bool kMfma = fast_pv_mfma<E, TILES>();
  float* s_p = sm.p;
  float* s_o = sm.o;
  char* s_v = sm.v;
  float* s_m = sm.m;
  float* s_l = sm.l;
  int* s_pos = sm.pos;
  FastTailSmem<D, G>& s_tail = *sm.tail;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wg = blockIdx.x;
  const int local = ONE ? wg : wg - a.tab.wg_begin[e];
  const int nchunk = a.tab.ent[e].nsplit;
  const int g = local / nchunk;
  const int chunk = local - g * nchunk;
  const int b = a.tab.ent[e].seq;
  const int t = row_ctx(a.tab, e);
  const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
  const SupportGeom sg = support_geom(t, a.n_sink, a.n_recent, a.top_k, a.sel_cnt, bg);
  const int32_t* sel_row = a.sel_idx + bg * a.top_k;
  const int c0 = chunk * CH;

  for (int i = tid; i < CH; i += kFastThreads) s_pos[i] = support_pos(sg, c0 + i, t, sel_row);
  __syncthreads();

  const int64_t kv_row0 = bg * a.t_cap;
  const char* Kb = static_cast<const char*>(a.k) + kv_row0 * RB;
  const char* Vb = static_cast<const char*>(a.v) + kv_row0 * RB;
  const int64_t qh0 = static_cast<int64_t>(b) * a.n_q_heads + g * G;

  uint4 qa[A::kNL];
  load_q<E, D, G>(a.q, qh0, lane, qa);
  A st;
  st.init();
  {
    const int kr = lane & 15, kg = lane >> 4;
    const int vr = lane / A::kPPR, vp = lane % A::kPPR;
    const int w0 = wave * ROWS;  // first row of this wave inside the chunk
    uint4 kb[TILES][A::kNL];
    uint4 vb[NV];
    bool kvalid[TILES];
    bool any = false;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) {
      const int pos = s_pos[w0 + 16 * tt + kr];
      kvalid[tt] = pos >= 0;
      any |= kvalid[tt];
      const char* src = Kb + static_cast<int64_t>(pos >= 0 ? pos : 0) * RB + 16 * kg;
#pragma unroll
      for (int kk = 0; kk < A::kNL; ++kk) kb[tt][kk] = ld16_stream(src + 64 * kk);
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int pos = s_pos[w0 + vr + A::kRPL * i];
      vb[i] = ld16_stream(Vb + static_cast<int64_t>(pos >= 0 ? pos : 0) * RB + 16 * vp);
    }
    // a wave whose rows are all outside the support keeps the empty state
    if (__ballot(any) != 0) {
      if constexpr (kMfma) {
        st.template consume_pv_mfma<TILES>(qa, kb, vb, kvalid, s_p + wave * ROWS * G, s_v + wave * ROWS * RB,
                                           a.scale_log2, lane);
      } else {
        st.template consume<TILES, true>(qa, kb, vb, kvalid, s_p + wave * ROWS * G, a.scale_log2, nullptr, 0, 0,
                                         lane);
      }
    }
    // Deferred packing: the selected rows this wave loaded also go to the
    // packed buffers at their selection slots (support element p is slot
    // p - fixed), through range-checked buffer stores: rows that are not
    // selected, or whose index is not a position of the context, get an
    // offset past the buffer and are dropped, as the packing pass skips them.
    auto pack_rows = [&] {
      if constexpr (PACK == kPackNone) return;
      const int fixed = sg.ns_eff + sg.w_eff;
      const uint32_t pbytes = static_cast<uint32_t>(a.top_k) * RB;
      const __amdgpu_buffer_rsrc_t rpk =
          buf_rsrc_u(static_cast<char*>(a.pack_out_k) + bg * a.top_k * RB, pbytes);
      const __amdgpu_buffer_rsrc_t rpv =
          buf_rsrc_u(static_cast<char*>(a.pack_out_v) + bg * a.top_k * RB, pbytes);
      auto slot_of = [&](int l) {
        const int slot = c0 + l - fixed;
        return slot >= 0 && slot < sg.cnt && s_pos[l] >= 0 ? slot : -1;
      };
#pragma unroll
      for (int tt = 0; tt < TILES; ++tt) {
        const int slot = slot_of(w0 + 16 * tt + kr);
#pragma unroll
        for (int kk = 0; kk < A::kNL; ++kk)
          buf_st16_stream(rpk, slot >= 0 ? static_cast<uint32_t>(slot) * RB + 64 * kk + 16 * kg : kOutOfRange, kb[tt][kk]);
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int slot = slot_of(w0 + vr + A::kRPL * i);
        buf_st16_stream(rpv, slot >= 0 ? static_cast<uint32_t>(slot) * RB + 16 * vp : kOutOfRange, vb[i]);
      }
    };
    if constexpr (PACK == kPackAfterMath) pack_rows();
    fast_finish<A, D, G, NW, ROWS, kMfma>(st, s_m, s_l, s_o, s_v, s_tail, wave, lane, tid, a,
                                          static_cast<int64_t>(e) * a.n_kv_heads + g, qh0, chunk, nchunk, [&] {
                                            if constexpr (PACK == kPackAfterTicket) pack_rows();
                                          });
  }
}

// Fast step over the packed support: the selected rows were copied into a
// contiguous buffer after the slow step (the memory-coalesced sparse layout
// of "Slow-Fast Inference ...", gist.science technical summary, 3
// "Systemdesign und Kernel-Optimierung"); sinks and the recent window are
// read from the cache.  Every row address follows from host-known lengths,
// so all K/V loads are issued at once with no index lookups; only the end of
// the selected rows (sel_cnt) masks the tail.
template <typename E, int D, int G, int TILES, bool ONE>
__device__ __forceinline__ void fast_packed_body(const FastArgs& a, const FastSmem<E, D, G, TILES>& sm, int e) {
  using A = Attn<E, D, G>;
  constexpr int RB = A::kRowBytes;
  constexpr int ROWS = TILES * 16;
  constexpr int NW = kFastThreads / 64;
  constexpr int NV = ROWS / A::kRPL;

  constexpr bool kMfma = fast_pv_mfma<E, TILES>();
  float* s_p = sm.p;
  float* s_o = sm.o;
  char* s_v = sm.v;
  float* s_m = sm.m;
  float* s_l = sm.l;
  FastTailSmem<D, G>& s_tail = *sm.tail;

  // the wave index as a scalar, so every test on a wave's rows is a scalar branch
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wg = blockIdx.x;
  const int local = ONE ? wg : wg - a.tab.wg_begin[e];
  const int nchunk = a.tab.ent[e].nsplit;
  const int g = local / nchunk;
  const int chunk = local - g * nchunk;
  const int b = a.tab.ent[e].seq;
  const int t = row_ctx(a.tab, e);
  const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
  const int ns_eff = min(a.n_sink, t);
  const int w_lo = max(a.n_sink, t - a.n_recent);
  const int w_eff = max(0, t - w_lo);
  const int kmax = min(a.top_k, max(0, t - a.n_sink - a.n_recent));
  const int fixed = ns_eff + w_eff;
  const char* Kc = static_cast<const char*>(a.k) + bg * a.t_cap * RB;
  const char* Vc = static_cast<const char*>(a.v) + bg * a.t_cap * RB;
  const char* Kp = static_cast<const char*>(a.packed_k) + bg * a.top_k * RB;
  const char* Vp = static_cast<const char*>(a.packed_v) + bg * a.top_k * RB;
  const int64_t qh0 = static_cast<int64_t>(b) * a.n_q_heads + g * G;
  uint4 qa[A::kNL];
  load_q<E, D, G>(a.q, qh0, lane, qa);
  A st;
  st.init();
  const int w0 = chunk * (NW * ROWS) + wave * ROWS;  // first support row of this wave
  const int kr = lane & 15, kg = lane >> 4;
  const int vr = lane / A::kPPR, vp = lane % A::kPPR;
  uint4 kb[TILES][A::kNL];
  uint4 vb[NV];
  // Row addresses, by wave-uniform tests: in waves whose rows are all packed
  // slots (most of them) a row is its buffer's base plus a 32-bit offset,
  // slots past kmax re-reading the last one (masked below); waves that reach
  // into the sinks or the window pick each row's source with selects; waves
  // past the largest possible support read cache row 0 (and compute
  // nothing).  Every wave then issues the same straight run of loads, so the
  // MFMAs wait for them one by one.
  const char* krow[TILES];
  const char* vrow[NV];
  if (w0 >= fixed + kmax) {
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) krow[tt] = Kc + 16 * kg;
#pragma unroll
    for (int i = 0; i < NV; ++i) vrow[i] = Vc + 16 * vp;
  } else if (w0 >= fixed) {
    const int q0 = w0 - fixed, qlast = kmax - 1;
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt)
      krow[tt] = Kp + (static_cast<uint32_t>(min(q0 + 16 * tt + kr, qlast)) * RB + 16 * kg);
#pragma unroll
    for (int i = 0; i < NV; ++i)
      vrow[i] = Vp + (static_cast<uint32_t>(min(q0 + vr + A::kRPL * i, qlast)) * RB + 16 * vp);
  } else {
    // support element p: a sink or window row of the cache, a packed slot,
    // or (past kmax) cache row 0
    auto src = [&](int p, const char* cache, const char* packed) -> const char* {
      const bool pk = p >= fixed && p - fixed < kmax;
      const int crow = p < ns_eff ? p : (p < fixed ? w_lo + p - ns_eff : 0);
      return pk ? packed + static_cast<int64_t>(p - fixed) * RB : cache + static_cast<int64_t>(crow) * RB;
    };
#pragma unroll
    for (int tt = 0; tt < TILES; ++tt) krow[tt] = src(w0 + 16 * tt + kr, Kc, Kp) + 16 * kg;
#pragma unroll
    for (int i = 0; i < NV; ++i) vrow[i] = src(w0 + vr + A::kRPL * i, Vc, Vp) + 16 * vp;
  }
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt)
#pragma unroll
    for (int kk = 0; kk < A::kNL; ++kk) kb[tt][kk] = ld16_stream(krow[tt] + 64 * kk);
#pragma unroll
  for (int i = 0; i < NV; ++i) vb[i] = ld16_stream(vrow[i]);
  const int cnt = min(max(a.sel_cnt[bg], 0), kmax);
  const int size = fixed + cnt;
  bool kvalid[TILES];
#pragma unroll
  for (int tt = 0; tt < TILES; ++tt) kvalid[tt] = (w0 + 16 * tt + kr) < size;
  // Rows past the support (packed slots cnt .. kmax - 1 were not written by
  // this span's selection) get zero V: their probability is zero, but 0 * V
  // would still turn a non-finite stale value into NaN.  Only the wave that
  // straddles the end of the support takes this branch.
  if (w0 < size && w0 + ROWS > size) {
#pragma unroll
    for (int i = 0; i < NV; ++i)
      if (w0 + vr + A::kRPL * i >= size) vb[i] = make_uint4(0u, 0u, 0u, 0u);
  }
  if (w0 < size) {
    if constexpr (kMfma) {
      st.template consume_pv_mfma<TILES>(qa, kb, vb, kvalid, s_p + wave * ROWS * G, s_v + wave * ROWS * RB,
                                         a.scale_log2, lane);
    } else {
      st.template consume<TILES, true>(qa, kb, vb, kvalid, s_p + wave * ROWS * G, a.scale_log2, nullptr, 0, 0,
                                       lane);
    }
  }
  fast_finish<A, D, G, NW, ROWS, kMfma>(st, s_m, s_l, s_o, s_v, s_tail, wave, lane, tid, a,
                                        static_cast<int64_t>(e) * a.n_kv_heads + g, qh0, chunk, nchunk, [] {});
}

// Waves per SIMD a fast-step kernel is compiled for.  Launches of several
// rows hold more workgroups than the CUs, so more of them resident means more
// loads in flight: for bf16 caches at two tiles per wave the code fits 128
// VGPRs without spilling, which with its LDS (under 40 KB) lets four
// workgroups share a CU instead of three.  One-row launches, which the
// in-kernel merge serves one workgroup per CU, and the other shapes keep the
// compiler's register choice.
template <typename E, int TILES, bool ONE>
constexpr int fast_waves_per_simd() {
  return !ONE && std::is_same<E, BF16>::value && TILES == 2 ? 4 : 1;
}

// ONE: a one-row launch, whose entry sits at fixed kernel-argument offsets
// that load with the other arguments (no table search).
template <typename E, int D, int G, int TILES, bool ONE>
__global__ __launch_bounds__(kFastThreads, (fast_waves_per_simd<E, TILES, ONE>())) void
fast_packed_kernel(FastArgs a) {
  fast_packed_body<E, D, G, TILES, ONE>(a, fast_smem<E, D, G, TILES>(), ONE ? 0 : find_entry(a.tab, blockIdx.x));
}

// PACK != kPackNone: the variants of sfi_fast_step_pack, which also write the
// selected rows they load to the packed buffers (separate instantiations, so
// that the plain fast step keeps its register budget)
template <typename E, int D, int G, int TILES, bool ONE, int PACK>
__global__ __launch_bounds__(kFastThreads, (fast_waves_per_simd<E, TILES, ONE || PACK == kPackAfterTicket>())) void
fast_partial_kernel(FastArgs a) {
  fast_gather_body<E, D, G, TILES, ONE, PACK>(a, fast_smem<E, D, G, TILES>(),
                                              ONE ? 0 : find_entry(a.tab, blockIdx.x));
}

// A launch of several sequences of which some gather and pack their selected
// rows (bit e of pack_mask set for table entry e: the span's first fast step)
// and the others read their packed support: each workgroup runs one of the two
// paths for its entry, sharing one LDS layout.  Such launches hold several
// rows and rarely fit the CUs in one pass, so the packing stores follow the
// attention math.
template <typename E, int D, int G, int TILES>
__global__ __launch_bounds__(kFastThreads, (fast_waves_per_simd<E, TILES, false>())) void
fast_mixed_kernel(FastArgs a) {
  const FastSmem<E, D, G, TILES> sm = fast_smem<E, D, G, TILES>();
  const int e = find_entry(a.tab, blockIdx.x);
  if ((a.pack_mask >> e) & 1u) {
    fast_gather_body<E, D, G, TILES, false, kPackAfterMath>(a, sm, e);
  } else {
    fast_packed_body<E, D, G, TILES, false>(a, sm, e);
  }
}

// Copies the selected K/V rows of each (sequence, KV head) into the packed
// buffers: packed[i] = cache[sel_idx[i]] for i < sel_cnt.
template <int RB>
__global__ __launch_bounds__(256) void pack_kernel(PackArgs a) {
  constexpr int NP = RB / 16;  // 16-byte pieces per row
  __shared__ int s_row[kPackRows];
  const int wg = blockIdx.x;
  const int e = find_entry(a.tab, wg);
  const int local = wg - a.tab.wg_begin[e];
  const int nchunk = a.tab.ent[e].nsplit;
  const int g = local / nchunk;
  const int chunk = local - g * nchunk;
  const int b = a.tab.ent[e].seq;
  const int t = row_ctx(a.tab, e);
  const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
  const int kmax = min(a.top_k, max(0, t - a.n_sink - a.n_recent));
  const int cnt = min(max(a.sel_cnt[bg], 0), kmax);
  const int r0 = chunk * kPackRows;
  for (int i = threadIdx.x; i < kPackRows; i += 256) {
    const int r = r0 + i;
    int j = -1;
    if (r < cnt) {
      j = a.sel_idx[bg * a.top_k + r];
      if (j < 0 || j >= t) j = -1;
    }
    s_row[i] = j;
  }
  __syncthreads();
  const char* K = static_cast<const char*>(a.k) + bg * a.t_cap * RB;
  const char* V = static_cast<const char*>(a.v) + bg * a.t_cap * RB;
  char* PK = static_cast<char*>(a.packed_k) + bg * a.top_k * RB;
  char* PV = static_cast<char*>(a.packed_v) + bg * a.top_k * RB;
  constexpr int kItems = kPackRows * NP * 2;
  constexpr int kPer = kItems / 256;
  uint4 val[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int item = threadIdx.x + 256 * u;
    const int isv = item >= kPackRows * NP;
    const int rem = isv ? item - kPackRows * NP : item;
    const int row = rem / NP, pc = rem - row * NP;
    const int j = s_row[row];
    val[u] = j >= 0 ? ld16((isv ? V : K) + static_cast<int64_t>(j) * RB + 16 * pc) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int item = threadIdx.x + 256 * u;
    const int isv = item >= kPackRows * NP;
    const int rem = isv ? item - kPackRows * NP : item;
    const int row = rem / NP, pc = rem - row * NP;
    if (s_row[row] >= 0)
      *reinterpret_cast<uint4*>((isv ? PV : PK) + static_cast<int64_t>(r0 + row) * RB + 16 * pc) = val[u];
  }
}

// Merge of the chunk states of one (sequence, KV head) after a fast-step
// launch that published them with plain stores: the output of its G query
// heads, renormalised over the whole support.
template <int D, int G, bool ONE>
__global__ __launch_bounds__(kFastThreads) void fast_merge_kernel(FastArgs a) {
  __shared__ FastTailSmem<D, G> s_tail;
  const int e = ONE ? 0 : blockIdx.x / a.n_kv_heads;
  const int g = ONE ? blockIdx.x : blockIdx.x - e * a.n_kv_heads;
  const int b = a.tab.ent[e].seq;
  const int nchunk = a.tab.ent[e].nsplit;
  if (nchunk == 1) return;  // the partial kernel wrote the output
  const int64_t qh0 = static_cast<int64_t>(b) * a.n_q_heads + g * G;
  fast_merge_slots<D, G, false>(a, static_cast<int64_t>(e) * a.n_kv_heads + g, qh0, nchunk, s_tail, threadIdx.x);
}

// ---------------------------------------------------------------------------
// debug: materialise the fast-step support
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void support_kernel(SupportArgs a) {
  const int e = blockIdx.x / a.n_kv_heads;
  const int g = blockIdx.x - e * a.n_kv_heads;
  const int b = a.tab.ent[e].seq;
  const int t = row_ctx(a.tab, e);
  const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
  const SupportGeom sg = support_geom(t, a.n_sink, a.n_recent, a.top_k, a.sel_cnt, bg);
  const int32_t* sel_row = a.sel_idx + bg * a.top_k;
  int32_t* out = a.support_out + bg * a.cap_per_head;
  for (int p = threadIdx.x; p < a.cap_per_head; p += blockDim.x)
    out[p] = p < sg.size ? support_pos(sg, p, t, sel_row) : -1;
  if (threadIdx.x == 0) a.support_cnt[bg] = sg.size;
}

// ---------------------------------------------------------------------------
// KV append and workspace clearing
// ---------------------------------------------------------------------------
// Appends one token to each listed row: K/V of every KV head go to row t of
// the cache, t = the row's context length.  With device context lengths the
// row's value is read once by the whole workgroup and then advanced by one in
// place (a full cache, t >= T_cap, is left unchanged).
template <int RB>
__global__ __launch_bounds__(256) void append_kernel(AppendArgs a) {
  __shared__ int s_t;
  const int e = blockIdx.x;
  const int b = a.tab.ent[e].seq;
  if (threadIdx.x == 0) s_t = a.tab.ctx_dev != nullptr ? a.tab.ctx_dev[b] : a.tab.ent[e].ctx;
  __syncthreads();
  const int t = s_t;
  if (t < 0 || t >= a.t_cap) return;
  constexpr int NP = RB / 16;
  for (int i = threadIdx.x; i < a.n_kv_heads * 2 * NP; i += 256) {
    const int g = i / (2 * NP), r = i - g * 2 * NP;
    const bool isv = r >= NP;
    const int pc = isv ? r - NP : r;
    const int64_t bg = static_cast<int64_t>(b) * a.n_kv_heads + g;
    const char* src = static_cast<const char*>(isv ? a.v_new : a.k_new) + bg * RB + 16 * pc;
    char* dst = static_cast<char*>(isv ? a.v : a.k) + (bg * a.t_cap + t) * RB + 16 * pc;
    *reinterpret_cast<uint4*>(dst) = ld16(src);
  }
  if (a.tab.ctx_dev != nullptr && threadIdx.x == 0) const_cast<int32_t*>(a.tab.ctx_dev)[b] = t + 1;
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint32_t* p, size_t words) {
  for (size_t i = blockIdx.x * 256ull + threadIdx.x; i < words; i += gridDim.x * 256ull) p[i] = 0u;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
template <typename E, int D, bool NORMS>
static hipError_t slow_partial_gn(const SlowArgs& a, int group, int grid, hipStream_t s) {
  switch (group) {
    case 1: launch(slow_partial_kernel<E, D, 1, NORMS>, grid, kSlowThreads, s, a); break;
    case 2: launch(slow_partial_kernel<E, D, 2, NORMS>, grid, kSlowThreads, s, a); break;
    case 4: launch(slow_partial_kernel<E, D, 4, NORMS>, grid, kSlowThreads, s, a); break;
    case 8: launch(slow_partial_kernel<E, D, 8, NORMS>, grid, kSlowThreads, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename E, int D>
static hipError_t slow_partial_g(const SlowArgs& a, int group, int grid, hipStream_t s) {
  return a.knorm != nullptr ? slow_partial_gn<E, D, true>(a, group, grid, s)
                            : slow_partial_gn<E, D, false>(a, group, grid, s);
}

hipError_t launch_slow_partial(const SlowArgs& a, int dtype, int head_dim, int group, int grid,
                               hipStream_t s) {
  if (dtype == SFI_BF16) {
    return head_dim == 128 ? slow_partial_g<BF16, 128>(a, group, grid, s)
                           : slow_partial_g<BF16, 64>(a, group, grid, s);
  }
  return head_dim == 128 ? slow_partial_g<F32, 128>(a, group, grid, s)
                         : slow_partial_g<F32, 64>(a, group, grid, s);
}

template <int D, bool HIST>
static hipError_t slow_combine_g(const CombineArgs& a, int group, int grid, hipStream_t s) {
  switch (group) {
    case 1: launch(slow_combine_kernel<D, 1, HIST>, grid, kCombineThreads, s, a); break;
    case 2: launch(slow_combine_kernel<D, 2, HIST>, grid, kCombineThreads, s, a); break;
    case 4: launch(slow_combine_kernel<D, 4, HIST>, grid, kCombineThreads, s, a); break;
    case 8: launch(slow_combine_kernel<D, 8, HIST>, grid, kCombineThreads, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_slow_combine(const CombineArgs& a, int head_dim, int group, int grid,
                               hipStream_t s) {
  if (a.sel_hist != nullptr && a.mass != nullptr)
    return head_dim == 128 ? slow_combine_g<128, true>(a, group, grid, s)
                           : slow_combine_g<64, true>(a, group, grid, s);
  return head_dim == 128 ? slow_combine_g<128, false>(a, group, grid, s)
                         : slow_combine_g<64, false>(a, group, grid, s);
}

// Fast-step rows per wave (16 per tile).  Small chunks keep many workgroups
// in flight, which a latency-bound gather of ~10 MB needs; the count is a
// launch parameter (1, 2 or 4 tiles per wave; 2 measured fastest on the 128K
// layer).
int fast_tiles() {
  static const int t = [] {
    const char* s = std::getenv("SFI_FAST_TILES");
    const int v = s ? std::atoi(s) : 2;
    return (v == 1 || v == 4) ? v : 2;
  }();
  return t;
}

int fast_chunk_rows() { return (kFastThreads / 64) * fast_tiles() * 16; }

template <typename E, int D, int G, int TILES>
static void fast_partial_launch(const FastArgs& a, int grid, hipStream_t s) {
  const bool one = a.tab.n == 1;
  if (a.packed_k != nullptr && a.pack_out_k != nullptr) {
    launch(fast_mixed_kernel<E, D, G, TILES>, grid, kFastThreads, s, a);
  } else if (a.packed_k != nullptr) {
    if (one) launch(fast_packed_kernel<E, D, G, TILES, true>, grid, kFastThreads, s, a);
    else launch(fast_packed_kernel<E, D, G, TILES, false>, grid, kFastThreads, s, a);
  } else if (a.pack_out_k != nullptr && a.ticket != nullptr) {
    if (one) launch(fast_partial_kernel<E, D, G, TILES, true, kPackAfterTicket>, grid, kFastThreads, s, a);
    else launch(fast_partial_kernel<E, D, G, TILES, false, kPackAfterTicket>, grid, kFastThreads, s, a);
  } else if (a.pack_out_k != nullptr) {
    if (one) launch(fast_partial_kernel<E, D, G, TILES, true, kPackAfterMath>, grid, kFastThreads, s, a);
    else launch(fast_partial_kernel<E, D, G, TILES, false, kPackAfterMath>, grid, kFastThreads, s, a);
  } else {
    if (one) launch(fast_partial_kernel<E, D, G, TILES, true, kPackNone>, grid, kFastThreads, s, a);
    else launch(fast_partial_kernel<E, D, G, TILES, false, kPackNone>, grid, kFastThreads, s, a);
  }
}

template <typename E, int D>
static hipError_t fast_partial_g(const FastArgs& a, int group, int grid, hipStream_t s) {
  const int tiles = a.chunk_rows / ((kFastThreads / 64) * 16);
  switch (group * 8 + tiles) {
    case 1 * 8 + 1: fast_partial_launch<E, D, 1, 1>(a, grid, s); break;
    case 1 * 8 + 2: fast_partial_launch<E, D, 1, 2>(a, grid, s); break;
    case 1 * 8 + 4: fast_partial_launch<E, D, 1, 4>(a, grid, s); break;
    case 2 * 8 + 1: fast_partial_launch<E, D, 2, 1>(a, grid, s); break;
    case 2 * 8 + 2: fast_partial_launch<E, D, 2, 2>(a, grid, s); break;
    case 2 * 8 + 4: fast_partial_launch<E, D, 2, 4>(a, grid, s); break;
    case 4 * 8 + 1: fast_partial_launch<E, D, 4, 1>(a, grid, s); break;
    case 4 * 8 + 2: fast_partial_launch<E, D, 4, 2>(a, grid, s); break;
    case 4 * 8 + 4: fast_partial_launch<E, D, 4, 4>(a, grid, s); break;
    case 8 * 8 + 1: fast_partial_launch<E, D, 8, 1>(a, grid, s); break;
    case 8 * 8 + 2: fast_partial_launch<E, D, 8, 2>(a, grid, s); break;
    case 8 * 8 + 4: fast_partial_launch<E, D, 8, 4>(a, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fast_partial(const FastArgs& a, int dtype, int head_dim, int group, int grid,
                               hipStream_t s) {
  if (dtype == SFI_BF16) {
    return head_dim == 128 ? fast_partial_g<BF16, 128>(a, group, grid, s)
                           : fast_partial_g<BF16, 64>(a, group, grid, s);
  }
  return head_dim == 128 ? fast_partial_g<F32, 128>(a, group, grid, s)
                         : fast_partial_g<F32, 64>(a, group, grid, s);
}

template <int D, bool ONE>
static hipError_t fast_merge_one(const FastArgs& a, int group, hipStream_t s) {
  const int grid = a.tab.n * a.n_kv_heads;
  switch (group) {
    case 1: launch(fast_merge_kernel<D, 1, ONE>, grid, kFastThreads, s, a); break;
    case 2: launch(fast_merge_kernel<D, 2, ONE>, grid, kFastThreads, s, a); break;
    case 4: launch(fast_merge_kernel<D, 4, ONE>, grid, kFastThreads, s, a); break;
    case 8: launch(fast_merge_kernel<D, 8, ONE>, grid, kFastThreads, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
static hipError_t fast_merge_g(const FastArgs& a, int group, hipStream_t s) {
  return a.tab.n == 1 ? fast_merge_one<D, true>(a, group, s) : fast_merge_one<D, false>(a, group, s);
}

hipError_t launch_fast_merge(const FastArgs& a, int head_dim, int group, hipStream_t s) {
  return head_dim == 128 ? fast_merge_g<128>(a, group, s) : fast_merge_g<64>(a, group, s);
}

hipError_t launch_support(const SupportArgs& a, int grid, hipStream_t s) {
  launch(support_kernel, grid, 256, s, a);
  return hipGetLastError();
}

hipError_t launch_pack(const PackArgs& a, int dtype, int head_dim, int grid, hipStream_t s) {
  const int rb = head_dim * (dtype == SFI_BF16 ? 2 : 4);
  switch (rb) {
    case 128: launch(pack_kernel<128>, grid, 256, s, a); break;
    case 256: launch(pack_kernel<256>, grid, 256, s, a); break;
    case 512: launch(pack_kernel<512>, grid, 256, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_append(const AppendArgs& a, int dtype, int head_dim, int grid, hipStream_t s) {
  const int rb = head_dim * (dtype == SFI_BF16 ? 2 : 4);
  switch (rb) {
    case 128: launch(append_kernel<128>, grid, 256, s, a); break;
    case 256: launch(append_kernel<256>, grid, 256, s, a); break;
    case 512: launch(append_kernel<512>, grid, 256, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return hipSuccess;
  const int grid = static_cast<int>(std::min<size_t>((words + 255) / 256, 1024));
  launch(fill_zero_kernel, grid, 256, s, static_cast<uint32_t*>(p), words);
  return hipGetLastError();
}

}  // namespace sfi
