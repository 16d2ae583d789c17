// Device helpers for the gfx950 kernels: element traits, 16-byte loads,
// bf16 widening, the 16x16 MFMA logit tile and 16-lane DPP reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sfi {

typedef __attribute__((__vector_size__(8 * sizeof(short)))) short bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

struct BF16 {};
struct F32 {};

template <typename E> struct Elem;
template <> struct Elem<BF16> {
  static constexpr int kBytes = 2;
  static constexpr int kPerPiece = 8;  // elements in a 16-byte piece
};
template <> struct Elem<F32> {
  static constexpr int kBytes = 4;
  static constexpr int kPerPiece = 4;
};

// 16-byte global load (global_load_dwordx4).
__device__ __forceinline__ uint4 ld16(const void* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// 16-byte streaming load: the non-temporal hint (`nt`) marks data read once,
// so streaming it does not push reusable lines (such as the logits the next
// kernel reads back) out of the caches.
__device__ __forceinline__ uint4 ld16_stream(const void* p) {
  typedef unsigned int u4v __attribute__((ext_vector_type(4)));
  const u4v v = __builtin_nontemporal_load(reinterpret_cast<const u4v*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Write-through stores (system coherence, sc0 sc1): the data goes out to
// memory as it is stored instead of staying dirty in the XCD's L2 until an
// eviction.  Used for the slow step's logits, written while the kernel
// streams K and V, where it measured faster than write-back stores; the
// other bulk outputs keep plain stores, which measured as fast or faster.
//
// st16_wt: 16 bytes at byte offset `off` of the buffer [base, base + bytes),
// one buffer_store_dwordx4 per lane (a store outside the range is dropped by
// the buffer's range check).  0x00020000 is the gfx9 buffer descriptor's
// word 3 for untyped 32-bit data; 17 = sc0 | sc1 cache-policy bits.
__device__ __forceinline__ void st16_wt(float* base, int32_t bytes, int32_t off, float4 v) {
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(base, static_cast<short>(0), bytes, 0x00020000);
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4 d = {static_cast<int>(__float_as_uint(v.x)), static_cast<int>(__float_as_uint(v.y)),
                static_cast<int>(__float_as_uint(v.z)), static_cast<int>(__float_as_uint(v.w))};
  __builtin_amdgcn_raw_buffer_store_b128(d, rs, off, 0, 17);
}
// st4_wt: one float (a relaxed system-scope atomic store: global_store_dword
// with sc0 sc1).
__device__ __forceinline__ void st4_wt(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

// Device-coherent accesses: cache policy sc1, the bits the gfx950 memory model
// gives relaxed agent-scope atomic loads and stores, so a store is visible to
// a later sc1 load from any XCD without an L2 write-back or invalidate.  The
// fast step's workgroups publish their partial states this way and the last
// one of a head reads them back this way.  `bytes` bounds the buffer that
// starts at `base`; accesses at byte offset `off`.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, int32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), bytes, 0x00020000);
}
constexpr int kCpolDevice = 16;  // sc1
__device__ __forceinline__ void st16_dev(float* base, int32_t bytes, int32_t off, float4 v) {
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4 d = {static_cast<int>(__float_as_uint(v.x)), static_cast<int>(__float_as_uint(v.y)),
                static_cast<int>(__float_as_uint(v.z)), static_cast<int>(__float_as_uint(v.w))};
  __builtin_amdgcn_raw_buffer_store_b128(d, buf_rsrc(base, bytes), off, 0, kCpolDevice);
}
__device__ __forceinline__ void st8_dev(float* base, int32_t bytes, int32_t off, float2 v) {
  typedef int i2 __attribute__((ext_vector_type(2)));
  const i2 d = {static_cast<int>(__float_as_uint(v.x)), static_cast<int>(__float_as_uint(v.y))};
  __builtin_amdgcn_raw_buffer_store_b64(d, buf_rsrc(base, bytes), off, 0, kCpolDevice);
}
__device__ __forceinline__ float4 ld16_dev(const float* base, int32_t bytes, int32_t off) {
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4 d = __builtin_amdgcn_raw_buffer_load_b128(buf_rsrc(base, bytes), off, 0, kCpolDevice);
  return make_float4(__int_as_float(d.x), __int_as_float(d.y), __int_as_float(d.z), __int_as_float(d.w));
}
__device__ __forceinline__ float2 ld8_dev(const float* base, int32_t bytes, int32_t off) {
  typedef int i2 __attribute__((ext_vector_type(2)));
  const i2 d = __builtin_amdgcn_raw_buffer_load_b64(buf_rsrc(base, bytes), off, 0, kCpolDevice);
  return make_float2(__int_as_float(d.x), __int_as_float(d.y));
}
// Range-checked 16-byte accesses through a wave-uniform buffer descriptor: a
// load at an offset past the buffer returns zeros without touching memory and
// a store there is dropped, so work lists that fill a wave only partly need no
// branches (and the compiler keeps exact counts of the accesses in flight).
// `bytes` is the buffer's size, below the out-of-range offset (0xFFFFFFFF)
// by at least 16.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc_u(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int32_t>(bytes), 0x00020000);
}
// streaming (non-temporal, cache policy nt) load
__device__ __forceinline__ uint4 buf_ld16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4 d = __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int32_t>(off), 0, 2);
  return make_uint4(static_cast<uint32_t>(d.x), static_cast<uint32_t>(d.y), static_cast<uint32_t>(d.z),
                    static_cast<uint32_t>(d.w));
}
// streaming (nt) store of 16 bytes: for rows written once and not read again
// in the same kernel, the packed support rows (the fast step's packing
// measured about 1 us faster with it than with plain stores, the Selector's
// emission about 0.5 us).
__device__ __forceinline__ void buf_st16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off, uint4 v) {
  typedef int i4 __attribute__((ext_vector_type(4)));
  const i4 d = {static_cast<int>(v.x), static_cast<int>(v.y), static_cast<int>(v.z), static_cast<int>(v.w)};
  __builtin_amdgcn_raw_buffer_store_b128(d, r, static_cast<int32_t>(off), 0, 2);
}

// s_waitcnt vmcnt(0): this wave's earlier vector memory accesses, stores
// included, have completed (expcnt and lgkmcnt fields left at their maxima).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float4 ld16_stream_f(const float* p) {
  const uint4 u = ld16_stream(p);
  return make_float4(__uint_as_float(u.x), __uint_as_float(u.y), __uint_as_float(u.z), __uint_as_float(u.w));
}

// Widen a 16-byte piece to floats.  bf16 -> f32 is exact (shift into the
// high half of the word).
__device__ __forceinline__ void widen(BF16, const uint4& u, float* f) {
  const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(w[i] << 16);
    f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void widen(F32, const uint4& u, float* f) {
  f[0] = __uint_as_float(u.x);
  f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z);
  f[3] = __uint_as_float(u.w);
}

// One 16-byte piece of K (operand B, 16 rows x 32 or 4x4 k-values) times the
// matching piece of Q (operand A, 16 head rows), accumulated into c.
//   lane l supplies row (l % 16) and k-group (l / 16) of both operands;
//   c item e of lane l is C[head 4 * (l / 16) + e][row l % 16].
__device__ __forceinline__ f32x4_t mfma_piece(BF16, const uint4& q, const uint4& k, f32x4_t c) {
  bf16x8_t a, b;
  __builtin_memcpy(&a, &q, 16);
  __builtin_memcpy(&b, &k, 16);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4_t mfma_piece(F32, const uint4& q, const uint4& k, f32x4_t c) {
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.x), __uint_as_float(k.x), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.y), __uint_as_float(k.y), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.z), __uint_as_float(k.z), c, 0, 0, 0);
  c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(q.w), __uint_as_float(k.w), c, 0, 0, 0);
  return c;
}

// gfx950 transposing LDS read (ds_read_b64_tr_b16) of the 8 bytes at `p`, an
// address in LDS.  Within each 16-lane group, lane 4 s + e receives element e
// (of four 16-bit elements) of the words read by lanes s, 4 + s, 8 + s and
// 12 + s.
typedef short v4i16_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16_t lds_v4i16_t;
__device__ __forceinline__ v4i16_t lds_read_tr16(const char* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16_t*)(p));
}

// DPP lane exchanges inside a row of 16 lanes.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppQuadSwap1 = 0xB1;  // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;  // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;

// Max / sum over the 16 lanes of a row; every lane of the row gets the result.
__device__ __forceinline__ float row16_max(float x) {
  x = fmaxf(x, dpp<kDppQuadSwap1>(x));
  x = fmaxf(x, dpp<kDppQuadSwap2>(x));
  x = fmaxf(x, dpp<kDppHalfMirror>(x));
  x = fmaxf(x, dpp<kDppMirror>(x));
  return x;
}
__device__ __forceinline__ float row16_sum(float x) {
  x += dpp<kDppQuadSwap1>(x);
  x += dpp<kDppQuadSwap2>(x);
  x += dpp<kDppHalfMirror>(x);
  x += dpp<kDppMirror>(x);
  return x;
}

__device__ __forceinline__ float lane_bcast(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Context length of launch-table entry e: the device value when the table
// carries one (clamped to [1, the planned bound]), else the planned one.
template <typename Table>
__device__ __forceinline__ int row_ctx(const Table& t, int e) {
  const int bound = t.ent[e].ctx;
  if (t.ctx_dev == nullptr) return bound;
  return min(max(t.ctx_dev[t.ent[e].seq], 1), bound);
}

// Locate the table entry owning workgroup `wg` (tables are short).
template <typename Table>
__device__ __forceinline__ int find_entry(const Table& t, int wg) {
  int e = 0;
  while (e + 1 < t.n && t.wg_begin[e + 1] <= wg) ++e;
  return e;
}

}  // namespace sfi
