// Internal declarations shared by the HIP kernel sources and the host runtime
// of the SFI decode-attention library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sfi.h"

namespace sfi {

// Batch rows handled by one launch; larger lists are split into several
// launches.  The table travels in the kernel-argument block.
constexpr int kMaxSeqPerLaunch = 64;

// Workgroup shapes.
constexpr int kSlowThreads = 256;    // 4 waves, split-K partial kernel
constexpr int kCombineThreads = 256; // merge + mass kernel
constexpr int kMassChunk = 4096;     // positions per mass workgroup
constexpr int kSelectThreads = 1024; // one workgroup per (sequence, KV head)
constexpr int kFastThreads = 256;    // 4 waves, gather kernel

struct SeqTable {
  int32_t n;                              // entries used
  int32_t seq[kMaxSeqPerLaunch];          // batch row
  int32_t ctx[kMaxSeqPerLaunch];          // context length T_b
  int32_t nsplit[kMaxSeqPerLaunch];       // workgroups per KV head of this row
  int32_t wg_begin[kMaxSeqPerLaunch + 1]; // prefix over entries of Hkv * nsplit
};

// ---- slow step -----------------------------------------------------------
struct SlowArgs {
  const void* k;
  const void* v;
  const void* q;
  float* logits;   // [B][Hq][T_cap] scaled log2-domain logits, or nullptr
  float* part_ml;  // [B][Hq][part_stride][2]  (running max, running sum)
  float* part_o;   // [B][Hq][part_stride][D]  un-normalised output
  float* out;      // [B][Hq][D]
  float* mass;     // [B][Hkv][T_cap] or nullptr
  int64_t t_cap;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t split_rows;   // rows per split-K workgroup (multiple of 4 * block rows)
  int32_t part_stride;  // max splits per head (workspace pitch)
  float scale_log2;     // logit scale times log2(e)
  SeqTable tab;
};

struct CombineArgs {
  const float* logits;
  const float* part_ml;
  const float* part_o;
  float* out;
  float* mass;
  int64_t t_cap;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t part_stride;
  SeqTable tab;  // nsplit = split-K splits; wg_begin counts combine workgroups
  int32_t mass_blocks[kMaxSeqPerLaunch];  // per entry: mass workgroups per KV head
};

// ---- select --------------------------------------------------------------
struct SelectArgs {
  const float* mass;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  int64_t t_cap;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  float lambda;
  SeqTable tab;  // wg_begin = entry * Hkv
};

// ---- fast step -----------------------------------------------------------
struct FastArgs {
  const void* k;
  const void* v;
  const void* q;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  float* part_ml;   // [B][Hq][part_stride][2]
  float* part_o;    // [B][Hq][part_stride][D]
  int32_t* counter; // [B][Hkv] arrival counters (zero between launches)
  float* out;
  int64_t t_cap;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  int32_t chunk_rows;   // support rows per workgroup
  int32_t part_stride;
  float scale_log2;
  SeqTable tab;         // nsplit = chunks per KV head
};

struct SupportArgs {
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int32_t* support_out;
  int32_t* support_cnt;
  int64_t t_cap;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  int32_t cap_per_head;
  SeqTable tab;
};

struct AppendArgs {
  void* k;
  void* v;
  const void* k_new;
  const void* v_new;
  int64_t t_cap;
  int32_t n_kv_heads;
  SeqTable tab;
};

// Launchers (defined next to their kernels).  They only enqueue; arguments
// were validated by the caller.  Return the launch's hipError_t.
hipError_t launch_slow_partial(const SlowArgs& a, int dtype, int head_dim, int group,
                               int grid, hipStream_t s);
hipError_t launch_slow_combine(const CombineArgs& a, int head_dim, int group, int grid,
                               hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int grid, hipStream_t s);
hipError_t launch_fast(const FastArgs& a, int dtype, int head_dim, int group, int grid,
                       hipStream_t s);
hipError_t launch_support(const SupportArgs& a, int grid, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, int dtype, int head_dim, int grid,
                         hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// Support rows handled by one fast-step workgroup.
int fast_chunk_rows();

// Rows handled per wave per pipeline block: 16 KiB of K (and of V) per block.
__host__ __device__ constexpr int block_rows(int row_bytes) { return 16384 / row_bytes; }

}  // namespace sfi
