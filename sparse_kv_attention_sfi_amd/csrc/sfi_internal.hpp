// Internal declarations shared by the HIP kernel sources and the host runtime
// of the SFI decode-attention library (gfx950 only).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sfi.h"

namespace sfi {

// Batch rows handled by one launch; larger lists are split into several
// launches.  The table travels in the kernel-argument block.
constexpr int kMaxSeqPerLaunch = 64;

// Largest batch and KV-head count a descriptor may name: with them every
// workspace size fits 64 bits and every launch grid 32 bits.
constexpr int kMaxBatch = 65536;
constexpr int kMaxKvHeads = 256;

// Workgroup shapes.
constexpr int kSlowThreads = 256;    // 4 waves, split-K partial kernel
constexpr int kCombineThreads = 1024; // merge + mass kernel
constexpr int kMassChunk = 8192;      // positions per mass workgroup
constexpr int kSelThreads = 512;     // Selector workgroups
constexpr int kSelListCap = 8192;    // threshold-bin keys resolved in LDS
constexpr int kSelMaxChunks = 1024;  // candidate chunks per (sequence, KV head)
constexpr int kSelMinChunk = 4096;   // candidates per chunk (at least)
constexpr int kFastThreads = 256;    // 4 waves, fast-step kernels
constexpr int kMaxMergeSlots = 512;  // partial slots per (sequence, head) a merge accepts
constexpr int kSlowTargetWgs = 1024;  // slow partial workgroups aimed at per launch
constexpr int kLogitBufRows = 1024;   // slow partial: a split's logits are buffered in LDS up to this size
constexpr int kSlowMinRows = 512;     // slow partial: splits of at least this many rows where possible
constexpr int kTicketStride = 32;     // fast-step chunk counters, one per 128-byte line
constexpr uint32_t kOutOfRange = 0xFFFFFFFFu;  // a buffer offset past every buffer: loads give 0, stores drop

// One launch's rows.  A row's fields sit together in one 16-byte record, so
// a workgroup fetches them with one scalar load.
struct SeqEntry {
  int32_t seq;     // batch row
  int32_t ctx;     // context length T_b
  int32_t nsplit;  // workgroups per KV head of this row
  int32_t pad;
};

struct SeqTable {
  int32_t n;  // entries used
  int32_t pad;
  // device context lengths [B] or nullptr; when set, a row's context length
  // is read here and its entry's ctx is the upper bound the launch was
  // planned for (row_ctx clamps to [1, bound])
  const int32_t* ctx_dev;
  SeqEntry ent[kMaxSeqPerLaunch];
  int32_t wg_begin[kMaxSeqPerLaunch + 1];  // prefix over entries of Hkv * nsplit
};

// ---- slow step -----------------------------------------------------------
struct SlowArgs {
  const void* k;
  const void* v;
  const void* q;
  float* logits;   // [B][Hq][logit_pitch] scaled log2-domain logits, or nullptr
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
  int64_t logit_pitch;  // floats per logit row (multiple of 64)
  // optional: Selector bookkeeping the first split of each head clears
  uint32_t* clear_hist;    // [B * Hkv][4096] or nullptr
  int32_t* clear_list_n;   // [B * Hkv]
  // optional: key norms of every row, and per split the sums of the
  // candidates' norms and squared norms (the key-norm prior's statistics)
  float* knorm;            // [B][Hkv][T_cap] or nullptr
  double* knorm_part;      // [B * Hkv][part_stride][2]
  int32_t n_sink;          // candidates are [n_sink, T - n_recent)
  int32_t n_recent;
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
  int64_t logit_pitch;
  // optional: the Selector's top-digit histogram built next to the mass
  uint32_t* sel_hist;  // [B * Hkv][4096] or nullptr
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  float lambda;
  // optional: the key-norm prior's statistics and normaliser partial sums
  const double* knorm_part;  // [B * Hkv][part_stride][2] or nullptr
  const float* knorm;        // [B][Hkv][T_cap]
  double* knorm_stat;        // [B * Hkv][2]: mean and standard deviation of the candidates' norms
  double* zpart;             // [B * Hkv][zpart_stride]: per mass block, sum of the penalised positional weights
  int32_t zpart_stride;
  float knorm_beta;
  float knorm_c;
  SeqTable tab;  // nsplit = split-K splits; wg_begin counts combine workgroups
  int32_t mass_blocks[kMaxSeqPerLaunch];  // per entry: mass workgroups per KV head
};

// ---- select --------------------------------------------------------------
struct SelectArgs {
  const float* mass;
  int32_t* sel_idx;
  int32_t* sel_cnt;
  // per-head bookkeeping, zero at the start of every call
  uint32_t* hist;        // [B * Hkv][4096] top-digit histogram
  int32_t* list_n;       // [B * Hkv] keys appended to the threshold-bin list
  // per-call scratch
  uint64_t* list;        // [B * Hkv][kSelListCap] keys of the threshold bin
  int32_t* chunk_above;  // [B * Hkv][kSelMaxChunks] keys above the bin per chunk
  int32_t* above_pos;    // [B * Hkv][t_cap]: from each chunk's first candidate on, the
                         // candidate indices of its keys above the bin, ascending
  int32_t* head_info;    // [B * Hkv][2] threshold bin, keys above it
  int64_t t_cap;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  int32_t chunk;         // candidates per workgroup
  float lambda;
  bool hist_ready;       // the top-digit histogram was built with the mass
  bool pre_scores;       // `mass` holds the candidates' final scores (select_score_kernel)
  // optional: copy the kept rows into packed buffers while emitting them
  const void* k;
  const void* v;
  void* packed_k;        // [B][Hkv][top_k][D] or nullptr
  void* packed_v;
  int32_t row_bytes;
  bool rows32;           // a KV head's cache rows and packed slots fit 32-bit byte offsets
  SeqTable tab;          // nsplit = chunks per KV head
};

// ---- fast step -----------------------------------------------------------
struct FastArgs {
  const void* k;
  const void* v;
  const void* packed_k;  // [B][Hkv][top_k][D] selected rows, or nullptr (gather by index)
  const void* packed_v;
  const void* q;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  // gather path only: also write the selected rows it reads into these packed
  // buffers ([B][Hkv][top_k][D], at their selection slots), or nullptr
  void* pack_out_k;
  void* pack_out_v;
  // with both packed_k and pack_out_k set (a mixed launch, the same buffers):
  // bit e set = table entry e gathers and packs, clear = it reads packed_k
  uint64_t pack_mask;
  // chunk states and counters are indexed by the row's entry in the launch
  // table (not its batch row), so they scale with kMaxSeqPerLaunch only
  float* part_ml;   // [entries][Hq][part_stride][2]
  float* part_o;    // [entries][Hq][part_stride][D]
  int32_t* ticket;  // [entries * Hkv][kTicketStride] chunks finished (element 0), zero between calls;
                    // nullptr: publish plainly for fast_merge_kernel
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

// Final candidate scores with the optional Selector steps: the prior (with
// the key-norm correction), its mixture with the evidence, Soft-NMS within a
// head and exclusivity across heads.  One workgroup scores `chunk` candidate
// positions of one row for all its KV heads.
struct ScoreArgs {
  const float* mass;         // [B][Hkv][T_cap]
  const float* knorm;        // [B][Hkv][T_cap] or nullptr (no key-norm correction)
  const double* knorm_stat;  // [B * Hkv][2]
  const double* zpart;       // [B * Hkv][zpart_stride]
  float* score;              // [B][Hkv][T_cap]: entries [n_sink, T - n_recent) written
  int64_t t_cap;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int32_t zpart_stride;
  int32_t chunk;
  float lambda;
  float knorm_beta;
  float knorm_c;
  int32_t nms_radius;
  float nms_decay;
  float excl;
  SeqTable tab;              // nsplit = chunks per row
};
constexpr int kScoreThreads = 512;
constexpr int kScoreLds = 16384;  // floats of LDS for a workgroup's scores

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

struct PackArgs {
  const void* k;
  const void* v;
  void* packed_k;        // [B][Hkv][top_k][D]
  void* packed_v;
  const int32_t* sel_idx;
  const int32_t* sel_cnt;
  int64_t t_cap;
  int32_t n_kv_heads;
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  SeqTable tab;          // nsplit = row chunks per KV head
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

// Devices the host runtime keeps per-device state for.
constexpr int kMaxDevices = 64;

// Fixed per-device scratch of sfi_fast_step_packed_noalloc: kNoAllocCounters
// fast-step chunk counters (one per 128-byte line) first, then the chunk
// states of one call.  noalloc_scratch returns the calling device's address
// of it, looked up (and its counters cleared on `s`) on the first call on that
// device; it allocates nothing.
constexpr int kNoAllocCounters = 1024;
constexpr size_t kNoAllocCounterBytes = static_cast<size_t>(kNoAllocCounters) * kTicketStride * sizeof(int32_t);
int32_t noalloc_scratch(hipStream_t s, char** out);
int32_t fail(int32_t status, const char* fmt, ...);

// Launchers (defined next to their kernels).  They only enqueue; arguments
// were validated by the caller.  Return the launch's hipError_t.
hipError_t launch_slow_partial(const SlowArgs& a, int dtype, int head_dim, int group,
                               int grid, hipStream_t s);  // a.knorm set: the variant that also emits key norms
hipError_t launch_slow_combine(const CombineArgs& a, int head_dim, int group, int grid,
                               hipStream_t s);
hipError_t launch_select(const SelectArgs& a, int grid, hipStream_t s);
hipError_t launch_score(const ScoreArgs& a, int grid, hipStream_t s);
hipError_t launch_fast_partial(const FastArgs& a, int dtype, int head_dim, int group, int grid,
                               hipStream_t s);
hipError_t launch_fast_merge(const FastArgs& a, int head_dim, int group, hipStream_t s);
hipError_t launch_support(const SupportArgs& a, int grid, hipStream_t s);
hipError_t launch_pack(const PackArgs& a, int dtype, int head_dim, int grid, hipStream_t s);
hipError_t launch_append(const AppendArgs& a, int dtype, int head_dim, int grid,
                         hipStream_t s);
hipError_t launch_fill_zero(void* p, size_t bytes, hipStream_t s);

// Support rows handled by one fast-step workgroup; selected rows copied per
// pack workgroup.
int fast_chunk_rows();
constexpr int kPackRows = 64;

// Kernel timing: while the host runtime times a launch group, launches stamp
// HIP events from their own dispatch packets (the start event on the group's
// first kernel, the stop event on every kernel, so the last one wins).
struct LaunchTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
LaunchTiming* launch_timing();  // the calling thread's context, or nullptr

template <typename Kern, typename... Args>
inline void launch(Kern kern, int grid, int block, hipStream_t s, Args... args) {
  LaunchTiming* t = launch_timing();
  if (t == nullptr) {
    kern<<<grid, block, 0, s>>>(args...);
    return;
  }
  hipExtLaunchKernelGGL(kern, dim3(grid), dim3(block), 0, s, t->start, t->stop, 0, args...);
  t->start = nullptr;
}

// Rows handled per wave per pipeline block: 16 KiB of K (and of V) per block.
__host__ __device__ constexpr int block_rows(int row_bytes) { return 16384 / row_bytes; }

}  // namespace sfi
