/*
 * sfi.h -- C ABI of the MI355X (gfx950) decode-attention path of
 * Slow-Fast Inference (SFI).
 *
 * What the calls compute (pages cited by title and section):
 *
 *  - sfi_slow_step: the slow step, dense attention of each query head over the
 *    whole KV history of its sequence, which also records how much softmax
 *    mass every position received ("Training-Free LLM Inference Acceleration
 *    by Exploiting Attention Stability Within Sentences", section "How SFI
 *    Works: Two Gears for Decoding"; "Slow-Fast Inference: Training-Free
 *    Inference Acceleration via Within-Sentence Support Stability",
 *    gist.science technical summary, 2.A "Das Slow-Fast Paradigma").
 *  - sfi_select: the Selector, which fuses that evidence with a prior as the
 *    mixture s = (1 - lambda) f + lambda r and keeps the top-k positions per
 *    KV head (same summary, 2.B "Der Training-Free Selector").
 *  - sfi_fast_step: the fast step, attention restricted to the sparse state:
 *    sink tokens, the recent window and the selected memory (2.A, items 1-3).
 *  - sfi_kv_append: grows the history by one token per sequence.
 *  - sfi_sched_*: the host-side boundary scheduler that opens every span with
 *    a slow step and can force a refresh after t_max fast steps (2.C
 *    "Trigger-Policy"); span lengths are drawn from splitmix64.
 *
 * Conventions
 *  - Every function returns an sfi_status (0 = SFI_OK, negative = error)
 *    unless stated otherwise.  All arguments are validated before anything is
 *    enqueued: on an error nothing is launched and no output is touched;
 *    sfi_last_error() then holds a message (per calling thread).  The one
 *    exception is SFI_ERR_HIP from a launch after validation passed: kernels
 *    the call enqueued before it stay enqueued, and the outputs of the listed
 *    rows are then unspecified.
 *  - Pointers documented as "device" must point to device memory of the
 *    current HIP device; "host" pointers are read during the call only.
 *    The caller owns every buffer.  The library allocates no device memory.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Work is only
 *    enqueued; nothing synchronises.  Asynchronous device faults surface at
 *    the caller's next synchronisation.
 *  - KV cache layout: K and V are [B][Hkv][T_cap][D] row-major, element type
 *    kv_dtype.  Query head h reads KV head h / (Hq / Hkv).
 *  - Queries q are [B][Hq][D] in kv_dtype.  Outputs are float32.
 *  - Only the batch rows named in seq_ids (host array, distinct values in
 *    [0, B)) are read or written by a call.
 *  - Arrays with a top_k extent (sel_idx, packed_k, packed_v) may be NULL
 *    when top_k = 0.
 *  - Alignment: K, V, q, k_new, v_new, out, mass, packed_k, packed_v and the
 *    workspace start on a 16-byte boundary, the int32 arrays on a 4-byte
 *    one (fresh allocations and whole-row views of them do).  A misaligned
 *    buffer fails validation with SFI_ERR_INVALID_ARG.
 *  - Supported shapes: head_dim 64 or 128; Hq / Hkv in {1, 2, 4, 8};
 *    kv_dtype SFI_F32 or SFI_BF16; 1 <= ctx_len[b] <= kv_capacity <= 2^30;
 *    batch <= 65536; n_kv_heads <= 256.  Support parameters: n_sink and
 *    n_recent <= 2^30, top_k <= 2^24; the fast steps take supports of at
 *    most n_sink + n_recent + top_k <= 512 * R rows, R = 128 rows per
 *    workgroup by default (65536 rows), and fail with SFI_ERR_UNSUPPORTED
 *    beyond.
 *  - Tuning knobs, read from the environment once per process (at the first
 *    call that needs them): SFI_FAST_TILES = 1, 2 or 4 (default 2) sets the
 *    fast steps' rows per wave to 16 times that value (R = 64, 128, 256);
 *    SFI_SLOW_TARGET_WGS (default 1024, at least 64) is the number of
 *    split-K workgroups the slow step aims at (splits keep at least 512
 *    rows, and with mass at most 1024, where the context allows).  Results stay within the same
 *    tolerances for every setting; the defaults measured fastest on MI355X.
 */
#ifndef SFI_H_
#define SFI_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SFI_VERSION_MAJOR 0
#define SFI_VERSION_MINOR 5

typedef enum {
  SFI_OK = 0,
  SFI_ERR_INVALID_ARG = -1, /* null pointer, bad shape, out-of-range id ... */
  SFI_ERR_UNSUPPORTED = -2, /* shape or dtype this build has no kernel for */
  SFI_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  SFI_ERR_HIP = -4,         /* a HIP runtime call or launch failed */
  SFI_ERR_INJECTED = -5,    /* failure forced by SFI_FAULT_INJECT (testing) */
  SFI_ERR_NO_MEMORY = -6    /* a host allocation (the scheduler's state) failed */
} sfi_status;

typedef enum { SFI_F32 = 0, SFI_BF16 = 1 } sfi_dtype;

typedef enum { SFI_OP_SLOW = 0, SFI_OP_SELECT = 1, SFI_OP_FAST = 2, SFI_OP_SLOW_SELECT = 3 } sfi_op;

/* One layer's KV cache and the current context lengths.
 *
 * Context lengths live on the host (ctx_len_host), or on the device
 * (ctx_len, "the growing history" of the decode loop: "Slow-Fast Inference
 * ...", fugumt.com abstract).  With ctx_len == NULL the host values are the
 * lengths and every call reads them when it is made.  With ctx_len set the
 * kernels read each row's length from device memory when they run, so one
 * captured graph serves a history that grows between replays:
 * sfi_kv_append advances ctx_len[b] by one on the device, and the host values
 * are only upper bounds the launches are planned for (grid sizes, splits):
 * every call needs 1 <= ctx_len[b] <= ctx_len_host[b] <= kv_capacity when it
 * runs, and clamps ctx_len[b] into [1, ctx_len_host[b]]. */
typedef struct {
  int32_t batch;               /* B */
  int32_t n_q_heads;           /* Hq */
  int32_t n_kv_heads;          /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;            /* D: 64 or 128 */
  int32_t kv_dtype;            /* sfi_dtype of K, V and q */
  int64_t kv_capacity;         /* T_cap: rows allocated per (b, kv head) */
  void* k;                     /* device [B][Hkv][T_cap][D]; read-only except sfi_kv_append */
  void* v;                     /* device [B][Hkv][T_cap][D]; read-only except sfi_kv_append */
  const int32_t* ctx_len_host; /* host [B]: valid rows of each sequence (T_b), or their bounds */
  float scale;                 /* logit scale; 0 selects 1/sqrt(D) */
  int32_t* ctx_len;            /* device [B] (4-byte aligned) or NULL; see above */
} sfi_kv_desc;

/* The sparse state kept for fast steps: n_sink sink tokens, a recent window
 * of n_recent tokens, and top_k selected tokens chosen by the Selector with
 * mixture weight lambda in [0, 1].  Sinks, window and selected memory are
 * disjoint; top_k counts only the selected memory.
 *
 * Optional Selector steps ("Slow-Fast Inference ...", gist.science
 * technical summary, 2.B: the prior also corrects extreme key norms, and the
 * scores are discretised by Soft-NMS within a head and a soft exclusivity
 * between heads before the top-k).  The page gives no formulas; the readings
 * implemented, all off at 0:
 *  - knorm_beta, knorm_c: each candidate's positional prior weight is
 *    multiplied by exp(-knorm_beta * max(0, z - knorm_c)), z its key norm in
 *    standard deviations above the candidates' mean (population statistics
 *    of the KV head), and the prior is renormalised.  Needs the slow step's
 *    key norms: sfi_slow_step_select / _async only (sfi_select rejects it).
 *  - nms_radius, nms_decay: one parallel round of linear Soft-NMS along the
 *    candidates: a neighbour d <= nms_radius positions away that ranks above
 *    candidate j (higher score, or equal score at a lower position) decays
 *    it to s_j * (1 - nms_decay * (1 - d / (nms_radius + 1))), the nearest
 *    such neighbour's factor applying.
 *  - excl: each KV head's score at a position is multiplied by its share of
 *    the sequence's heads' total score there, to the power excl.
 * Ranges: knorm_beta >= 0, knorm_c finite, 0 <= nms_radius <= 32,
 * 0 <= nms_decay <= 1, excl >= 0, and with any option on
 * n_kv_heads * (64 + 2 * nms_radius) <= 16384.  With an option on the
 * Selector scores the candidates in a pass of its own before the top-k, and
 * sfi_workspace_bytes, given these parameters, includes its buffers. */
typedef struct {
  int32_t n_sink;
  int32_t n_recent;
  int32_t top_k;
  float lambda;
  float knorm_beta;
  float knorm_c;
  int32_t nms_radius;
  float nms_decay;
  float excl;
} sfi_support_params;

/* Bytes of workspace `op` needs for this cache shape (the maximum over all
 * context lengths up to kv_capacity and all batch rows).  `sp` may be NULL
 * for SFI_OP_SLOW.  Returns 0 and sets sfi_last_error() on invalid input. */
size_t sfi_workspace_bytes(const sfi_kv_desc* desc, const sfi_support_params* sp, int32_t op);

/* Zero-fills a workspace (device, ws_bytes).  Call it once on a new
 * workspace before its first fast step: the fast step counts finished support
 * chunks per (sequence, KV head) in the workspace, needs those counters at
 * zero and leaves them at zero.  Every other part is prepared by the call
 * that uses it (the Selector's per-head histogram and list counter are
 * cleared by the first kernel of each call that builds them).  Workspaces
 * must not be shared by calls that may run concurrently. */
int32_t sfi_workspace_init(void* ws, size_t ws_bytes, void* stream);

/* Slow step (dense decode attention over the whole history).
 *   q    : device [B][Hq][D], kv_dtype
 *   out  : device float32 [B][Hq][D]; out[b][h] = sum_j p_hj v_j with
 *          p_h = softmax_j(scale * q_h . k_j) over j < ctx_len[b]
 *   mass : device float32 [B][Hkv][T_cap] or NULL.  When non-NULL, row
 *          [b][g][j] for j < ctx_len[b] receives the softmax mass of position
 *          j averaged over the query heads of KV head g (each row sums to 1);
 *          the Selector's evidence.  Entries j >= ctx_len[b] are not written.
 *   ws   : device workspace of at least sfi_workspace_bytes(desc, NULL, SFI_OP_SLOW). */
int32_t sfi_slow_step(const sfi_kv_desc* desc, const int32_t* seq_ids_host, int32_t n_seq,
                      const void* q, float* out, float* mass, void* ws, size_t ws_bytes,
                      void* stream);

/* Launch plan of sfi_slow_step / sfi_slow_step_select for these rows: writes
 * to splits_host[i] (host int32 [n_seq]) how many split-K partials the slow
 * step forms for each of the KV heads of sequence seq_ids_host[i], which sets
 * how much partial state its merge reads.  with_mass != 0 plans a step that
 * writes mass (sfi_slow_step with mass, sfi_slow_step_select), whose splits
 * may be shorter; 0 plans the dense-only step.  Launches nothing. */
int32_t sfi_slow_plan(const sfi_kv_desc* desc, const int32_t* seq_ids_host, int32_t n_seq,
                      int32_t with_mass, int32_t* splits_host);

/* Launch plan of sfi_fast_step / sfi_fast_step_packed for these rows: writes
 * to chunks_host[i] (host int32 [n_seq]) how many partials (one per chunk of
 * support rows) the fast step forms for each KV head of sequence
 * seq_ids_host[i] and its merge then reads.  Launches nothing. */
int32_t sfi_fast_plan(const sfi_kv_desc* desc, const sfi_support_params* sp,
                      const int32_t* seq_ids_host, int32_t n_seq, int32_t* chunks_host);

/* Selector.  For each listed sequence b (context T = ctx_len[b]) and KV head
 * g: candidates are positions [n_sink, T - n_recent) (n of them); candidate
 * at 1-based offset a from the sinks gets the prior
 *   r = (1/a + 1/(n + 1 - a)) / (2 H_n),   H_n = 1 + 1/2 + ... + 1/n,
 * and the score s = (1 - lambda) * mass[b][g][j] + lambda * r, computed in
 * float32.  The min(top_k, n) highest scores are kept, ties going to the
 * lower position.
 *   mass    : device float32 [B][Hkv][T_cap] (as written by sfi_slow_step)
 *   sel_idx : device int32 [B][Hkv][top_k]; the kept positions in ascending
 *             order, then -1 up to top_k
 *   sel_cnt : device int32 [B][Hkv]; min(top_k, n) (0 when T <= n_sink + n_recent)
 *   ws      : at least sfi_workspace_bytes(desc, sp, SFI_OP_SELECT) bytes. */
int32_t sfi_select(const sfi_kv_desc* desc, const sfi_support_params* sp,
                   const int32_t* seq_ids_host, int32_t n_seq, const float* mass,
                   int32_t* sel_idx, int32_t* sel_cnt, void* ws, size_t ws_bytes, void* stream);

/* Fast step (attention over the sparse state).  For sequence b at context
 * length t = ctx_len[b], KV head g attends to
 *   [0, min(n_sink, t))  u  [max(n_sink, t - n_recent), t)  u  sel_idx[b][g][0 : sel_cnt[b][g]]
 * with the softmax renormalised over that support.
 *   q, out           : as for sfi_slow_step
 *   sel_idx, sel_cnt : device, as written by sfi_select.  Entries outside
 *                      [0, t) and counts above min(top_k, n) are ignored.
 *   ws               : at least sfi_workspace_bytes(desc, sp, SFI_OP_FAST) bytes.
 * An empty support (possible only with n_sink = n_recent = 0 and a zero count)
 * yields a zero output. */
int32_t sfi_fast_step(const sfi_kv_desc* desc, const sfi_support_params* sp,
                      const int32_t* seq_ids_host, int32_t n_seq, const void* q,
                      const int32_t* sel_idx, const int32_t* sel_cnt, float* out, void* ws,
                      size_t ws_bytes, void* stream);

/* Memory-coalesced layout of the selected memory ("Slow-Fast Inference ...",
 * gist.science technical summary, 3 "Systemdesign und Kernel-Optimierung":
 * after each slow step the selected tokens are packed into a contiguous
 * buffer, while sinks and the recent window are read from the cache).
 *
 * sfi_pack_support copies, for each listed (b, g), the rows
 * K[b][g][sel_idx[b][g][i]] and V[...] for i < sel_cnt[b][g] into
 * packed_k[b][g][i] and packed_v[b][g][i] (device [B][Hkv][top_k][D],
 * kv_dtype).  Indices outside [0, ctx_len[b]) are skipped: their slots keep
 * whatever they held.  The Selector never emits such an index; a caller that
 * passes its own sel_idx must keep every index below sel_cnt inside the
 * context, because sfi_fast_step_packed attends to every slot below sel_cnt
 * (a skipped slot's stale row included) while sfi_fast_step ignores an
 * out-of-range index. */
int32_t sfi_pack_support(const sfi_kv_desc* desc, const sfi_support_params* sp,
                         const int32_t* seq_ids_host, int32_t n_seq, const int32_t* sel_idx,
                         const int32_t* sel_cnt, void* packed_k, void* packed_v, void* stream);

/* sfi_fast_step that also packs: besides the output it writes the selected
 * rows it reads, K[b][g][sel_idx[b][g][i]] and V[...] for i below the count
 * the fast step uses (min(sel_cnt, the current candidate count)), into
 * packed_k[b][g][i] and packed_v[b][g][i] (device [B][Hkv][top_k][D],
 * kv_dtype; indices outside the context are skipped, as sfi_pack_support skips
 * them).  The output is sfi_fast_step's, bit for bit, and the packed rows are
 * sfi_pack_support's: the first fast step of a span can pack the support for
 * the sfi_fast_step_packed calls that follow, instead of the refresh packing
 * it (the memory-coalesced layout of "Slow-Fast Inference ...", gist.science
 * technical summary, 3 "Systemdesign und Kernel-Optimierung", made on the
 * first read of the selected rows).
 *   pack_flags : host, n_seq entries, or NULL (every row packs).  Row
 *                seq_ids[i] packs when pack_flags[i] != 0; a row whose flag is
 *                0 is computed as by sfi_fast_step_packed from the packed rows
 *                an earlier call wrote (its buffers are only read), so one
 *                launch serves a batch whose rows are at different points of
 *                their spans.
 * Other arguments and the workspace as for sfi_fast_step; packed_k /
 * packed_v may be NULL only when top_k = 0. */
int32_t sfi_fast_step_pack(const sfi_kv_desc* desc, const sfi_support_params* sp, const int32_t* seq_ids_host,
                           int32_t n_seq, const int32_t* pack_flags, const void* q, const int32_t* sel_idx,
                           const int32_t* sel_cnt, float* out, void* packed_k, void* packed_v, void* ws,
                           size_t ws_bytes, void* stream);

/* Fast step over a packed support: the same result as sfi_fast_step with the
 * sel_idx that filled packed_k / packed_v, provided every index below sel_cnt
 * lay inside the context when it was packed (always so for the Selector's
 * output); the selected rows are read contiguously from the packed buffers
 * (no index lookups).  Slots at or past min(sel_cnt, the current candidate
 * count) are never attended, whatever they hold. */
int32_t sfi_fast_step_packed(const sfi_kv_desc* desc, const sfi_support_params* sp,
                             const int32_t* seq_ids_host, int32_t n_seq, const void* q,
                             const void* packed_k, const void* packed_v, const int32_t* sel_cnt,
                             float* out, void* ws, size_t ws_bytes, void* stream);

/* sfi_fast_step_packed without a workspace, for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, harnesses
 * that forbid allocation.  It launches the same kernels with the same launch
 * shape (so it writes the same bits) and allocates nothing: its chunk states
 * and per-head counters live in a fixed scratch array of the library,
 * SFI_NOALLOC_SCRATCH_BYTES on every GPU it runs on, held until the process
 * ends.  Its address is looked up on the first call on each device; that
 * call also enqueues a small kernel on `stream` that zeroes the counters.
 * Every call on a GPU shares that GPU's array: calls that may overlap in time
 * on one GPU (other streams, other threads) race and must not be issued.
 * Limits (SFI_ERR_UNSUPPORTED before anything is enqueued): n_seq <= 64,
 * n_seq * n_kv_heads <= 1024, and n_seq * n_q_heads * chunks * (head_dim + 2)
 * * 4 bytes of chunk states (chunks: ceil((n_sink + n_recent + top_k) / 128),
 * the fast step's largest plan) within the array after its 128 KiB of
 * counters. */
#define SFI_NOALLOC_SCRATCH_BYTES (16u << 20)
int32_t sfi_fast_step_packed_noalloc(const sfi_kv_desc* desc, const sfi_support_params* sp,
                                     const int32_t* seq_ids_host, int32_t n_seq, const void* q,
                                     const void* packed_k, const void* packed_v,
                                     const int32_t* sel_cnt, float* out, void* stream);

/* The slow step and the Selector in one call, with the selected rows packed
 * as they are chosen: the whole refresh that opens a span ("Slow-Fast
 * Inference ...", gist.science technical summary, 2.A and 2.B; packing: 3
 * "Systemdesign und Kernel-Optimierung").  Writes exactly what
 *   sfi_slow_step(q, out, mass); sfi_select(mass, sel_idx, sel_cnt);
 *   sfi_pack_support(sel_idx, sel_cnt, packed_k, packed_v)
 * would, bit for bit, in fewer kernels: the merge that produces the mass also
 * builds the Selector's first radix histogram, and the pass that emits the
 * kept positions also copies their K/V rows.
 *   q, out, mass     : as for sfi_slow_step; mass must not be NULL
 *   sel_idx, sel_cnt : as for sfi_select
 *   packed_k/_v      : as for sfi_pack_support, or both NULL to skip packing
 *   ws               : at least sfi_workspace_bytes(desc, sp, SFI_OP_SLOW_SELECT)
 *                      bytes. */
int32_t sfi_slow_step_select(const sfi_kv_desc* desc, const sfi_support_params* sp,
                             const int32_t* seq_ids_host, int32_t n_seq, const void* q, float* out,
                             float* mass, int32_t* sel_idx, int32_t* sel_cnt, void* packed_k,
                             void* packed_v, void* ws, size_t ws_bytes, void* stream);

/* sfi_slow_step_select with the Selector's kernels (and the packing) on a
 * second stream, so that they overlap with whatever the caller enqueues on
 * `stream` next, typically the next layer's attention: the pages' pipeline
 * runs a layer's Selector and cache reorganisation asynchronously with the
 * following layer ("Slow-Fast Inference ...", gist.science technical
 * summary, 3 "Systemdesign und Kernel-Optimierung").  Results are those of
 * sfi_slow_step_select, bit for bit.
 *   stream        : runs the slow step; `out` is ready in its order
 *   select_stream : waits for the slow step, then runs the Selector; mass,
 *                   sel_idx, sel_cnt and packed_k/v are ready in its order.
 * mass, the output arrays and ws stay in use until select_stream reaches
 * that point: the caller orders any later use of them (a fast step, another
 * call on the same ws or mass) after it, e.g. with an event.  Two layers in
 * flight need two workspaces and two mass buffers.  With more than 64 rows
 * the calls' launch groups run one after another through the same two
 * streams.  Given the same stream twice it behaves as sfi_slow_step_select. */
int32_t sfi_slow_step_select_async(const sfi_kv_desc* desc, const sfi_support_params* sp,
                                   const int32_t* seq_ids_host, int32_t n_seq, const void* q,
                                   float* out, float* mass, int32_t* sel_idx, int32_t* sel_cnt,
                                   void* packed_k, void* packed_v, void* ws, size_t ws_bytes,
                                   void* stream, void* select_stream);

/* Appends one token per listed sequence: writes k_new[b][g][:] and
 * v_new[b][g][:] (device [B][Hkv][D], kv_dtype) into row T_b of desc->k and
 * desc->v, T_b the sequence's context length.
 *  - host lengths (desc->ctx_len == NULL): requires ctx_len_host[b] <
 *    kv_capacity; the caller then increments its ctx_len_host[b].
 *  - device lengths: T_b = desc->ctx_len[b], read when the kernel runs, and
 *    the kernel then sets desc->ctx_len[b] = T_b + 1; a row with T_b >=
 *    kv_capacity is left unchanged. */
int32_t sfi_kv_append(const sfi_kv_desc* desc, const int32_t* seq_ids_host, int32_t n_seq,
                      const void* k_new, const void* v_new, void* stream);

/* Debug: writes the positions the fast-step kernel enumerates for each
 * listed (b, g), in its own order, into support_out (device int32
 * [B][Hkv][cap_per_head]), and their count into support_cnt (device int32
 * [B][Hkv]).  Uses the same device index function as sfi_fast_step. */
int32_t sfi_debug_support(const sfi_kv_desc* desc, const sfi_support_params* sp,
                          const int32_t* seq_ids_host, int32_t n_seq, const int32_t* sel_idx,
                          const int32_t* sel_cnt, int32_t* support_out, int32_t* support_cnt,
                          int32_t cap_per_head, void* stream);

/* ---- host-side boundary scheduler (no device work) -------------------- */
typedef struct sfi_sched sfi_sched;
typedef enum { SFI_SPAN_FIXED = 0, SFI_SPAN_GEOMETRIC = 1 } sfi_span_mode;

/* batch sequences; sequence b draws from splitmix64 started at seed + b.
 * FIXED: every span has span_param steps (a positive integer).
 * GEOMETRIC: span length = index of the first draw x < floor(2^64 / span_param),
 * span_param in [1, 2^52).  t_max > 0 forces a slow step after t_max
 * consecutive fast steps (0 = off). */
int32_t sfi_sched_create(int32_t batch, uint64_t seed, int32_t mode, double span_param,
                         int32_t t_max, sfi_sched** out);
/* Advances every sequence by one decode step.  slow_ids / fast_ids (host,
 * capacity batch each) receive the sequence ids, in increasing order. */
int32_t sfi_sched_step(sfi_sched* s, int32_t* slow_ids, int32_t* n_slow, int32_t* fast_ids,
                       int32_t* n_fast);
/* The next step of sequence `seq` will be slow (e.g. after a failed select). */
int32_t sfi_sched_force_slow(sfi_sched* s, int32_t seq);
void sfi_sched_destroy(sfi_sched* s);

/* ---- errors, version, kernel timing ------------------------------------ */
const char* sfi_status_str(int32_t status);
const char* sfi_last_error(void);
int32_t sfi_version(void); /* MAJOR * 100 + MINOR */

/* Kernel timing with HIP events recorded on the launch stream around each
 * launch of the named kernel (off by default).  sfi_profile_read waits for
 * the recorded events and returns the summed milliseconds and launch count
 * since the last reset. */
typedef enum {
  SFI_K_SLOW_PARTIAL = 0, /* split-K dense partials (+ logit scratch) */
  SFI_K_SLOW_COMBINE = 1, /* split merge + per-position mass */
  SFI_K_SELECT = 2,       /* Selector (all of its kernels of one call together) */
  SFI_K_FAST = 3,         /* the fast step: sparse attention over support chunks (gather
                             or packed); a launch that fits the GPU in one pass also
                             merges the chunks in the same kernel */
  SFI_K_APPEND = 4,
  SFI_K_PACK = 5,         /* packing of the selected rows */
  SFI_K_FAST_MERGE = 6,   /* merge of the fast step's chunk states, for launches with more
                             workgroups than the GPU has compute units */
  SFI_K_FAST_PACK = 7,    /* a fast-step launch of sfi_fast_step_pack in which some row packs */
  SFI_K_COUNT = 8
} sfi_kernel_id;
int32_t sfi_profile_enable(int32_t on);
int32_t sfi_profile_reset(void);
int32_t sfi_profile_read(int32_t kernel, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* SFI_H_ */
