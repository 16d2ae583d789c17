/* A plain C (C99) client of the library's C ABI: includes include/sfi.h,
 * links libsfi.so and exercises calls that need no GPU (version, status
 * strings, validation errors, workspace sizing, the span scheduler).  It
 * prints the first scheduler steps so the test can compare them with the
 * oracle's schedule. */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "sfi.h"

static int fails = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      fprintf(stderr, "line %d: check failed: %s\n", __LINE__, #cond); \
      ++fails;                                                        \
    }                                                                 \
  } while (0)

int main(void) {
  EXPECT(sfi_version() == SFI_VERSION_MAJOR * 100 + SFI_VERSION_MINOR);
  EXPECT(strlen(sfi_status_str(SFI_ERR_WORKSPACE)) > 0);

  /* validation errors leave a message and launch nothing */
  int32_t ctx[2] = {100, 50};
  int32_t ids[2] = {0, 1};
  sfi_kv_desc d;
  memset(&d, 0, sizeof d);
  d.batch = 2;
  d.n_q_heads = 8;
  d.n_kv_heads = 2;
  d.head_dim = 64;
  d.kv_dtype = SFI_BF16;
  d.kv_capacity = 100;
  d.k = (void*)0x10000;
  d.v = (void*)0x20000;
  d.ctx_len_host = ctx;
  EXPECT(sfi_slow_step(NULL, ids, 2, NULL, NULL, NULL, NULL, 0, NULL) == SFI_ERR_INVALID_ARG);
  EXPECT(strlen(sfi_last_error()) > 0);
  d.head_dim = 96;
  EXPECT(sfi_slow_step(&d, ids, 2, (void*)0x30000, (float*)0x40000, NULL, (void*)0x50000, (size_t)1 << 40,
                       NULL) == SFI_ERR_UNSUPPORTED);
  d.head_dim = 64;
  sfi_support_params sp = {.n_sink = 4, .n_recent = 16, .top_k = 32, .lambda = 0.1f};
  size_t need = sfi_workspace_bytes(&d, &sp, SFI_OP_SLOW_SELECT);
  EXPECT(need > 0);
  /* the optional Selector steps: their scores need more workspace; an out-of-range radius fails */
  sfi_support_params opt = sp;
  opt.nms_radius = 2;
  opt.nms_decay = 0.5f;
  opt.excl = 1.0f;
  EXPECT(sfi_workspace_bytes(&d, &opt, SFI_OP_SLOW_SELECT) > need);
  opt.nms_radius = 40;
  EXPECT(sfi_workspace_bytes(&d, &opt, SFI_OP_SLOW_SELECT) == 0 && strstr(sfi_last_error(), "nms_radius") != NULL);
  EXPECT(sfi_slow_step_select(&d, &sp, ids, 2, (void*)0x30000, (float*)0x40000, (float*)0x60000,
                              (int32_t*)0x70000, (int32_t*)0x80000, NULL, NULL, (void*)0x50000, need - 1,
                              NULL) == SFI_ERR_WORKSPACE);
  int32_t splits[2] = {0, 0};
  EXPECT(sfi_slow_plan(&d, ids, 2, 1, splits) == SFI_OK && splits[0] >= 1 && splits[1] >= 1);
  /* the packing fast step: its packed buffers are required, and its workspace is the fast step's */
  int32_t flags[2] = {1, 0};
  size_t need_fast = sfi_workspace_bytes(&d, &sp, SFI_OP_FAST);
  EXPECT(need_fast > 0);
  EXPECT(sfi_fast_step_pack(&d, &sp, ids, 2, flags, (void*)0x30000, (int32_t*)0x70000, (int32_t*)0x80000,
                            (float*)0x40000, NULL, NULL, (void*)0x50000, need_fast, NULL) == SFI_ERR_INVALID_ARG);
  EXPECT(strstr(sfi_last_error(), "packed") != NULL);
  EXPECT(sfi_fast_step_pack(&d, &sp, ids, 2, flags, (void*)0x30000, (int32_t*)0x70000, (int32_t*)0x80000,
                            (float*)0x40000, (void*)0x90000, (void*)0xA0000, (void*)0x50000, need_fast - 1,
                            NULL) == SFI_ERR_WORKSPACE);

  /* the scheduler: geometric spans of mean 18 for 3 sequences, seed 7 */
  sfi_sched* s = NULL;
  EXPECT(sfi_sched_create(3, 7u, SFI_SPAN_GEOMETRIC, 18.0, 0, &s) == SFI_OK && s != NULL);
  if (s != NULL) {
    int32_t slow[3], fast[3], ns = 0, nf = 0;
    for (int t = 0; t < 64; ++t) {
      EXPECT(sfi_sched_step(s, slow, &ns, fast, &nf) == SFI_OK && ns + nf == 3);
      printf("step %d slow", t);
      for (int i = 0; i < ns; ++i) printf(" %d", slow[i]);
      printf("\n");
    }
    sfi_sched_destroy(s);
  }
  if (fails == 0) printf("c client ok\n");
  return fails == 0 ? 0 : 1;
}
