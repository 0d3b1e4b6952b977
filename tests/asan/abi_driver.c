/*
 * Host-side checks of the C ABI, built with AddressSanitizer and
 * UndefinedBehaviorSanitizer over the ABI layer (api.cpp).  Every call below
 * must be decided on the host: argument and shape rejections, workspace
 * queries, the no-allocation limit, status strings and empty inputs that
 * launch nothing.  Device pointers are fakes that are never dereferenced, so
 * no GPU is needed.  Exit status = number of failed checks.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "kvs.h"

static int failures = 0;
#define CHECK(expr, want)                                                              \
  do {                                                                                 \
    long long got_ = (long long)(expr);                                                \
    if (got_ != (long long)(want)) {                                                   \
      fprintf(stderr, "%s:%d: %s = %lld, want %lld\n", __FILE__, __LINE__, #expr, got_, \
              (long long)(want));                                                      \
      ++failures;                                                                      \
    }                                                                                  \
  } while (0)

int main(void) {
  void* F = (void*)(uintptr_t)0x1000;   /* 16-byte aligned fake device pointer */
  const double inf = INFINITY;

  /* status strings, including an unknown code */
  for (int s = -1; s <= 8; ++s) CHECK(kvs_status_string(s) != NULL, 1);
  CHECK(strcmp(kvs_status_string(KVS_OK), "ok"), 0);
  CHECK(kvs_version() >= 100, 1);

  /* QueryMemory */
  CHECK(kvs_qmem_update(NULL, KVS_BF16, 2, 4, 8, 128, 0.5f, 1, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_qmem_update(F, 7, 2, 4, 8, 128, 0.5f, 1, F, NULL), KVS_ERR_DTYPE);
  CHECK(kvs_qmem_update(F, KVS_BF16, 2, 4, 0, 128, 0.5f, 1, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_qmem_update(F, KVS_BF16, 2, 4, 8, 128, -1.0f, 1, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_qmem_update(F, KVS_BF16, 2, 4, 8, 128, NAN, 1, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_qmem_update(F, KVS_BF16, 2, 4, 8, 96, 0.5f, 1, F, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_qmem_update(F, KVS_BF16, 1 << 30, 1 << 30, 1 << 30, 128, 0.5f, 1, F, NULL), KVS_ERR_SHAPE);

  /* rule score, dense and paged */
  size_t ws = kvs_rule_score_workspace(2, 4, 2, 1024);
  CHECK(ws >= 2 * 4 * 1024 * 4, 1);
  CHECK(kvs_rule_score_workspace(0, 4, 2, 1024), 0);
  CHECK(kvs_rule_score(NULL, 1, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_ARG);
  CHECK(kvs_rule_score(F, 5, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_DTYPE);
  CHECK(kvs_rule_score(F, 1, F, 2, 5, 2, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_rule_score(F, 1, F, 2, 4, 2, 128, 1024, 16, 10, 5, F, F, ws, NULL), KVS_ERR_ARG);
  CHECK(kvs_rule_score(F, 1, F, 2, 4, 2, 80, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_rule_score(F, 1, F, 2, 34, 2, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_rule_score(F, 1, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, NULL, ws, NULL), KVS_ERR_WORKSPACE);
  CHECK(kvs_rule_score(F, 1, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, F, ws - 1, NULL), KVS_ERR_WORKSPACE);
  CHECK(kvs_rule_score(F, 1, F, 2, 4, 2, 128, (int64_t)1 << 31, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_rule_score(F, 1, F, 2, 4, 2, 128, 0, 16, 992, 1024, F, F, ws, NULL), KVS_OK);   /* nothing launched */
  CHECK(kvs_rule_score(NULL, 1, F, 2, 4, 2, 128, 0, 16, 992, 1024, NULL, F, ws, NULL), KVS_OK); /* empty K, rule */
  CHECK(kvs_rule_score(F, 1, NULL, 2, 4, 2, 128, 0, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_ARG); /* M never empty */
  CHECK(kvs_meank_score(NULL, NULL, 2, 8, 2, 128, 0, 0, 4, 7, NULL, NULL, 0, NULL), KVS_OK);  /* nB = 0 */
  CHECK(kvs_meank_score(NULL, F, 2, 8, 2, 128, 5, 300, 4, 7, F, F, 1 << 20, NULL), KVS_ERR_ARG);
  CHECK(kvs_rule_score_paged(F, 1, NULL, 2048, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_ARG);
  CHECK(kvs_rule_score_paged(F, 1, F, 0, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_ARG);
  CHECK(kvs_rule_score_paged(F, 1, F, 2048, F, 2, 4, 3, 128, 1024, 16, 992, 1024, F, F, ws, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_rule_score_paged(F, 1, F, 2048, F, 2, 4, 2, 128, 1024, 16, 992, 1024, F, F, ws - 1, NULL),
        KVS_ERR_WORKSPACE);

  /* window score */
  size_t wws = kvs_window_score_workspace(2, 8, 2, 16, 1000);
  CHECK(wws > 0, 1);
  CHECK(kvs_window_score(F, F, 2, 8, 2, 128, 1000, 0, 4, 990, 1000, F, F, wws, NULL), KVS_ERR_ARG);
  CHECK(kvs_window_score(F, F, 2, 8, 3, 128, 1000, 16, 4, 990, 1000, F, F, wws, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_window_score(F, F, 2, 8, 2, 128, 1000, 16, 4, 990, 1000, F, F, wws - 1, NULL), KVS_ERR_WORKSPACE);
  CHECK(kvs_window_score(F, F, 2, 8, 2, 96, 1000, 16, 4, 990, 1000, F, F, wws, NULL), KVS_ERR_UNSUPPORTED);

  /* top-k, with and without a workspace, and the no-allocation variant */
  CHECK(kvs_topk_workspace(32768), 0);
  size_t tws = kvs_topk_workspace(92160);
  CHECK(tws >= 4 * (256 + 2 * 45), 1);
  CHECK(kvs_topk_select(NULL, 10, 0, 1, 5, 6, 3, F, F, F, NULL, 0, NULL), KVS_ERR_ARG);
  CHECK(kvs_topk_select(F, 10, 3, 1, 5, 6, 3, F, F, F, NULL, 0, NULL), KVS_ERR_ARG);
  CHECK(kvs_topk_select(F, 10, 0, 1, 5, 6, -1, F, F, F, NULL, 0, NULL), KVS_ERR_ARG);
  CHECK(kvs_topk_select(F, (int64_t)1 << 31, 0, 1, 5, 6, 3, F, F, F, NULL, 0, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_topk_select(F, 92160, 0, 64, 92096, 92160, 8192, F, F, F, F, tws - 1, NULL), KVS_ERR_WORKSPACE);
  const int64_t nmax = kvs_topk_noalloc_max();
  CHECK(nmax, (int64_t)1 << 24);
  CHECK(kvs_topk_select_noalloc(F, nmax + 1, 0, 64, 0, 0, 8192, F, F, F, NULL), KVS_ERR_LIMIT);
  CHECK(kvs_topk_select_noalloc(NULL, 10, 0, 1, 5, 6, 3, F, F, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_topk_select_noalloc(F, 10, 0, 1, 5, 6, 3, F, F, NULL, NULL), KVS_ERR_ARG);

  /* slot redirect */
  CHECK(kvs_slotmap_redirect(NULL, F, 10, -1, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_slotmap_redirect(F, F, -1, -1, F, NULL), KVS_ERR_ARG);

  /* Mean-K build and append */
  CHECK(kvs_meank_build(F, 2, 2, 128, 64, 16, 0, 0, 1e6, NULL, F, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_meank_build(F, 2, 2, 128, 64, 32, 1, 0, inf, NULL, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_meank_build(F, 2, 2, 128, 64, 32, 1, -5, 1e6, NULL, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_meank_build(NULL, 2, 2, 128, 64, 32, 0, 0, 1e6, NULL, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_meank_append(F, 2, 2, 128, 40, 30, 0, 1e6, F, 64, F, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_meank_append(F, 2, 2, 128, -1, 30, 0, 1e6, F, 64, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_meank_append(F, 2, 2, 128, 0, 30, 0, 0.0, F, 64, F, NULL), KVS_ERR_ARG);
  CHECK(kvs_meank_append(F, 2, 2, 96, 0, 30, 0, 1e6, F, 64, F, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_meank_append(NULL, 2, 2, 128, 10, 0, 0, 1e6, NULL, 64, NULL, NULL), KVS_OK);   /* empty chunk */

  /* R_b */
  size_t mws = kvs_meank_score_workspace(2, 8, 2, 50, 300);
  CHECK(mws > 0, 1);
  CHECK(kvs_meank_score_workspace(2, 8, 3, 50, 300), 0);
  CHECK(kvs_meank_score(F, F, 2, 8, 3, 128, 50, 300, 4, 7, F, F, mws, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_meank_score(F, F, 2, 8, 2, 128, 50, 300, 4, 7, F, F, mws - 1, NULL), KVS_ERR_WORKSPACE);
  CHECK(kvs_meank_score(F, F, 2, 8, 2, 128, 50, 300, -1, 7, F, F, mws, NULL), KVS_ERR_ARG);
  CHECK(kvs_meank_score(F, F, 2, 8, 2, 96, 50, 300, 4, 7, F, F, mws, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_meank_score(F, F, 4, 8, 2, 128, 50, ((int64_t)1 << 31) - 1, 4, 7, F, F, (size_t)1 << 30, NULL),
        KVS_ERR_SHAPE);

  /* re-RoPE scatter */
  CHECK(kvs_rerope_scatter(F, F, 640, F, NULL, 3, 2, 2, 128, 32, 0, 1e6, F, NULL, 8, NULL, NULL), KVS_ERR_ARG);
  CHECK(kvs_rerope_scatter(F, F, 650, F, NULL, 3, 2, 2, 128, 32, 0, 1e6, F, F, 8, NULL, NULL), KVS_ERR_SHAPE);
  CHECK(kvs_rerope_scatter(F, F, 640, F, NULL, 3, 2, 2, 128, 64, 0, 1e6, F, F, 8, NULL, NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_rerope_scatter(F, F, 640, F, NULL, 3, 2, 2, 128, 32, 0, -1.0, F, F, 8, NULL, NULL), KVS_ERR_ARG);
  CHECK(kvs_rerope_scatter(F, NULL, 640, F, NULL, (int64_t)1 << 24, 2, 2, 128, 32, 0, 1e6, F, NULL, 8, NULL, NULL),
        KVS_ERR_SHAPE);

  /* working-set update */
  size_t sws = kvs_working_set_workspace(8);
  CHECK(sws >= 8 * 4, 1);
  CHECK(kvs_working_set_update(F, F, 640, F, F, 3, F, 9, 2, 2, 128, 32, 0, 1e6, F, F, 8, F, F, F, F, NULL, F, sws,
                               NULL), KVS_ERR_SHAPE);
  CHECK(kvs_working_set_update(F, F, 640, F, F, 3, F, 4, 2, 2, 128, 16, 0, 1e6, F, F, 8, F, F, F, F, NULL, F, sws,
                               NULL), KVS_ERR_UNSUPPORTED);
  CHECK(kvs_working_set_update(F, NULL, 640, F, F, 3, F, 4, 2, 2, 128, 32, 0, 1e6, F, F, 8, F, F, F, F, NULL, F,
                               sws, NULL), KVS_ERR_ARG);
  CHECK(kvs_working_set_update(F, F, 640, F, F, 3, F, 4, 2, 2, 128, 32, 0, 1e6, F, F, 8, F, F, F, F, NULL, F,
                               sws - 1, NULL), KVS_ERR_WORKSPACE);

  printf("abi_driver: %d failed checks\n", failures);
  return failures;
}
