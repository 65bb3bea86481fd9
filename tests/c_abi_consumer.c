/* A plain C99 consumer of include/stem.h, linked against libstem.so: it exercises the host-only entry
 * points and the host-side validation of the stage entry points (no device is touched), so that the
 * boundary is shown to be usable from C with no Python or C++ in between.  Exit status 0 = all checks
 * passed; the first failing check is printed. */
#include <stdio.h>
#include <string.h>

#include "stem.h"

static int failures = 0;
#define CHECK(cond)                                                      \
  do {                                                                   \
    if (!(cond)) {                                                       \
      printf("check failed (line %d): %s\n", __LINE__, #cond);           \
      failures++;                                                        \
    }                                                                    \
  } while (0)

int main(void) {
  /* two requests of 300 and 129 tokens, 8 query / 2 KV heads, d = 128, block 128, bf16 */
  const int32_t cu[3] = {0, 300, 429};
  stem_problem p;
  memset(&p, 0, sizeof(p));
  p.num_reqs = 2;
  p.cu_seqlens = cu;
  p.hq = 8;
  p.hkv = 2;
  p.head_dim = 128;
  p.block = 128;
  p.dtype = STEM_BF16;

  int64_t nb = 0;
  int32_t max_n = 0;
  CHECK(stem_block_counts(&p, &nb, &max_n) == STEM_OK);
  CHECK(nb == 3 + 2 && max_n == 3);

  size_t oq = 0, ok = 0, om = 0;
  const size_t ws = stem_workspace_bytes(&p);
  CHECK(ws > 0);
  CHECK(stem_workspace_layout(&p, &oq, &ok, &om) == STEM_OK);
  CHECK(oq % 256 == 0 && ok % 256 == 0 && om % 256 == 0);
  CHECK(ok >= oq + (size_t)8 * 5 * 128 * sizeof(float));
  CHECK(om >= ok + (size_t)2 * 5 * 128 * sizeof(float));
  CHECK(ws >= om + (size_t)2 * 5 * sizeof(float));

  /* TPD budgets at n = 1024, 25%, mu = 7/10: total 131200, rows 0..157 dense, last row 116 */
  static int32_t k[1024];
  CHECK(stem_tpd_budgets_host(1024, 25, 100, 7, 10, k) == STEM_OK);
  long long total = 0;
  int bounded = 1;
  for (int i = 0; i < 1024; ++i) {
    total += k[i];
    if (k[i] < 1 || k[i] > i + 1) bounded = 0;
  }
  CHECK(total == 131200);
  CHECK(bounded);
  CHECK(k[0] == 1 && k[157] == 158 && k[1023] == 116);

  /* validation happens on the host, before any device call */
  CHECK(stem_tpd_budgets_host(0, 25, 100, 7, 10, k) == STEM_E_INVALID_ARG);
  CHECK(strlen(stem_last_error()) > 0);
  CHECK(stem_tpd_budgets_host(8, 25, 100, 7, 10, k) == STEM_OK);
  CHECK(strlen(stem_last_error()) == 0); /* a successful call clears the message */

  float scores[16];
  CHECK(stem_score(&p, NULL, NULL, NULL, 0.2f, scores, 3, NULL, 0, NULL) == STEM_E_INVALID_ARG);
  stem_problem bad = p;
  bad.head_dim = 96;
  CHECK(stem_block_counts(&bad, &nb, &max_n) == STEM_E_UNSUPPORTED);
  bad = p;
  bad.hkv = 3;
  CHECK(stem_block_counts(&bad, &nb, &max_n) == STEM_E_INVALID_ARG);
  CHECK(bsa_prefill(&bad, scores, scores, scores, NULL, 0, 0.f, scores, NULL, NULL) == STEM_E_INVALID_ARG);

  CHECK(strcmp(stem_status_string(STEM_E_HIP), "STEM_E_HIP") == 0);
  CHECK(strcmp(stem_status_string(STEM_OK), "STEM_OK") == 0);

  if (failures == 0) printf("c consumer ok\n");
  return failures == 0 ? 0 : 1;
}
