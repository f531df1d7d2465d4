/*
 * A plain C11 client of libcpa, built by tests/test_c_client.py with gcc
 * against include/cpa.h: the header has to compile as C and the host entry
 * points have to work when called from C (no GPU is touched). Prints one
 * "ok <name>" line per check and exits non-zero at the first failure.
 */
#include <math.h>
#include <stdio.h>
#include <string.h>

#include "cpa.h"

#define CHECK(name, cond)                                              \
  do {                                                                 \
    if (!(cond)) {                                                     \
      printf("FAIL %s: %s (%s)\n", name, #cond, cpa_last_error());     \
      return 1;                                                        \
    }                                                                  \
    printf("ok %s\n", name);                                           \
  } while (0)

int main(void) {
  CHECK("version", strncmp(cpa_version(), "cpa ", 4) == 0);

  /* Llama-3-8B layer (32 q / 8 kv heads, d = 128, page 128): one chunk of
     512 tokens after 12288 cached tokens. Eight KV heads x eight 64-token
     row tiles, each split four ways to fill 256 CUs. */
  cpa_layer_desc desc = {32, 8, 128, 128, 104, 104, 0.08838834764831845f, 0};
  const int32_t ql[1] = {512}, sl[1] = {12800};
  cpa_plan plan = NULL;
  size_t ws = 0;
  CHECK("plan_create", cpa_plan_create(&desc, ql, sl, 1, NULL, &plan, &ws) == CPA_OK);
  cpa_plan_info info;
  CHECK("plan_info", cpa_plan_get_info(plan, &info) == CPA_OK);
  CHECK("plan_items", info.num_tokens == 512 && info.num_prefill_items == 256 &&
                          info.num_combine_items == 64 && info.num_decode_items == 0);
  CHECK("plan_pairs", info.visible_pairs == 32LL * (512LL * 12288 + 512LL * 513 / 2));
  CHECK("plan_workspace", info.workspace_bytes == ws && ws > 0);
  CHECK("plan_destroy", cpa_plan_destroy(plan) == CPA_OK);

  /* Refusals carry a message. */
  cpa_layer_desc bad = desc;
  bad.head_dim = 96;
  CHECK("plan_unsupported",
        cpa_plan_create(&bad, ql, sl, 1, NULL, &plan, &ws) == CPA_ERR_UNSUPPORTED &&
            plan == NULL && strlen(cpa_last_error()) > 0);

  /* Predictor: the 64 profile sizes, a noise-free quadratic recovered, and
     the first chunk of a fresh prompt equal to the base size. */
  int64_t sizes[64];
  CHECK("profile_sizes", cpa_predictor_profile_sizes(2048, 64, 32, sizes) == CPA_OK &&
                             sizes[0] == 2048 && sizes[1] == 2016 && sizes[63] == 32);
  double lens[64], ms[64];
  const double a0 = 2e-9, b0 = 5e-6, c0 = 0.012;
  for (int i = 0; i < 64; ++i) {
    lens[i] = (double)sizes[i];
    ms[i] = a0 * lens[i] * lens[i] + b0 * lens[i] + c0;
  }
  double a, b, c, T;
  CHECK("fit", cpa_predictor_fit(lens, ms, 64, &a, &b, &c) == CPA_OK &&
                   fabs(a - a0) < 1e-9 * a0 * 1e3 && fabs(b - b0) < 1e-6 * b0 &&
                   fabs(c - c0) < 1e-6 * c0);
  const cpa_predictor_cfg cfg = {2048, 128, 64, 2048, 32768, 1.0};
  CHECK("target", cpa_predictor_target(&cfg, a, b, &T) == CPA_OK &&
                      fabs(T - (a * 2048.0 * 2048.0 + b * 2048.0)) <= 1e-15);
  int64_t chunk = 0;
  double raw = 0.0;
  CHECK("next_chunk", cpa_predictor_next_chunk(&cfg, a0, b0, a0 * 2048.0 * 2048.0 + b0 * 2048.0,
                                               0, 32768, &chunk, &raw) == CPA_OK &&
                          chunk == 2048);
  CHECK("next_chunk_later", cpa_predictor_next_chunk(&cfg, a0, b0, a0 * 2048.0 * 2048.0 + b0 * 2048.0,
                                                     16384, 16384, &chunk, &raw) == CPA_OK &&
                                chunk < 2048 && chunk % 128 == 0 && chunk >= 64);

  /* Two-micro-batch split of 16 decode rows and two 512-token chunks. */
  int32_t q18[18];
  for (int i = 0; i < 16; ++i) q18[i] = 1;
  q18[16] = q18[17] = 512;
  int32_t seq_split = -1, tok_split = -1;
  CHECK("split_simple", cpa_split_point(q18, 18, CPA_SPLIT_SIMPLE, 0.0, 0, &seq_split,
                                        &tok_split) == CPA_OK &&
                            seq_split == 9 && tok_split == 9);
  printf("done\n");
  return 0;
}
