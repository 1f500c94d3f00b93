/* Host-side paths of the library under AddressSanitizer: every size query, the planner,
 * the host policy and every argument check that fails before the library touches a GPU,
 * with extreme and invalid arguments.  tests/test_asan_host.py builds the library's host
 * code with -fsanitize=address, links this program against it and runs it; any invalid
 * memory access aborts the run.  Prints "ok <number of calls>" at the end. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "flce.h"

static int calls = 0;

static void expect(int got, int want, const char *what) {
  ++calls;
  if (got != want) {
    printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, flce_last_error());
  }
}

int main(void) {
  static const int64_t shapes[][4] = {
      {0, 8, 1, 1},          {1, 8, 1, 1},           {67, 128, 1000, 16},
      {256, 2048, 248320, 256}, {16384, 4096, 151936, 256}, {131072, 4096, 151936, 256},
      {1 << 30, 65536, 1 << 30, 1 << 30}, {(1 << 30) + 1, 8, 1, 1}, {-1, 8, 1, 1},
      {5, 0, 5, 5},          {5, 12, 5, 5},          {5, 8, 0, 5},
      {5, 8, 5, 0},          {5, 1 << 17, 5, 5},     {3, 8, 1000003, 1},
  };
  int64_t info[12];
  size_t total = 0;
  for (size_t i = 0; i < sizeof(shapes) / sizeof(shapes[0]); ++i) {
    const int64_t *s = shapes[i];
    total += flce_workspace_bytes(s[0], s[1], s[2], s[3]);
    memset(info, 0, sizeof(info));
    (void)flce_describe_plan(s[0], s[1], s[2], s[3], info);
    total += flce_distill_workspace_bytes(s[0], s[1], s[1] + 8, s[2], s[3]);
    total += flce_policy_workspace_bytes(s[0], s[1], s[2], s[3], 1);
    total += flce_policy_workspace_bytes(s[0], s[1], s[2], s[3], 0);
    calls += 5;
  }
  expect(flce_describe_plan(16, 64, 100, 16, NULL), FLCE_ERR_ARG, "plan without info");

  for (int64_t ctx = -5; ctx < 300000; ctx = ctx * 3 + 7) {
    for (int64_t m = -1; m < 70; m += 7) total += (size_t)flce_chunk_rows_for(ctx, m);
    ++calls;
  }
  int64_t mb = 0, cr = 0;
  size_t need = 0;
  const size_t budgets[] = {0, 1, (size_t)1 << 20, (size_t)8 << 30, (size_t)1 << 40, SIZE_MAX};
  for (size_t b = 0; b < sizeof(budgets) / sizeof(budgets[0]); ++b) {
    (void)flce_tune(4, 8192, 4096, 128000, budgets[b], &mb, &cr, &need);
    (void)flce_tune(1, 131072, 4096, 151936, budgets[b], &mb, &cr, NULL);
    (void)flce_tune(0, 8192, 4096, 128000, budgets[b], &mb, &cr, &need);
    (void)flce_tune(4, -1, 4096, 128000, budgets[b], &mb, &cr, &need);
    calls += 4;
  }
  expect(flce_tune(4, 8192, 4096, 128000, 1 << 30, NULL, &cr, &need), FLCE_ERR_ARG,
         "tune without outputs");

  /* forward / backward argument checks (all fail before any device call) */
  char *p16 = (char *)(uintptr_t)4096, *p8 = (char *)(uintptr_t)4104;
  const flce_logit_transform bad[] = {{-1.f, 0.f, 0.f, 1.f}, {0.f, 0.f, 0.f, 0.f},
                                      {0.f, 0.f, -3.f, 1.f}, {1e30f, 1e-30f, 0.f, 1.f}};
  expect(flce_forward(p16, p16, (int64_t *)p8, -3, 64, 100, -100, 16, 0, NULL, (float *)p16,
                      (float *)p16, NULL, p16, 1 << 30, NULL), FLCE_ERR_SHAPE, "forward T<0");
  expect(flce_forward(NULL, p16, (int64_t *)p8, 4, 64, 100, -100, 16, 0, NULL, (float *)p16,
                      (float *)p16, NULL, p16, 1 << 30, NULL), FLCE_ERR_ARG, "forward NULL");
  expect(flce_forward(p8, p16, (int64_t *)p8, 4, 64, 100, -100, 16, 0, NULL, (float *)p16,
                      (float *)p16, NULL, p16, 1 << 30, NULL), FLCE_ERR_ARG, "forward misaligned");
  expect(flce_forward(p16, p16, (int64_t *)p8, 4, 64, 100, -100, 16, 7, NULL, (float *)p16,
                      (float *)p16, NULL, p16, 1 << 30, NULL), FLCE_ERR_ARG, "forward mode");
  expect(flce_forward(p16, p16, (int64_t *)p8, 4, 64, 100, -100, 16, 0, NULL, (float *)p16,
                      (float *)p16, NULL, p16, 16, NULL), FLCE_ERR_WORKSPACE, "forward workspace");
  for (size_t i = 0; i < sizeof(bad) / sizeof(bad[0]); ++i)
    expect(flce_forward(p16, p16, (int64_t *)p8, 4, 64, 100, -100, 16, 0, &bad[i],
                        (float *)p16, (float *)p16, NULL, p16, 1 << 30, NULL),
           FLCE_ERR_ARG, "forward transform");
  expect(flce_forward_noalloc(p16, p16, (int64_t *)p8, 1400000, 4096, 151936, -100, 256, 0, NULL,
                              (float *)p16, (float *)p16, NULL, NULL),
         FLCE_ERR_WORKSPACE, "noalloc beyond its array");
  expect(flce_backward(p16, p16, (int64_t *)p8, (float *)p16, 4, 64, 100, -100, 16, 0, NULL,
                       NULL, NULL, p16, (float *)p16, 0, p16, 1 << 30, NULL),
         FLCE_ERR_ARG, "backward without grad");
  expect(flce_backward(p16, p16, (int64_t *)p8, (float *)p16, 4, 64, 100, -100, 16, 0, NULL,
                       (float *)p16, NULL, NULL, NULL, 0, p16, 1 << 30, NULL),
         FLCE_ERR_ARG, "backward without outputs");
  expect(flce_backward(p16, p16, (int64_t *)p8, (float *)p16, 4, 64, 100, -100, 16, 0, NULL,
                       (float *)p16, NULL, p16, (float *)p8, 0, p16, 1 << 30, NULL),
         FLCE_ERR_ARG, "backward misaligned dW");

  /* distillation and policy checks */
  expect(flce_distill_jsd(p16, p16, 64, p16, p16, 64, NULL, -100, 4, 100, 16, NULL, 1.5f, NULL,
                          NULL, NULL, NULL, NULL, NULL, 0, p16, 1 << 30, NULL),
         FLCE_ERR_ARG, "jsd beta");
  expect(flce_distill(NULL, p16, 64, p16, p16, 64, NULL, -100, 4, 100, 16, NULL, NULL, NULL,
                      NULL, NULL, NULL, NULL, 0, p16, 1 << 30, NULL),
         FLCE_ERR_ARG, "distill NULL");
  flce_policy_params pp = {0.04f, 0.2f, 0.2f, 1.f, 1.f};
  expect(flce_grpo_loss(p16, p16, (int64_t *)p8, -100, 6, 64, 100, 16, NULL, 4, (float *)p16,
                        NULL, NULL, &pp, (float *)p16, NULL, NULL, NULL, NULL, 0, p16, 1 << 30,
                        NULL),
         FLCE_ERR_SHAPE, "grpo n_seq does not divide T");
  expect(flce_dpo_loss(p16, p16, (int64_t *)p8, -100, 6, 64, 100, 16, NULL, 3, (float *)p16, &pp,
                       (float *)p16, NULL, NULL, NULL, NULL, 0, p16, 1 << 30, NULL),
         FLCE_ERR_SHAPE, "dpo odd n_seq");
  expect(flce_kto_loss(p16, p16, (int64_t *)p8, -100, 4, 64, 100, 16, NULL, 2, (float *)p16, NULL,
                       NULL, NULL, (float *)p16, NULL, NULL, NULL, NULL, 0, p16, 1 << 30, NULL),
         FLCE_ERR_ARG, "kto without params");

  /* timing bookkeeping that needs no device */
  expect(flce_timing_begin(0), FLCE_ERR_ARG, "timing capacity");
  expect(flce_timing_end(NULL, NULL, 0, NULL, NULL), FLCE_ERR_ARG, "timing end NULL");
  {
    int32_t ids[4];
    float ms[4];
    int32_t n = 0;
    expect(flce_timing_end(ids, ms, 4, &n, NULL), FLCE_ERR_ARG, "timing end when off");
  }
  for (int32_t id = -3; id < FLCE_KERNEL_COUNT + 3; ++id) total += strlen(flce_kernel_name(id));
  for (int s = -2; s < 9; ++s) total += strlen(flce_status_string(s));
  total += strlen(flce_last_error());
  printf("ok %d %zu\n", calls, total > 0 ? (size_t)1 : (size_t)0);
  return 0;
}
