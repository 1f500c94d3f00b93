/* A C99 caller of the library: include/flce.h must compile as C, and the host-only
 * entry points (workspace sizes, plan, host policy, status text) must link and answer
 * without a GPU.  Prints one line per check; tests/test_abi_c.py compiles and runs it. */
#include <stdio.h>

#include "flce.h"

int main(void) {
  int64_t info[12];
  int64_t mb = 0, cr = 0;
  size_t need = 0;
  flce_policy_params pp = {0.04f, 0.2f, 0.2f, 1.0f, 1.0f};
  flce_logit_transform xf = {0.0f, 0.0f, 30.0f, 0.7f};
  (void)pp;
  (void)xf;
  printf("workspace %zu\n", flce_workspace_bytes(16384, 4096, 151936, 256));
  flce_status st = flce_describe_plan(16384, 4096, 151936, 256, info);
  printf("plan %d %lld\n", (int)st, (long long)info[3]);
  printf("distill %zu\n", flce_distill_workspace_bytes(16384, 4096, 5120, 151936, 256));
  printf("policy %zu\n", flce_policy_workspace_bytes(32768, 4096, 128000, 256, 4));
  printf("chunk_rows %lld\n", (long long)flce_chunk_rows_for(8192, 0));
  st = flce_tune(4, 8192, 4096, 128000, (size_t)8 << 30, &mb, &cr, &need);
  printf("tune %d %lld %lld\n", (int)st, (long long)mb, (long long)cr);
  printf("bad_shape %d\n", (int)flce_describe_plan(16, 60, 100, 16, info));
  printf("status %s\n", flce_status_string(FLCE_ERR_WORKSPACE));
  printf("bad_shape_error %s\n", flce_last_error());
  printf("forward_scratch %zu\n", (size_t)FLCE_FORWARD_SCRATCH_BYTES);
  printf("kernel %s %s\n", flce_kernel_name(FLCE_KERNEL_BWD_GRAD), flce_kernel_name(FLCE_KERNEL_COUNT));
  printf("timing_off %d\n", (int)flce_timing_end(NULL, NULL, 0, NULL, NULL));
  printf("last_error %s\n", flce_last_error());
  return 0;
}
