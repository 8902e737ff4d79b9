/*
 * reject_paths.c -- the C ABI's argument checks, called from plain C (test
 * program for the host-sanitizer run; no GPU needed: every call below is
 * refused before anything touches a device).  Exit status 0 = every call
 * returned the documented status.
 */
#include <stdio.h>
#include <stdint.h>

#include "moe_dispatch.h"

static int failures = 0;

static void expect(const char *what, int got, int want) {
  if (got != want) {
    fprintf(stderr, "%s: got %d, want %d\n", what, got, want);
    ++failures;
  }
}

int main(void) {
  /* stand-in device addresses: aligned, never dereferenced on these paths */
  void *p = (void *)(uintptr_t)4096;
  int32_t *ip = (int32_t *)p;
  float *fp = (float *)p;
  moe_layout lay = {ip, ip, ip, ip, ip, NULL, ip};
  moe_layout no_status = {ip, ip, ip, ip, ip, NULL, NULL};
  const moe_shape ok = {4, 64, 8, 2, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape bad_h = {4, 12, 8, 2, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape bad_fp8_h = {4, 64, 8, 2, 2, 0, MOE_PAYLOAD_FP8_E4M3_B128};
  const moe_shape k_over_e = {4, 64, 8, 9, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape e_mod_n = {4, 64, 9, 2, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape big_e = {4, 64, 2048, 2, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape big_k = {4, 64, 64, 33, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape neg_t = {-1, 64, 8, 2, 2, 0, MOE_PAYLOAD_BF16};
  const moe_shape huge = {600000, 8, 64, 8, 8, 0, MOE_PAYLOAD_BF16};
  const moe_shape chunked = {1100, 64, 8, 8, 2, 0, MOE_PAYLOAD_BF16};  /* 8800 pairs */

  expect("recv rows", (int)moe_recv_rows(&ok), 8);
  expect("recv rows of a bad shape", (int)moe_recv_rows(&e_mod_n), -1);
  expect("workspace of a bad shape", (int)moe_dispatch_workspace_size(&bad_h), 0);
  expect("workspace one-kernel", (int)moe_dispatch_workspace_size(&ok), 0);
  expect("workspace multi-kernel", moe_dispatch_workspace_size(&chunked) > 0, 1);

  expect("route T<0", moe_route_topk(fp, NULL, -1, 8, 2, MOE_SCORE_SIGMOID, ip, fp, NULL),
         MOE_ERR_INVALID_ARG);
  expect("route k>E", moe_route_topk(fp, NULL, 4, 8, 9, MOE_SCORE_SIGMOID, ip, fp, NULL),
         MOE_ERR_INVALID_ARG);
  expect("route score", moe_route_topk(fp, NULL, 4, 8, 2, 7, ip, fp, NULL), MOE_ERR_INVALID_ARG);
  expect("route E>max", moe_route_topk(fp, NULL, 4, 2048, 2, 0, ip, fp, NULL),
         MOE_ERR_UNSUPPORTED);
  expect("route null logits", moe_route_topk(NULL, NULL, 4, 8, 2, 0, ip, fp, NULL),
         MOE_ERR_INVALID_ARG);
  expect("grouped E%G", moe_route_topk_grouped(fp, NULL, 4, 10, 2, 0, 3, 1, ip, fp, NULL),
         MOE_ERR_INVALID_ARG);
  expect("grouped kept>G", moe_route_topk_grouped(fp, NULL, 4, 8, 2, 0, 2, 3, ip, fp, NULL),
         MOE_ERR_INVALID_ARG);
  expect("grouped G>max", moe_route_topk_grouped(fp, NULL, 4, 256, 2, 0, 128, 2, ip, fp, NULL),
         MOE_ERR_UNSUPPORTED);

  const moe_shape *bad[] = {&bad_h, &bad_fp8_h, &k_over_e, &e_mod_n, &neg_t};
  for (int i = 0; i < 5; ++i) {
    expect("dispatch bad shape", moe_dispatch(bad[i], p, ip, p, fp, &lay, NULL, 0, NULL),
           MOE_ERR_INVALID_ARG);
    expect("static bad shape", moe_dispatch_static(bad[i], p, ip, p, fp, &lay, NULL),
           MOE_ERR_INVALID_ARG);
    expect("combine bad shape", moe_combine(bad[i], p, fp, &lay, fp, p, NULL),
           MOE_ERR_INVALID_ARG);
    expect("expert scale bad shape", moe_expert_scale(bad[i], p, fp, &lay, fp, p, fp, NULL),
           MOE_ERR_INVALID_ARG);
  }
  expect("dispatch E>max", moe_dispatch(&big_e, p, ip, p, NULL, &lay, NULL, 0, NULL),
         MOE_ERR_UNSUPPORTED);
  expect("dispatch k>max", moe_dispatch(&big_k, p, ip, p, NULL, &lay, NULL, 0, NULL),
         MOE_ERR_UNSUPPORTED);
  expect("dispatch null x", moe_dispatch(&ok, NULL, ip, p, NULL, &lay, NULL, 0, NULL),
         MOE_ERR_INVALID_ARG);
  expect("dispatch misaligned x", moe_dispatch(&ok, (char *)p + 8, ip, p, NULL, &lay, NULL, 0,
                                               NULL),
         MOE_ERR_INVALID_ARG);
  expect("dispatch no status", moe_dispatch(&ok, p, ip, p, NULL, &no_status, NULL, 0, NULL),
         MOE_ERR_INVALID_ARG);
  expect("dispatch null layout", moe_dispatch(&ok, p, ip, p, NULL, NULL, NULL, 0, NULL),
         MOE_ERR_INVALID_ARG);
  expect("dispatch missing workspace",
         moe_dispatch(&chunked, p, ip, p, NULL, &lay, NULL, 0, NULL), MOE_ERR_INVALID_ARG);
  expect("dispatch small workspace",
         moe_dispatch(&chunked, p, ip, p, NULL, &lay, p, 16, NULL), MOE_ERR_INVALID_ARG);
  expect("static beyond its scratch", moe_dispatch_static(&huge, p, ip, p, NULL, &lay, NULL),
         MOE_ERR_UNSUPPORTED);
  expect("sources S<1", moe_dispatch_sources(&ok, 0, p, ip, p, NULL, &lay, ip, ip, NULL, 0, NULL),
         MOE_ERR_INVALID_ARG);
  expect("sources null counts",
         moe_dispatch_sources(&ok, 2, p, ip, p, NULL, &lay, NULL, ip, NULL, 0, NULL),
         MOE_ERR_INVALID_ARG);
  expect("combine null weights", moe_combine(&ok, p, NULL, &lay, NULL, p, NULL),
         MOE_ERR_INVALID_ARG);
  expect("partial send null ids",
         moe_combine_partial_send(&ok, p, NULL, &lay, NULL, fp, p, ip, NULL), MOE_ERR_INVALID_ARG);
  expect("partial recv null out", moe_combine_partial_recv(&ok, p, ip, NULL, NULL),
         MOE_ERR_INVALID_ARG);
  expect("dispatch recv null offsets",
         moe_dispatch_recv(&ok, p, NULL, &lay, p, NULL, NULL, NULL), MOE_ERR_INVALID_ARG);
  expect("combine send misaligned",
         moe_combine_send(&ok, (char *)p + 4, NULL, &lay, p, NULL, NULL), MOE_ERR_INVALID_ARG);
  for (int s = 0; s <= 4; ++s)
    if (!moe_status_string((moe_status)s)) ++failures;
  if (failures) return 1;
  printf("reject_paths: ok\n");
  return 0;
}
