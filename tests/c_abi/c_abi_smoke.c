/*
 * c_abi_smoke.c -- the library used from plain C, through include/moe_dispatch.h
 * only (test program; it also links the CPU oracle, which is test
 * infrastructure).
 *
 * Routes seeded logits with moe_route_topk, dispatches bf16 tokens into
 * fixed-capacity regions with moe_dispatch, treats the receive regions as the
 * expert outputs (identity experts) and combines them with moe_combine.  It
 * checks that the ids match the oracle's top-k, that the layout metadata match
 * oracle_layout bit for bit, that every placed row equals its token's row,
 * and that combining identity experts with weights 1/2 and 1/2 returns the
 * tokens exactly.  It also checks that a null token pointer is rejected
 * without a launch.  Exit status 0 = pass.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_dispatch.h"
#include "moe_oracle.h"

#define HIP_OK(call)                                                          \
  do {                                                                        \
    hipError_t e_ = (call);                                                   \
    if (e_ != hipSuccess) {                                                   \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));       \
      return 2;                                                               \
    }                                                                         \
  } while (0)

#define MOE_OK_OR_FAIL(call)                                                  \
  do {                                                                        \
    moe_status s_ = (call);                                                   \
    if (s_ != MOE_OK) {                                                       \
      fprintf(stderr, "%s: %s\n", #call, moe_status_string(s_));              \
      return 3;                                                               \
    }                                                                         \
  } while (0)

static uint32_t lcg(uint64_t *s) {
  *s = *s * 6364136223846793005ull + 1442695040888963407ull;
  return (uint32_t)(*s >> 33);
}

int main(void) {
  enum { T = 96, H = 520, E = 16, K = 2, N = 4 };
  const int L = E / N;
  const int C = T * (K < L ? K : L);
  const moe_shape shape = {T, H, E, K, N, C, MOE_PAYLOAD_BF16};
  const int64_t rows = moe_recv_rows(&shape);
  uint64_t seed = 1234;

  /* host inputs: logits, and bf16 tokens with small integer values */
  float *logits = malloc(sizeof(float) * T * E);
  uint16_t *x = malloc(sizeof(uint16_t) * T * H);
  for (int i = 0; i < T * E; ++i) logits[i] = (float)(lcg(&seed) % 1000) / 97.0f - 5.0f;
  for (int i = 0; i < T * H; ++i) {
    const float v = (float)((int)(lcg(&seed) % 64) - 32);
    uint32_t u;
    memcpy(&u, &v, 4);
    x[i] = (uint16_t)(u >> 16); /* exact: small integers are bf16 values */
  }

  /* device buffers */
  float *d_logits, *d_w;
  int32_t *d_ids, *d_meta, *d_token_row;
  uint16_t *d_x, *d_recv, *d_out;
  HIP_OK(hipMalloc((void **)&d_logits, sizeof(float) * T * E));
  HIP_OK(hipMalloc((void **)&d_w, sizeof(float) * T * K));
  HIP_OK(hipMalloc((void **)&d_ids, sizeof(int32_t) * T * K));
  HIP_OK(hipMalloc((void **)&d_meta, sizeof(int32_t) * (2 * E + 2 * N + 1)));
  HIP_OK(hipMalloc((void **)&d_token_row, sizeof(int32_t) * T * K));
  HIP_OK(hipMalloc((void **)&d_x, sizeof(uint16_t) * T * H));
  HIP_OK(hipMalloc((void **)&d_recv, sizeof(uint16_t) * rows * H));
  HIP_OK(hipMalloc((void **)&d_out, sizeof(uint16_t) * T * H));
  HIP_OK(hipMemcpy(d_logits, logits, sizeof(float) * T * E, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x, x, sizeof(uint16_t) * T * H, hipMemcpyHostToDevice));

  moe_layout lay;
  lay.expert_counts = d_meta;
  lay.expert_offsets = d_meta + E;
  lay.rank_counts = d_meta + 2 * E;
  lay.rank_offsets = d_meta + 2 * E + N;
  lay.status = d_meta + 2 * E + 2 * N;
  lay.token_row = d_token_row;
  lay.row_src = NULL;

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));

  /* a null token pointer is a host-detectable error: nothing is launched */
  if (moe_dispatch(&shape, NULL, d_ids, d_recv, NULL, &lay, NULL, 0, st) !=
      MOE_ERR_INVALID_ARG) {
    fprintf(stderr, "null x was not rejected\n");
    return 4;
  }

  MOE_OK_OR_FAIL(moe_route_topk(d_logits, NULL, T, E, K, MOE_SCORE_SOFTMAX, d_ids, d_w, st));
  MOE_OK_OR_FAIL(moe_dispatch(&shape, d_x, d_ids, d_recv, NULL, &lay, NULL, 0, st));
  /* identity experts; weights 1/2 and 1/2 make the combine return x exactly */
  float *w_half = malloc(sizeof(float) * T * K);
  for (int i = 0; i < T * K; ++i) w_half[i] = 0.5f;
  HIP_OK(hipMemcpyAsync(d_w, w_half, sizeof(float) * T * K, hipMemcpyHostToDevice, st));
  MOE_OK_OR_FAIL(moe_combine(&shape, d_recv, NULL, &lay, d_w, d_out, st));
  HIP_OK(hipStreamSynchronize(st));

  int32_t *ids = malloc(sizeof(int32_t) * T * K);
  int32_t *meta = malloc(sizeof(int32_t) * (2 * E + 2 * N + 1));
  int32_t *token_row = malloc(sizeof(int32_t) * T * K);
  uint16_t *recv = malloc(sizeof(uint16_t) * rows * H);
  uint16_t *out = malloc(sizeof(uint16_t) * T * H);
  HIP_OK(hipMemcpy(ids, d_ids, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(meta, d_meta, sizeof(int32_t) * (2 * E + 2 * N + 1), hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(token_row, d_token_row, sizeof(int32_t) * T * K, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(recv, d_recv, sizeof(uint16_t) * rows * H, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, sizeof(uint16_t) * T * H, hipMemcpyDeviceToHost));

  /* the oracle on the same logits and on the GPU's ids */
  int32_t o_ids[T * K];
  float o_w[T * K];
  if (oracle_route_topk(logits, NULL, T, E, K, 0, o_ids, o_w) != 0) return 5;
  if (memcmp(o_ids, ids, sizeof(o_ids)) != 0) {
    fprintf(stderr, "route ids differ from the oracle\n");
    return 6;
  }
  int32_t o_meta[2 * E + 2 * N + 1];
  int32_t o_token_row[T * K];
  o_meta[2 * E + 2 * N] = 0;
  if (oracle_layout(ids, T, K, E, N, C, o_meta, o_meta + E, o_meta + 2 * E,
                    o_meta + 2 * E + N, o_token_row, NULL, rows, o_meta + 2 * E + 2 * N) != 0)
    return 7;
  if (memcmp(o_meta, meta, sizeof(o_meta)) != 0 ||
      memcmp(o_token_row, token_row, sizeof(o_token_row)) != 0) {
    fprintf(stderr, "layout differs from the oracle\n");
    return 8;
  }
  for (int p = 0; p < T * K; ++p) {
    if (token_row[p] < 0) continue;
    if (memcmp(recv + (size_t)token_row[p] * H, x + (size_t)(p / K) * H, 2 * H) != 0) {
      fprintf(stderr, "row of pair %d differs from its token\n", p);
      return 9;
    }
  }
  if (memcmp(out, x, sizeof(uint16_t) * T * H) != 0) {
    fprintf(stderr, "combine of identity experts did not return the tokens\n");
    return 10;
  }
  printf("c_abi_smoke: ok (%d tokens, %d experts, top-%d, %d ranks, %lld rows)\n", T, E, K, N,
         (long long)rows);
  return 0;
}
