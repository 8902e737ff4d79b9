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
 * without a launch.
 *
 * Then, on ids and weights drawn directly, it runs moe_dispatch and
 * moe_combine on the multi-kernel layout path (T*k above the one-kernel
 * limit, with a workspace of moe_dispatch_workspace_size bytes) for the bf16
 * and the fp8 payload, and on the one-kernel path for both, and checks the
 * layout against oracle_layout, the whole poisoned receive buffer (payload,
 * fp8 scales and canary rows past the end) against oracle_dispatch_bf16 /
 * oracle_dispatch_fp8, and the output against oracle_combine_f32_ordered,
 * all bit for bit.  Exit status 0 = pass.
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

enum { CANARY = 4 };

/* One dispatch + combine on ids and weights drawn here; receive rows are the
 * expert outputs (identity experts).  Returns 0 on a bit-exact match with the
 * oracle, else a distinct non-zero code. */
static int direct_case(int T, int H, int E, int K, int N, int C, int payload,
                       uint64_t seed) {
  const moe_shape shape = {T, H, E, K, N, C, payload};
  const int fp8 = payload == MOE_PAYLOAD_FP8_E4M3_B128;
  const int64_t rows = moe_recv_rows(&shape);
  const size_t row_bytes = fp8 ? (size_t)H : 2 * (size_t)H;
  const size_t nb = fp8 ? (size_t)H / 128 : 0;
  const size_t buf_rows = (size_t)rows + CANARY;
  const size_t ws_bytes = moe_dispatch_workspace_size(&shape);
  const size_t nmeta = 2 * (size_t)E + 2 * (size_t)N + 1;
  if (rows < 0) return 20;

  uint16_t *x = malloc(2 * (size_t)T * H);
  int32_t *ids = malloc(4 * (size_t)T * K);
  float *w = malloc(4 * (size_t)T * K);
  for (size_t i = 0; i < (size_t)T * H; ++i) {
    /* values over a wide range of magnitudes, so fp8 blocks get varied scales */
    const int m = (int)(lcg(&seed) % 2001) - 1000;
    const float v = (float)m * (float)(1u << (lcg(&seed) % 8)) / 256.0f;
    uint32_t u;
    memcpy(&u, &v, 4);
    x[i] = (uint16_t)(u >> 16);
  }
  for (size_t i = 0; i < (size_t)T * K; ++i) {
    ids[i] = (int32_t)(lcg(&seed) % (uint32_t)E); /* repeats within a token allowed */
    w[i] = (float)(1 + lcg(&seed) % 1000) / 1000.0f;
  }

  uint16_t *d_x, *d_out;
  int32_t *d_ids, *d_meta, *d_token_row;
  float *d_w, *d_scales = NULL;
  void *d_recv, *d_ws = NULL;
  HIP_OK(hipMalloc((void **)&d_x, 2 * (size_t)T * H));
  HIP_OK(hipMalloc((void **)&d_out, 2 * (size_t)T * H));
  HIP_OK(hipMalloc((void **)&d_ids, 4 * (size_t)T * K));
  HIP_OK(hipMalloc((void **)&d_w, 4 * (size_t)T * K));
  HIP_OK(hipMalloc((void **)&d_meta, 4 * nmeta));
  HIP_OK(hipMalloc((void **)&d_token_row, 4 * (size_t)T * K));
  HIP_OK(hipMalloc(&d_recv, buf_rows * row_bytes));
  if (fp8) HIP_OK(hipMalloc((void **)&d_scales, buf_rows * nb * 4));
  if (ws_bytes) HIP_OK(hipMalloc(&d_ws, ws_bytes));
  /* poison: e4m3 NaN codes / bf16 NaN rows, NaN scales */
  HIP_OK(hipMemset(d_recv, fp8 ? 0x7F : 0xFF, buf_rows * row_bytes));
  if (fp8) HIP_OK(hipMemset(d_scales, 0xFF, buf_rows * nb * 4));
  HIP_OK(hipMemcpy(d_x, x, 2 * (size_t)T * H, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_ids, ids, 4 * (size_t)T * K, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_w, w, 4 * (size_t)T * K, hipMemcpyHostToDevice));

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
  if (ws_bytes && moe_dispatch(&shape, d_x, d_ids, d_recv, d_scales, &lay, NULL, 0, st) !=
                      MOE_ERR_INVALID_ARG) {
    fprintf(stderr, "a missing workspace was not rejected\n");
    return 21;
  }
  MOE_OK_OR_FAIL(moe_dispatch(&shape, d_x, d_ids, d_recv, d_scales, &lay, d_ws, ws_bytes, st));
  MOE_OK_OR_FAIL(moe_combine(&shape, d_recv, d_scales, &lay, d_w, d_out, st));
  HIP_OK(hipStreamSynchronize(st));

  int32_t *meta = malloc(4 * nmeta), *token_row = malloc(4 * (size_t)T * K);
  uint8_t *recv = malloc(buf_rows * row_bytes);
  float *scales = fp8 ? malloc(buf_rows * nb * 4) : NULL;
  uint16_t *out = malloc(2 * (size_t)T * H);
  HIP_OK(hipMemcpy(meta, d_meta, 4 * nmeta, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(token_row, d_token_row, 4 * (size_t)T * K, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(recv, d_recv, buf_rows * row_bytes, hipMemcpyDeviceToHost));
  if (fp8) HIP_OK(hipMemcpy(scales, d_scales, buf_rows * nb * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(out, d_out, 2 * (size_t)T * H, hipMemcpyDeviceToHost));

  /* the oracle on the same ids */
  int32_t *o_meta = calloc(nmeta, 4), *o_token_row = malloc(4 * (size_t)T * K);
  uint8_t *o_recv = malloc(buf_rows * row_bytes);
  float *o_scales = fp8 ? malloc(buf_rows * nb * 4) : NULL;
  uint16_t *o_out = malloc(2 * (size_t)T * H);
  if (oracle_layout(ids, T, K, E, N, C, o_meta, o_meta + E, o_meta + 2 * E,
                    o_meta + 2 * E + N, o_token_row, NULL, rows, o_meta + 2 * E + 2 * N) != 0)
    return 22;
  if (memcmp(o_meta, meta, 4 * nmeta) != 0 ||
      memcmp(o_token_row, token_row, 4 * (size_t)T * K) != 0) {
    fprintf(stderr, "layout differs from the oracle (T=%d E=%d k=%d fp8=%d)\n", T, E, K, fp8);
    return 23;
  }
  memset(o_recv, fp8 ? 0x7F : 0xFF, buf_rows * row_bytes);
  if (fp8) {
    memset(o_scales, 0xFF, buf_rows * nb * 4);
    oracle_dispatch_fp8(x, T, H, K, o_token_row, o_recv, o_scales);
  } else {
    oracle_dispatch_bf16(x, T, H, K, o_token_row, (uint16_t *)o_recv);
  }
  if (memcmp(o_recv, recv, buf_rows * row_bytes) != 0 ||
      (fp8 && memcmp(o_scales, scales, buf_rows * nb * 4) != 0)) {
    fprintf(stderr, "receive buffer differs from the oracle (T=%d fp8=%d)\n", T, fp8);
    return 24;
  }
  oracle_combine_f32_ordered(o_recv, o_scales, o_token_row, w, T, K, H, o_out);
  if (memcmp(o_out, out, 2 * (size_t)T * H) != 0) {
    fprintf(stderr, "combine differs from the oracle's fp32 chain (T=%d fp8=%d)\n", T, fp8);
    return 25;
  }
  printf("c_abi_smoke: %s, %d tokens, %d experts, top-%d, %d ranks, C=%d, workspace %zu "
         "bytes: ok\n", fp8 ? "fp8" : "bf16", T, E, K, N, C, ws_bytes);
  HIP_OK(hipStreamDestroy(st));
  hipFree(d_x); hipFree(d_out); hipFree(d_ids); hipFree(d_w); hipFree(d_meta);
  hipFree(d_token_row); hipFree(d_recv); hipFree(d_scales); hipFree(d_ws);
  free(x); free(ids); free(w); free(meta); free(token_row); free(recv); free(scales); free(out);
  free(o_meta); free(o_token_row); free(o_recv); free(o_scales); free(o_out);
  return 0;
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
  printf("c_abi_smoke: routed case (%d tokens, %d experts, top-%d, %d ranks, %lld rows) ok\n",
         T, E, K, N, (long long)rows);
  int rc;
  /* multi-kernel layout path with a workspace (more than 8192 pairs): bf16
     packed with the layout in one launch (9 chunks of 1024 pairs) and in two
     (17 chunks), fp8 with a capacity some ranks overflow; then the one-kernel
     path, bf16 (5600 pairs) and fp8 */
  {
    const moe_shape multi = {1100, 136, 32, 8, 4, 0, MOE_PAYLOAD_BF16};
    const moe_shape one = {700, 136, 32, 8, 4, 0, MOE_PAYLOAD_BF16};
    if (moe_dispatch_workspace_size(&multi) == 0 || moe_dispatch_workspace_size(&one) != 0) {
      fprintf(stderr, "workspace sizes do not follow the two dispatch paths\n");
      return 11;
    }
  }
  if ((rc = direct_case(1100, 136, 32, 8, 4, 0, MOE_PAYLOAD_BF16, 77)) != 0) return rc;
  if ((rc = direct_case(2100, 64, 32, 8, 4, 0, MOE_PAYLOAD_BF16, 80)) != 0) return rc;
  if ((rc = direct_case(1100, 256, 64, 8, 8, 950, MOE_PAYLOAD_FP8_E4M3_B128, 78)) != 0) return rc;
  if ((rc = direct_case(700, 136, 32, 8, 4, 0, MOE_PAYLOAD_BF16, 81)) != 0) return rc;
  if ((rc = direct_case(64, 384, 16, 4, 4, 256, MOE_PAYLOAD_FP8_E4M3_B128, 79)) != 0) return rc;
  printf("c_abi_smoke: ok\n");
  return 0;
}
