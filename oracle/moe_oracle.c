/*
 * moe_oracle.c -- plain CPU oracle for MoE dispatch and combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may call it; the
 * tests, the smoke check and the benchmark's CPU-baseline leg are its only
 * users.  It is deliberately slow and literal: every function follows the
 * plain definition of what it computes, with no blocking, fusion or reordering.
 * Build: gcc -O2 -std=c11 -fno-fast-math -ffp-contract=off -shared -fPIC.
 *
 * Citations are to two pages: "Enabling trillion-parameter models on AWS EFA"
 * (the EFA page) and "Lower Latency and Higher Throughput with Multi-Node
 * DeepSeek Deployment" (the DeepSeek-deployment page).
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* Scalar codecs, written from the number formats.                          */
/* ------------------------------------------------------------------------ */

/* bfloat16: sign, 8 exponent bits (bias 127), 7 stored mantissa bits, so 8
 * significant bits for normal values and a spacing of 2^-133 below 2^-126.
 * The nearest representable value is found by scaling |v| so that one unit in
 * the last place is 1, rounding that to an integer with ties to even
 * (nearbyint under the default rounding mode), and scaling back. */
uint16_t oracle_f64_to_bf16(double v) {
  if (isnan(v)) return signbit(v) ? 0xFFC0u : 0x7FC0u;
  uint16_t sign = signbit(v) ? 0x8000u : 0u;
  if (isinf(v)) return sign | 0x7F80u;
  double a = fabs(v);
  int e;
  frexp(a, &e); /* a in [2^(e-1), 2^e) */
  int ulp_exp = e - 8;
  if (ulp_exp < -133) ulp_exp = -133;
  double r = nearbyint(ldexp(a, -ulp_exp));
  double res = ldexp(r, ulp_exp);
  if (res >= ldexp(1.0, 128)) return sign | 0x7F80u; /* overflow */
  float f = (float)res; /* exact: res is a bfloat16 value */
  uint32_t u;
  memcpy(&u, &f, sizeof u);
  return sign | (uint16_t)((u >> 16) & 0x7FFFu);
}

/* fp32 -> double is exact, so this is one rounding of the fp32 value. */
uint16_t oracle_f32_to_bf16(float v) { return oracle_f64_to_bf16((double)v); }

float oracle_bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return f;
}

/* OCP fp8 e4m3fn: sign, 4 exponent bits (bias 7), 3 mantissa bits; no
 * infinities; only S.1111.111 is NaN, so the largest finite value is
 * 1.75 * 2^8 = 448.  Normal values start at 2^-6; subnormals are m * 2^-9.
 * Rounding is to nearest, ties to even; magnitudes beyond 448 (and infinity)
 * saturate to 448. */
uint8_t oracle_f32_to_e4m3(float v) {
  if (isnan(v)) return 0x7Fu;
  uint8_t sign = signbit(v) ? 0x80u : 0u;
  double a = fabs((double)v);
  double res;
  if (isinf(a)) {
    res = 448.0;
  } else {
    int e;
    frexp(a, &e); /* a in [2^(e-1), 2^e) */
    int ulp_exp = e - 4; /* 4 significant bits */
    if (ulp_exp < -9) ulp_exp = -9;
    double r = nearbyint(ldexp(a, -ulp_exp));
    res = ldexp(r, ulp_exp);
    if (res > 448.0) res = 448.0;
  }
  if (res < ldexp(1.0, -6)) {
    /* subnormal (or zero): the code is the multiple of 2^-9 (0..7) */
    return sign | (uint8_t)ldexp(res, 9);
  }
  int e2;
  double f = frexp(res, &e2); /* res = (2f) * 2^(e2-1), 2f in [1,2) */
  int biased = e2 - 1 + 7;
  int mant = (int)((2.0 * f - 1.0) * 8.0);
  return sign | (uint8_t)((biased << 3) | mant);
}

float oracle_e4m3_to_f32(uint8_t c) {
  int s = c >> 7, ex = (c >> 3) & 15, m = c & 7;
  if (ex == 15 && m == 7) return NAN;
  double v = (ex == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, ex - 7);
  return (float)(s ? -v : v);
}

/* ------------------------------------------------------------------------ */
/* Routing (EFA page, Introduction: a small linear router picks the experts */
/* of each token; DeepSeek-deployment page, MoE Router: top-k indices and   */
/* scores).  The biased logit is one fp32 add; the k largest are taken one  */
/* at a time, ties to the lower expert id, so slots come out in descending  */
/* order.  Weights are formed in double and rounded once to fp32, and sum   */
/* to one over the k chosen experts (the combine forms a weighted average). */
/* ------------------------------------------------------------------------ */
int oracle_route_topk(const float *logits, const float *bias, int T, int E,
                      int k, int score, int32_t *ids, float *weights) {
  if (T < 0 || E < 1 || k < 1 || k > E) return -1;
  if (score != ORACLE_SCORE_SOFTMAX && score != ORACLE_SCORE_SIGMOID) return -1;
  float *lp = (float *)malloc(sizeof(float) * (size_t)E);
  char *taken = (char *)malloc((size_t)E);
  double *s = (double *)malloc(sizeof(double) * (size_t)k);
  int rc = 0;
  for (int t = 0; t < T && rc == 0; ++t) {
    for (int e = 0; e < E; ++e) {
      lp[e] = bias ? logits[(size_t)t * E + e] + bias[e] : logits[(size_t)t * E + e];
      if (!isfinite(lp[e])) rc = -1;
    }
    if (rc) break;
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (!taken[e] && (best < 0 || lp[e] > lp[best])) best = e;
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      double l = (double)lp[ids[(size_t)t * k + j]];
      if (score == ORACLE_SCORE_SIGMOID)
        s[j] = 1.0 / (1.0 + exp(-l));
      else
        s[j] = exp(l - (double)lp[ids[(size_t)t * k]]);
      sum += s[j];
    }
    for (int j = 0; j < k; ++j) weights[(size_t)t * k + j] = (float)(s[j] / sum);
  }
  free(lp);
  free(taken);
  free(s);
  return rc;
}

/* Group-limited routing (DeepSeek-deployment page, MoE Router: the same   */
/* router serves every MoE model, plain top-k being the case where the top  */
/* group set is all experts).  Steps, per token: biased logits; each group's */
/* score = sum of its two largest biased logits (one fp32 add); keep the     */
/* topk_groups best groups, ties to the lower group id; then the plain top-k */
/* over the kept groups' experts and the same weights.                       */
int oracle_route_topk_grouped(const float *logits, const float *bias, int T,
                              int E, int k, int score, int n_groups,
                              int topk_groups, int32_t *ids, float *weights) {
  if (T < 0 || E < 1 || k < 1 || n_groups < 1 || E % n_groups != 0) return -1;
  if (topk_groups < 1 || topk_groups > n_groups) return -1;
  const int gsz = E / n_groups;
  if (k > topk_groups * gsz) return -1;
  if (score != ORACLE_SCORE_SOFTMAX && score != ORACLE_SCORE_SIGMOID) return -1;
  float *lp = (float *)malloc(sizeof(float) * (size_t)E);
  char *taken = (char *)malloc((size_t)E);
  double *s = (double *)malloc(sizeof(double) * (size_t)k);
  float *gscore = (float *)malloc(sizeof(float) * (size_t)n_groups);
  char *keep = (char *)malloc((size_t)n_groups);
  int rc = 0;
  for (int t = 0; t < T && rc == 0; ++t) {
    const float *row = logits + (size_t)t * E;
    for (int g = 0; g < n_groups; ++g) {
      /* the two largest biased logits of the group (first-seen on ties) */
      int b1 = -1, b2 = -1;
      float v1 = 0.0f, v2 = 0.0f;
      for (int e = g * gsz; e < (g + 1) * gsz; ++e) {
        float l = bias ? row[e] + bias[e] : row[e];
        if (!isfinite(l)) rc = -1;
        if (b1 < 0 || l > v1) {
          b2 = b1;
          v2 = v1;
          b1 = e;
          v1 = l;
        } else if (b2 < 0 || l > v2) {
          b2 = e;
          v2 = l;
        }
      }
      gscore[g] = (b2 < 0) ? v1 : v1 + v2;
    }
    if (rc) break;
    memset(keep, 0, (size_t)n_groups);
    for (int r = 0; r < topk_groups; ++r) {
      int best = -1;
      for (int g = 0; g < n_groups; ++g)
        if (!keep[g] && (best < 0 || gscore[g] > gscore[best])) best = g;
      keep[best] = 1;
    }
    /* the plain top-k over the experts of the kept groups */
    for (int e = 0; e < E; ++e) lp[e] = bias ? row[e] + bias[e] : row[e];
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
      int best = -1;
      for (int e = 0; e < E; ++e)
        if (keep[e / gsz] && !taken[e] && (best < 0 || lp[e] > lp[best])) best = e;
      taken[best] = 1;
      ids[(size_t)t * k + j] = best;
    }
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
      double l = (double)lp[ids[(size_t)t * k + j]];
      if (score == ORACLE_SCORE_SIGMOID)
        s[j] = 1.0 / (1.0 + exp(-l));
      else
        s[j] = exp(l - (double)lp[ids[(size_t)t * k]]);
      sum += s[j];
    }
    for (int j = 0; j < k; ++j) weights[(size_t)t * k + j] = (float)(s[j] / sum);
  }
  free(lp);
  free(taken);
  free(s);
  free(gscore);
  free(keep);
  return rc;
}

/* ------------------------------------------------------------------------ */
/* Layout (EFA page, Send and Receive Buffers and Dispatch and Combine:     */
/* per-expert counts, their cumulative sum, offsets of contiguous regions). */
/* Expert e lives on rank e / L with L = E / N.  The valid pairs are sorted */
/* by (rank, expert, token, slot); that order fills each rank's region.     */
/* ------------------------------------------------------------------------ */
typedef struct {
  int32_t rank, expert, token, slot;
} oracle_pair;

static int oracle_pair_cmp(const void *pa, const void *pb) {
  const oracle_pair *a = (const oracle_pair *)pa, *b = (const oracle_pair *)pb;
  if (a->rank != b->rank) return a->rank < b->rank ? -1 : 1;
  if (a->expert != b->expert) return a->expert < b->expert ? -1 : 1;
  if (a->token != b->token) return a->token < b->token ? -1 : 1;
  if (a->slot != b->slot) return a->slot < b->slot ? -1 : 1;
  return 0;
}

int oracle_layout(const int32_t *ids, int T, int k, int E, int N, int C,
                  int32_t *expert_counts, int32_t *expert_offsets,
                  int32_t *rank_counts, int32_t *rank_offsets,
                  int32_t *token_row, int32_t *row_src, int64_t rows,
                  int32_t *status) {
  if (T < 0 || k < 1 || E < 1 || N < 1 || E % N != 0 || C < 0) return -1;
  int64_t need = C > 0 ? (int64_t)N * C : (int64_t)T * k;
  if (row_src && rows < need) return -1;
  int L = E / N;
  size_t P = (size_t)T * (size_t)k;
  oracle_pair *pairs = (oracle_pair *)malloc(sizeof(oracle_pair) * (P ? P : 1));
  size_t n = 0;
  for (int e = 0; e < E; ++e) expert_counts[e] = 0;
  for (int r = 0; r < N; ++r) rank_counts[r] = 0;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int32_t e = ids[(size_t)t * k + j];
      token_row[(size_t)t * k + j] = -1;
      if (e < 0 || e >= E) {
        *status |= ORACLE_ST_BAD_ID;
        continue;
      }
      pairs[n].rank = e / L;
      pairs[n].expert = e;
      pairs[n].token = t;
      pairs[n].slot = j;
      ++n;
      expert_counts[e] += 1;
      rank_counts[e / L] += 1;
    }
  qsort(pairs, n, sizeof(oracle_pair), oracle_pair_cmp);

  int32_t run = 0;
  for (int r = 0; r < N; ++r) {
    if (C > 0) {
      rank_offsets[r] = r * C;
    } else {
      rank_offsets[r] = run;
      run += rank_counts[r];
    }
  }
  for (int e = 0; e < E; ++e) {
    int r = e / L;
    int32_t before = 0;
    for (int e2 = r * L; e2 < e; ++e2) before += expert_counts[e2];
    expert_offsets[e] = rank_offsets[r] + before;
  }

  int32_t *pos = (int32_t *)calloc((size_t)N, sizeof(int32_t));
  for (size_t i = 0; i < n; ++i) {
    int r = pairs[i].rank;
    size_t p = (size_t)pairs[i].token * k + pairs[i].slot;
    if (C > 0 && pos[r] >= C) {
      *status |= ORACLE_ST_CAPACITY;
    } else {
      int32_t row = rank_offsets[r] + pos[r];
      token_row[p] = row;
      if (row_src) row_src[row] = (int32_t)p;
    }
    pos[r] += 1;
  }
  free(pos);
  free(pairs);
  return 0;
}

/* Every rank dispatching at once (EFA page, Send and Receive Buffers: the  */
/* ranks first exchange their per-expert token counts, after which each     */
/* knows where its writes go and at which offset it receives each rank's    */
/* tokens).  Source s's tokens are global tokens s*T .. s*T+T-1, so sorting  */
/* by (rank, expert, source, token, slot) is sorting the S*T tokens by       */
/* (rank, expert, global token, slot): the single-source layout over all of  */
/* them.  The exchanged count vectors and the per-source offsets follow.     */
int oracle_layout_sources(const int32_t *ids, int S, int T, int k, int E, int N,
                          int C, int32_t *expert_counts,
                          int32_t *expert_offsets, int32_t *rank_counts,
                          int32_t *rank_offsets, int32_t *token_row,
                          int32_t *source_counts, int32_t *source_offsets,
                          int32_t *status) {
  if (S < 1 || T < 0 || (int64_t)S * T > INT32_MAX) return -1;
  int rc = oracle_layout(ids, S * T, k, E, N, C, expert_counts, expert_offsets,
                         rank_counts, rank_offsets, token_row, NULL, 0, status);
  if (rc) return rc;
  for (int s = 0; s < S; ++s) {
    for (int e = 0; e < E; ++e) source_counts[(size_t)s * E + e] = 0;
    for (size_t q = (size_t)s * T * k; q < (size_t)(s + 1) * T * k; ++q) {
      int32_t e = ids[q];
      if (e >= 0 && e < E) source_counts[(size_t)s * E + e] += 1;
    }
  }
  for (int e = 0; e < E; ++e) {
    int32_t run = expert_offsets[e];
    for (int s = 0; s < S; ++s) {
      source_offsets[(size_t)e * S + s] = run;
      run += source_counts[(size_t)s * E + e];
    }
  }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Dispatch (EFA page, Introduction and MoE all-to-all over EFA: each token */
/* goes to the ranks hosting its experts; Evaluation: block-scaled fp8      */
/* dispatch; DeepSeek-deployment page, Quantization: one dynamic scale per  */
/* 128-element activation vector).                                          */
/* ------------------------------------------------------------------------ */
void oracle_dispatch_bf16(const uint16_t *x, int T, int H, int k,
                          const int32_t *token_row, uint16_t *recv) {
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int32_t row = token_row[(size_t)t * k + j];
      if (row < 0) continue;
      memcpy(recv + (size_t)row * H, x + (size_t)t * H, sizeof(uint16_t) * (size_t)H);
    }
}

/* Per block of 128 columns: amax = max |x|, scale = amax / 448 (fp32
 * division), code = e4m3(x / scale) (fp32 division).  An all-zero block gets
 * scale 0 and codes 0. */
void oracle_quantize_row_fp8(const uint16_t *x, int H, uint8_t *q, float *scales) {
  for (int b = 0; b < H / 128; ++b) {
    float amax = 0.0f;
    for (int i = b * 128; i < b * 128 + 128; ++i) {
      float v = fabsf(oracle_bf16_to_f32(x[i]));
      if (v > amax) amax = v;
    }
    float s = amax / 448.0f;
    scales[b] = s;
    for (int i = b * 128; i < b * 128 + 128; ++i)
      q[i] = (amax == 0.0f) ? 0u : oracle_f32_to_e4m3(oracle_bf16_to_f32(x[i]) / s);
  }
}

void oracle_dispatch_fp8(const uint16_t *x, int T, int H, int k,
                         const int32_t *token_row, uint8_t *recv,
                         float *recv_scales) {
  int nb = H / 128;
  uint8_t *q = (uint8_t *)malloc((size_t)H);
  float *sc = (float *)malloc(sizeof(float) * (size_t)(nb ? nb : 1));
  for (int t = 0; t < T; ++t) {
    oracle_quantize_row_fp8(x + (size_t)t * H, H, q, sc);
    for (int j = 0; j < k; ++j) {
      int32_t row = token_row[(size_t)t * k + j];
      if (row < 0) continue;
      memcpy(recv + (size_t)row * H, q, (size_t)H);
      memcpy(recv_scales + (size_t)row * nb, sc, sizeof(float) * (size_t)nb);
    }
  }
  free(q);
  free(sc);
}

/* ------------------------------------------------------------------------ */
/* Expert stand-in.  The grouped GEMM between dispatch and combine (EFA     */
/* page, MoE all-to-all over EFA) needs trained weights; a per-expert       */
/* scalar keeps every row tied to the expert it was routed to.              */
/* ------------------------------------------------------------------------ */
void oracle_expert_scale_bf16(const uint16_t *recv, const int32_t *ids,
                              const int32_t *token_row, int T, int k, int H,
                              const float *alpha, uint16_t *y) {
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int32_t row = token_row[(size_t)t * k + j];
      if (row < 0) continue;
      float a = alpha[ids[(size_t)t * k + j]];
      for (int i = 0; i < H; ++i) {
        float p = a * oracle_bf16_to_f32(recv[(size_t)row * H + i]);
        y[(size_t)row * H + i] = oracle_f32_to_bf16(p);
      }
    }
}

void oracle_expert_scale_fp8(const uint8_t *recv, const float *recv_scales,
                             const int32_t *ids, const int32_t *token_row,
                             int T, int k, int H, const float *alpha,
                             uint8_t *y, float *y_scales) {
  int nb = H / 128;
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int32_t row = token_row[(size_t)t * k + j];
      if (row < 0) continue;
      float a = alpha[ids[(size_t)t * k + j]];
      memcpy(y + (size_t)row * H, recv + (size_t)row * H, (size_t)H);
      for (int b = 0; b < nb; ++b)
        y_scales[(size_t)row * nb + b] = recv_scales[(size_t)row * nb + b] * a;
    }
}

/* ------------------------------------------------------------------------ */
/* Combine (EFA page, Introduction: the processed rows come back and their  */
/* weighted average is formed; Evaluation: the accumulation happens on the  */
/* receiving side only).                                                    */
/* ------------------------------------------------------------------------ */
static double oracle_payload_f64(const void *y, const float *y_scales,
                                 int32_t row, int H, int i) {
  if (!y_scales) return (double)oracle_bf16_to_f32(((const uint16_t *)y)[(size_t)row * H + i]);
  uint8_t c = ((const uint8_t *)y)[(size_t)row * H + i];
  return (double)oracle_e4m3_to_f32(c) * (double)y_scales[(size_t)row * (H / 128) + i / 128];
}

void oracle_combine_exact(const void *y, const float *y_scales,
                          const int32_t *token_row, const float *w, int T,
                          int k, int H, uint16_t *out) {
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < H; ++i) {
      double acc = 0.0;
      for (int j = 0; j < k; ++j) {
        int32_t row = token_row[(size_t)t * k + j];
        if (row < 0) continue;
        acc += (double)w[(size_t)t * k + j] * oracle_payload_f64(y, y_scales, row, H, i);
      }
      out[(size_t)t * H + i] = oracle_f64_to_bf16(acc);
    }
}

void oracle_combine_f32_ordered(const void *y, const float *y_scales,
                                const int32_t *token_row, const float *w,
                                int T, int k, int H, uint16_t *out) {
  for (int t = 0; t < T; ++t)
    for (int i = 0; i < H; ++i) {
      float acc = 0.0f;
      for (int j = 0; j < k; ++j) {
        int32_t row = token_row[(size_t)t * k + j];
        if (row < 0) continue;
        float v;
        if (!y_scales) {
          v = oracle_bf16_to_f32(((const uint16_t *)y)[(size_t)row * H + i]);
        } else {
          uint8_t c = ((const uint8_t *)y)[(size_t)row * H + i];
          v = oracle_e4m3_to_f32(c) * y_scales[(size_t)row * (H / 128) + i / 128];
        }
        acc = fmaf(w[(size_t)t * k + j], v, acc);
      }
      out[(size_t)t * H + i] = oracle_f32_to_bf16(acc);
    }
}

/* ------------------------------------------------------------------------ */
/* Sender-side partial reduction (EFA page, Evaluation: the alternative of   */
/* accumulating on the sender reduces the data transferred, with possible    */
/* precision implications).  Each destination rank first sums a token's      */
/* rows for its own experts into one bf16 row per (token, rank); the origin  */
/* then sums those rows.                                                     */
/* ------------------------------------------------------------------------ */
void oracle_combine_send(const void *y, const float *y_scales,
                         const int32_t *token_row, const int32_t *ids,
                         const float *w, int T, int k, int H, int E, int N,
                         int M, int exact, uint16_t *partial,
                         int32_t *partial_rank) {
  const int L = E / N;
  for (int t = 0; t < T; ++t) {
    /* distinct ranks of the placed pairs, ascending */
    int m = 0;
    for (int r = 0; r < N; ++r) {
      int hit = 0;
      for (int j = 0; j < k; ++j) {
        size_t p = (size_t)t * k + j;
        if (token_row[p] >= 0 && ids[p] >= 0 && ids[p] < E && ids[p] / L == r) hit = 1;
      }
      if (hit) partial_rank[(size_t)t * M + m++] = r;
    }
    for (int i = m; i < M; ++i) partial_rank[(size_t)t * M + i] = -1;
    for (int i = 0; i < m; ++i) {
      const int r = partial_rank[(size_t)t * M + i];
      uint16_t *dst = partial + ((size_t)t * M + i) * H;
      for (int c = 0; c < H; ++c) {
        double accd = 0.0;
        float accf = 0.0f;
        for (int j = 0; j < k; ++j) {
          size_t p = (size_t)t * k + j;
          int32_t row = token_row[p];
          if (row < 0 || ids[p] < 0 || ids[p] >= E || ids[p] / L != r) continue;
          if (exact) {
            accd += (double)w[p] * oracle_payload_f64(y, y_scales, row, H, c);
          } else {
            float v;
            if (!y_scales) {
              v = oracle_bf16_to_f32(((const uint16_t *)y)[(size_t)row * H + c]);
            } else {
              uint8_t code = ((const uint8_t *)y)[(size_t)row * H + c];
              v = oracle_e4m3_to_f32(code) * y_scales[(size_t)row * (H / 128) + c / 128];
            }
            accf = fmaf(w[p], v, accf);
          }
        }
        dst[c] = exact ? oracle_f64_to_bf16(accd) : oracle_f32_to_bf16(accf);
      }
    }
  }
}

void oracle_combine_recv(const uint16_t *partial, const int32_t *partial_rank,
                         int T, int M, int H, int exact, uint16_t *out) {
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < H; ++c) {
      double accd = 0.0;
      float accf = 0.0f;
      for (int i = 0; i < M; ++i) {
        if (partial_rank[(size_t)t * M + i] < 0) continue;
        float v = oracle_bf16_to_f32(partial[((size_t)t * M + i) * H + c]);
        accd += (double)v;
        accf = accf + v;
      }
      out[(size_t)t * H + c] = exact ? oracle_f64_to_bf16(accd) : oracle_f32_to_bf16(accf);
    }
}

/* ------------------------------------------------------------------------ */
/* Receive-side shuffle (EFA page, Dispatch and Combine: once everything has */
/* arrived, tokens are shuffled from the receive buffers into the tensor     */
/* passed to the grouped GEMM), and its inverse for the combine.             */
/* ------------------------------------------------------------------------ */
void oracle_gemm_io(int pack, const uint8_t *src, const float *src_scales,
                    uint8_t *dst, float *dst_scales, const int32_t *expert_counts,
                    const int32_t *expert_offsets, int E, int N, int C,
                    int row_bytes, int nb, int32_t *dense) {
  const int L = E / N;
  int32_t run = 0;
  for (int e = 0; e < E; ++e) {
    int32_t placed = expert_counts[e];
    if (C > 0) {
      int32_t room = (e / L) * C + C - expert_offsets[e];
      if (room < 0) room = 0;
      if (placed > room) placed = room;
    }
    dense[e] = run;
    for (int32_t i = 0; i < placed; ++i) {
      size_t region = (size_t)expert_offsets[e] + (size_t)i;
      size_t packed = (size_t)run + (size_t)i;
      size_t from = pack ? region : packed, to = pack ? packed : region;
      memcpy(dst + to * (size_t)row_bytes, src + from * (size_t)row_bytes, (size_t)row_bytes);
      if (src_scales)
        memcpy(dst_scales + to * (size_t)nb, src_scales + from * (size_t)nb, sizeof(float) * (size_t)nb);
    }
    run += placed;
  }
  dense[E] = run;
}
