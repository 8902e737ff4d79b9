/*
 * moe_oracle.h -- plain, slow, single-threaded CPU oracle for MoE dispatch
 * and combine.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the
 * benchmark's CPU-baseline leg are its only users.  It shares no code, header,
 * constant or helper with the HIP library under combine_moe_dispatch_amd/.
 *
 * What is computed, and where the pages state it:
 *  - routing: a small linear router picks experts per token ("Enabling
 *    trillion-parameter models on AWS EFA", Introduction); the router emits
 *    top-k indices and scores ("Lower Latency and Higher Throughput with
 *    Multi-Node DeepSeek Deployment", section MoE Router).
 *  - layout: per-expert token counts, a cumulative sum of them giving the
 *    offsets of contiguous per-peer regions ("Enabling trillion-parameter
 *    models on AWS EFA", sections Send and Receive Buffers, Dispatch and
 *    Combine).
 *  - dispatch: each token row is sent to the ranks hosting its experts (same
 *    page, Introduction and MoE all-to-all over EFA); block-scaled fp8 rows
 *    (same page, Evaluation) with one dynamic scale per 128-element activation
 *    vector (DeepSeek-deployment page, section Quantization).
 *  - combine: the processed rows come back and their weighted average is
 *    formed on the receiving side (EFA page, Introduction, Send and Receive
 *    Buffers, Dispatch and Combine, Evaluation).
 *
 * Conventions the pages leave open are fixed here and listed with their
 * reasons in the design notes: contiguous expert->rank blocks, expert-ascending
 * then (token, slot)-ascending order inside a rank region, ties to the lower
 * expert id, round-to-nearest-even for bf16 and OCP e4m3fn (saturating) for fp8.
 *
 * All arrays are host arrays, row-major, owned by the caller.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status bits written by oracle_layout */
#define ORACLE_ST_CAPACITY 1 /* a pair did not fit its rank's capacity */
#define ORACLE_ST_BAD_ID 2   /* an expert id outside [0, E) */

/* score functions for oracle_route_topk */
#define ORACLE_SCORE_SOFTMAX 0
#define ORACLE_SCORE_SIGMOID 1

/* --- scalar codecs -------------------------------------------------------- */
uint16_t oracle_f32_to_bf16(float v);  /* round to nearest, ties to even */
float oracle_bf16_to_f32(uint16_t b);
uint16_t oracle_f64_to_bf16(double v); /* one rounding, ties to even */
uint8_t oracle_f32_to_e4m3(float v);   /* OCP e4m3fn, RNE, saturating */
float oracle_e4m3_to_f32(uint8_t c);

/* --- steps of the path ---------------------------------------------------- */

/* Top-k routing.  logits [T][E] fp32; bias [E] or NULL.  Writes ids [T][k]
 * and weights [T][k].  Returns 0, or -1 on bad arguments. */
int oracle_route_topk(const float *logits, const float *bias, int T, int E,
                      int k, int score, int32_t *ids, float *weights);

/* Group-limited top-k: experts form n_groups contiguous groups of E/n_groups;
 * a group's score is the fp32 sum of its two largest biased logits (its only
 * logit when a group has one expert); the topk_groups best groups are kept
 * (ties to the lower group id) and the top-k is taken over their experts only,
 * with the same ordering and weights as oracle_route_topk.  n_groups == 1
 * reduces to oracle_route_topk.  Returns 0, or -1 on bad arguments. */
int oracle_route_topk_grouped(const float *logits, const float *bias, int T,
                              int E, int k, int score, int n_groups,
                              int topk_groups, int32_t *ids, float *weights);

/* Layout: counts, offsets and the destination row of every (token, slot)
 * pair.  C > 0: rank r owns rows [r*C, r*C + C); C == 0: packed regions.
 * row_src may be NULL; otherwise it has `rows` entries and only rows that
 * receive a pair are written.  *status is OR-ed with ORACLE_ST_* bits.
 * Returns 0, or -1 on bad arguments. */
int oracle_layout(const int32_t *ids, int T, int k, int E, int N, int C,
                  int32_t *expert_counts, int32_t *expert_offsets,
                  int32_t *rank_counts, int32_t *rank_offsets,
                  int32_t *token_row, int32_t *row_src, int64_t rows,
                  int32_t *status);

/* Multi-source layout: S sources each hold T tokens (ids [S][T][k]); the
 * pairs of all sources are placed in (rank, expert, source, token, slot)
 * order, with the same capacity rule as oracle_layout (C counts rows per rank
 * across all sources).  token_row is [S*T*k].  Also writes source_counts
 * [S][E] (pairs of source s routed to expert e) and source_offsets [E][S]
 * (first row of source s's block inside expert e's segment). */
int oracle_layout_sources(const int32_t *ids, int S, int T, int k, int E, int N,
                          int C, int32_t *expert_counts,
                          int32_t *expert_offsets, int32_t *rank_counts,
                          int32_t *rank_offsets, int32_t *token_row,
                          int32_t *source_counts, int32_t *source_offsets,
                          int32_t *status);

/* bf16 dispatch: recv[token_row[t*k+j]] = x[t] for every placed pair. */
void oracle_dispatch_bf16(const uint16_t *x, int T, int H, int k,
                          const int32_t *token_row, uint16_t *recv);

/* Block-scaled fp8 quantisation of one bf16 row of H values (H % 128 == 0):
 * q [H] e4m3 codes, scales [H/128]. */
void oracle_quantize_row_fp8(const uint16_t *x, int H, uint8_t *q,
                             float *scales);

/* fp8 dispatch: quantise each token once, copy payload and scales to every
 * placed destination row. */
void oracle_dispatch_fp8(const uint16_t *x, int T, int H, int k,
                         const int32_t *token_row, uint8_t *recv,
                         float *recv_scales);

/* Expert stand-in (replaces the grouped GEMM): for every placed pair, the row
 * it landed in is scaled by alpha[e] of its expert.  bf16: y = bf16(fl32(a*x));
 * fp8: payload copied, scale' = fl32(scale * a). */
void oracle_expert_scale_bf16(const uint16_t *recv, const int32_t *ids,
                              const int32_t *token_row, int T, int k, int H,
                              const float *alpha, uint16_t *y);
void oracle_expert_scale_fp8(const uint8_t *recv, const float *recv_scales,
                             const int32_t *ids, const int32_t *token_row,
                             int T, int k, int H, const float *alpha,
                             uint8_t *y, float *y_scales);

/* Combine, exact form: out[t] = bf16( sum_j w[t][j] * y[token_row[t*k+j]] ),
 * the sum taken in double and rounded once.  Skipped pairs add nothing.
 * y_scales == NULL selects the bf16 payload; otherwise y is e4m3 codes. */
void oracle_combine_exact(const void *y, const float *y_scales,
                          const int32_t *token_row, const float *w, int T,
                          int k, int H, uint16_t *out);

/* Combine, fp32 form: acc = 0; acc = fmaf(w[t][j], v, acc) for j = 0..k-1 in
 * slot order; out = bf16(acc).  v = fp32(bf16) or fl32(fp32(q) * scale). */
void oracle_combine_f32_ordered(const void *y, const float *y_scales,
                                const int32_t *token_row, const float *w,
                                int T, int k, int H, uint16_t *out);

/* Receive-side shuffle into the grouped GEMM's input: expert e's placed rows
 * (its count, cut short by its rank's capacity when C > 0) are copied, in
 * segment order, to dense rows [dense[e], dense[e+1]); dense[] [E+1] is the
 * exclusive prefix of the placed counts.  row_bytes per row; scales (nb per
 * row) move along when non-NULL.  pack != 0: regions -> dense; pack == 0:
 * dense -> regions (the combine's send half). */
void oracle_gemm_io(int pack, const uint8_t *src, const float *src_scales,
                    uint8_t *dst, float *dst_scales, const int32_t *expert_counts,
                    const int32_t *expert_offsets, int E, int N, int C,
                    int row_bytes, int nb, int32_t *dense);

/* Sender-side partial reduction, stage 1: for token t, the distinct ranks of
 * its placed pairs in ascending order r_0 < r_1 < ... get partial slots
 * 0, 1, ... of M (M >= min(k, N)); slot i = bf16(sum over the pairs on rank
 * r_i, in slot order, of w * v) and partial_rank[t][i] = r_i; unused slots
 * get partial_rank -1 and their rows are left untouched.  exact != 0: the
 * sum in double, one rounding; exact == 0: the fp32 fused multiply-add chain
 * from 0.  partial is [T][M][H] bf16. */
void oracle_combine_send(const void *y, const float *y_scales,
                         const int32_t *token_row, const int32_t *ids,
                         const float *w, int T, int k, int H, int E, int N,
                         int M, int exact, uint16_t *partial,
                         int32_t *partial_rank);

/* Stage 2: out[t] = bf16(sum of the token's partial rows with rank >= 0, in
 * slot order): double then one rounding (exact != 0) or fp32 adds from 0. */
void oracle_combine_recv(const uint16_t *partial, const int32_t *partial_rank,
                         int T, int M, int H, int exact, uint16_t *out);

#ifdef __cplusplus
}
#endif

#endif
