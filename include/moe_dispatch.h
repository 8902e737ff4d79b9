/*
 * moe_dispatch.h -- C ABI of libmoe_dispatch.so: Mixture-of-Experts routing,
 * dispatch and combine on one AMD MI355X (gfx950), hand-written HIP kernels.
 *
 * The problem statement these calls follow comes from two pages:
 *   [EFA]  "Enabling trillion-parameter models on AWS EFA" (Perplexity, 2025)
 *   [DSK]  "Lower Latency and Higher Throughput with Multi-Node DeepSeek
 *          Deployment" (Perplexity)
 * A dispatch kernel splits the incoming tokens and sends each one to the ranks
 * hosting its experts; its dual, the combine kernel, receives the processed
 * rows and forms their weighted average ([EFA] Introduction).  Dispatch counts
 * tokens per expert, takes a cumulative sum of the counts and packs the tokens
 * into contiguous per-rank regions at the resulting offsets ([EFA] Send and
 * Receive Buffers; Dispatch and Combine).
 *
 * One GPU's share: this GPU is one source rank holding T tokens.  The N
 * expert-parallel destination ranks are virtual: their receive regions all
 * live in this GPU's memory, so a "send" is a store into the region of the
 * destination rank.  Expert e is hosted by rank e / L, L = E / N.
 *
 * Conventions common to every call
 *  - Every pointer is a DEVICE pointer unless marked "host".  The caller
 *    allocates and owns all memory; the library allocates nothing, keeps no
 *    state between calls, and is safe to call from several host threads.
 *    The one exception is moe_dispatch_static, whose scratch is a fixed array
 *    the library holds in each GPU's memory (see there).
 *  - Every call enqueues its kernels on `stream` and returns without waiting;
 *    no call copies anything device-to-host, so the sequence route -> dispatch
 *    -> combine can be captured in a HIP graph.  Buffers must stay valid until
 *    the stream has passed the call.
 *  - Arrays are dense row-major.  bf16 rows hold H values (2H bytes); fp8 rows
 *    hold H e4m3 codes (H bytes) plus H/128 fp32 scales in a separate array.
 *    Token, receive and output buffers must be 16-byte aligned.
 *  - Host-detectable errors (null pointers, bad sizes, misalignment) return
 *    MOE_ERR_INVALID_ARG or MOE_ERR_UNSUPPORTED and launch nothing.  A failed
 *    launch returns MOE_ERR_HIP.  Errors that depend on device data are
 *    reported in the layout's status word (MOE_DEV_* bits) and the affected
 *    pairs are skipped, deterministically.
 */
#ifndef MOE_DISPATCH_H
#define MOE_DISPATCH_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned buffer */
  MOE_ERR_UNSUPPORTED = 2, /* valid in principle, outside this library's limits */
  MOE_ERR_HIP = 3          /* a kernel launch failed */
} moe_status;

typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score;

typedef enum {
  MOE_PAYLOAD_BF16 = 0,          /* rows copied as bf16 */
  MOE_PAYLOAD_FP8_E4M3_B128 = 1  /* rows quantised to OCP e4m3fn, one fp32 scale per 128 columns */
} moe_payload;

/* bits of moe_layout.status */
#define MOE_DEV_CAPACITY 1 /* some pair did not fit its rank's capacity and was skipped */
#define MOE_DEV_BAD_ID 2   /* some expert id was outside [0, E) and its pair was skipped */

/* Limits of this library. */
#define MOE_MAX_EXPERTS 1024
#define MOE_MAX_TOP_K 32
#define MOE_MAX_GROUPS 64

/* Sizes of one dispatch/combine problem (host struct, read during the call). */
typedef struct {
  int32_t num_tokens;    /* T >= 0 tokens on this source rank; any T per call, no padding */
  int32_t hidden;        /* H > 0; bf16 payload: H % 8 == 0; fp8 payload: H % 128 == 0 */
  int32_t num_experts;   /* E, 1 <= E <= MOE_MAX_EXPERTS */
  int32_t top_k;         /* k, 1 <= k <= min(E, MOE_MAX_TOP_K) */
  int32_t num_ranks;     /* N >= 1 expert-parallel ranks, E % N == 0 */
  int32_t rank_capacity; /* C > 0: rank r owns receive rows [r*C, r*C + C);
                            C == 0: packed regions, back to back, sized by the counts */
  int32_t payload;       /* moe_payload */
} moe_shape;

/* Routing metadata, written by moe_dispatch and read by moe_combine and by
 * whatever consumes the receive buffer (the per-expert segments are the input
 * of a grouped GEMM).  All arrays are caller-owned device int32 arrays. */
typedef struct {
  int32_t *expert_counts;  /* [E] pairs routed to expert e (true counts, also on overflow) */
  int32_t *expert_offsets; /* [E] first receive row of expert e's segment */
  int32_t *rank_counts;    /* [N] pairs routed to rank r */
  int32_t *rank_offsets;   /* [N] first receive row of rank r's region */
  int32_t *token_row;      /* [T*k] receive row of pair (t, j), or -1 if skipped */
  int32_t *row_src;        /* [rows] optional (NULL = not written): t*k + j of the pair that
                              filled each row; rows that receive no pair are left untouched */
  int32_t *status;         /* [1] MOE_DEV_* bits of the last dispatch (overwritten, not OR-ed) */
} moe_layout;

/* Number of receive rows a problem addresses: N*C, or T*k when packed.
 * Returns -1 for a null or inconsistent shape.  Host function. */
int64_t moe_recv_rows(const moe_shape *shape);

/* Bytes of device workspace moe_dispatch needs for this shape (0 when the
 * single-kernel path applies).  Returns 0 for an invalid shape.  Host function. */
size_t moe_dispatch_workspace_size(const moe_shape *shape);

/*
 * moe_route_topk -- the router's top-k selection ([EFA] Introduction: a small
 * linear router decides which experts each token is multiplied with; [DSK] MoE
 * Router: the sparse kernels consume the top-k indices and scores).
 *
 *   logits        [T][E] fp32 router logits.  Must be finite.
 *   bias          [E] fp32 added to every token's logits before selection and
 *                 weighting, or NULL.
 *   T, E, k       0 <= T; 1 <= E <= MOE_MAX_EXPERTS; 1 <= k <= min(E, MOE_MAX_TOP_K).
 *   score         MOE_SCORE_SIGMOID: w_j = sigmoid(l_j) / sum_i sigmoid(l_i);
 *                 MOE_SCORE_SOFTMAX: w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0)
 *                 (the softmax over all E renormalised over the chosen k).
 *   topk_ids      [T][k] int32 out: the k largest biased logits, slot 0 the
 *                 largest; equal logits go to the lower expert id.
 *   topk_weights  [T][k] fp32 out: weights summing to one over the k slots.
 * Errors: MOE_ERR_INVALID_ARG for bad sizes or null pointers (T > 0).
 */
moe_status moe_route_topk(const float *logits, const float *bias, int32_t T,
                          int32_t E, int32_t k, int32_t score,
                          int32_t *topk_ids, float *topk_weights,
                          hipStream_t stream);

/*
 * moe_route_topk_grouped -- group-limited top-k ([DSK] MoE Router: one router
 * serves all MoE models; selecting among all experts is the special case in
 * which every group is kept).
 *
 *   Experts form n_groups contiguous groups of E/n_groups.  A group's score
 *   is the fp32 sum of its two largest biased logits (its only logit when a
 *   group holds one expert).  The topk_groups groups with the largest scores
 *   are kept (equal scores go to the lower group id); the top-k is then taken
 *   over the kept groups' experts with the ordering and weights of
 *   moe_route_topk.  n_groups == 1 or topk_groups == n_groups is exactly
 *   moe_route_topk.
 *   Other arguments as for moe_route_topk.
 * Errors: MOE_ERR_INVALID_ARG unless E % n_groups == 0, 1 <= topk_groups <=
 * n_groups and k <= topk_groups * (E / n_groups); MOE_ERR_UNSUPPORTED for
 * n_groups > MOE_MAX_GROUPS.
 */
moe_status moe_route_topk_grouped(const float *logits, const float *bias, int32_t T,
                                  int32_t E, int32_t k, int32_t score, int32_t n_groups,
                                  int32_t topk_groups, int32_t *topk_ids,
                                  float *topk_weights, hipStream_t stream);

/*
 * moe_dispatch -- count, scan, place and scatter ([EFA] Send and Receive
 * Buffers; Dispatch and Combine; block-scaled fp8 dispatch: [EFA] Evaluation
 * and [DSK] Quantization).
 *
 *   x             [T][H] bf16 tokens of this source rank.
 *   topk_ids      [T][k] int32 expert ids (moe_route_topk's output, or any
 *                 ids; duplicates in one token are separate pairs).
 *   recv_x        [rows][H] receive buffer, rows = moe_recv_rows(shape):
 *                 bf16 rows, or e4m3 codes for the fp8 payload.  Rank r's
 *                 region starts at rank_offsets[r]; inside it expert segments
 *                 follow in ascending expert order, and inside a segment the
 *                 pairs follow in ascending (token, slot) order.  Pair (t, j)
 *                 lands in row token_row[t*k + j].  Rows no pair reaches are
 *                 not written.
 *   recv_scales   [rows][H/128] fp32 scales for the fp8 payload (NULL for bf16):
 *                 per block of 128 columns, scale = amax/448 and
 *                 code = e4m3(x/scale), both IEEE fp32 divisions, ties to even;
 *                 an all-zero block gets scale 0 and codes 0.
 *   layout        metadata out (see moe_layout); all fields but row_src required.
 *   workspace     device scratch of moe_dispatch_workspace_size(shape) bytes
 *                 (NULL when that is 0); contents need no initialisation.
 * Data-dependent errors: an id outside [0, E) sets MOE_DEV_BAD_ID; with C > 0,
 * pairs past a rank's C rows (the last ones in that rank's order) set
 * MOE_DEV_CAPACITY.  Either way the pair gets token_row = -1 and no row.
 */
moe_status moe_dispatch(const moe_shape *shape, const void *x,
                        const int32_t *topk_ids, void *recv_x,
                        float *recv_scales, const moe_layout *layout,
                        void *workspace, size_t workspace_bytes,
                        hipStream_t stream);

/*
 * moe_dispatch_static -- moe_dispatch for callers that cannot allocate device
 * memory (code under stream capture, tight serving loops, harnesses that
 * forbid allocation): the same arguments without the workspace.
 *
 *   Where moe_dispatch needs a workspace (moe_dispatch_workspace_size > 0),
 *   this call uses a scratch array of MOE_STATIC_SCRATCH_BYTES that the
 *   library holds in each GPU's memory from the first such call on that GPU
 *   until the process ends.  It calls no allocating routine.  The current
 *   device must be the stream's device.
 *   Every call on one GPU shares that GPU's array: calls that may overlap on
 *   one GPU (several streams, or several host threads) race and must be
 *   ordered by the caller.  Nothing in the array needs clearing between calls.
 * Errors as moe_dispatch; MOE_ERR_UNSUPPORTED (nothing launched) when the
 * shape needs more than MOE_STATIC_SCRATCH_BYTES of workspace.
 */
#define MOE_STATIC_SCRATCH_BYTES (4u << 20)
moe_status moe_dispatch_static(const moe_shape *shape, const void *x,
                               const int32_t *topk_ids, void *recv_x,
                               float *recv_scales, const moe_layout *layout,
                               hipStream_t stream);

/*
 * moe_dispatch_sources -- every rank of the expert-parallel world dispatching
 * at once ([EFA] Send and Receive Buffers: ranks first exchange per-expert
 * token counts, after which each knows where its writes go and at which
 * offset it receives every rank's tokens).
 *
 *   shape         sizes of ONE source: num_tokens = T tokens per source; the
 *                 rank capacity C (or packed regions, C == 0) covers the rows
 *                 of all sources together.
 *   num_sources   S >= 1 source ranks, all on this GPU.
 *   x, topk_ids   [S][T][H] bf16 and [S][T][k] int32: source s's tokens are
 *                 the global tokens s*T .. s*T+T-1.
 *   recv_x, recv_scales, layout, workspace
 *                 exactly as moe_dispatch for S*T tokens (size the receive
 *                 buffer with moe_recv_rows and the workspace with
 *                 moe_dispatch_workspace_size on num_tokens = S*T); inside
 *                 each expert segment the pairs are in (source, token, slot)
 *                 order; layout->token_row is [S*T*k].
 *   source_counts [S][E] int32 out: pairs of source s routed to expert e (the
 *                 count vectors the ranks exchange).
 *   source_offsets [E][S] int32 out: first receive row of source s's block in
 *                 expert e's segment (expert_offsets[e] plus the counts of the
 *                 earlier sources); rows of pairs skipped for capacity are not
 *                 written.
 * The combine of the world is moe_combine with num_tokens = S*T.
 * Errors as moe_dispatch; MOE_ERR_INVALID_ARG for S < 1 or null count arrays.
 */
moe_status moe_dispatch_sources(const moe_shape *shape, int32_t num_sources,
                                const void *x, const int32_t *topk_ids, void *recv_x,
                                float *recv_scales, const moe_layout *layout,
                                int32_t *source_counts, int32_t *source_offsets,
                                void *workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * moe_dispatch_recv -- the receive half of dispatch: shuffle the tokens out of
 * the receive regions into the tensor handed to the experts' grouped GEMM
 * ([EFA] Dispatch and Combine: once all transfers are in, tokens are shuffled
 * from the receive buffers into the grouped GEMM's input; [DSK] Quantization:
 * kernels size their work from the routing counts, not the buffer bounds).
 * moe_dispatch is the send half.
 *
 *   recv_x/recv_scales  as written by moe_dispatch (regions may have gaps).
 *   layout        expert_counts and expert_offsets are read.
 *   gemm_x        [T*k][H] dense rows out (bf16, or e4m3 codes), gemm_scales
 *                 [T*k][H/128] for fp8 (else NULL): expert e's placed rows at
 *                 [gemm_offsets[e], gemm_offsets[e+1]) in the order of its
 *                 segment; rows past gemm_offsets[E] are not written.
 *   gemm_offsets  [E+1] int32 out: exclusive prefix of the placed rows per
 *                 expert (a segment may be cut short by its rank's capacity).
 */
moe_status moe_dispatch_recv(const moe_shape *shape, const void *recv_x,
                             const float *recv_scales, const moe_layout *layout,
                             void *gemm_x, float *gemm_scales, int32_t *gemm_offsets,
                             hipStream_t stream);

/*
 * moe_combine_send -- the send half of the receiver-side combine: each
 * expert's output rows go from the dense grouped-GEMM output back to the
 * receive-region layout that moe_combine (the receive half) gathers from
 * ([EFA] Send and Receive Buffers: the combine copies the tokens back with
 * one write per peer).  The inverse of moe_dispatch_recv for the same layout.
 *
 *   gemm_y/gemm_scales  [T*k][H] dense rows as laid out by moe_dispatch_recv.
 *   expert_y/expert_scales  receive-region layout out; rows no pair occupies
 *                 are not written.
 */
moe_status moe_combine_send(const moe_shape *shape, const void *gemm_y,
                            const float *gemm_scales, const moe_layout *layout,
                            void *expert_y, float *expert_scales, hipStream_t stream);

/*
 * moe_expert_scale -- stand-in for the experts' grouped GEMM between dispatch
 * and combine ([EFA] MoE all-to-all over EFA): every row of expert e's segment
 * is multiplied by alpha[e].  It reads the per-expert counts and offsets from
 * device memory, as a grouped GEMM would ([DSK] Quantization: kernels read the
 * routing information instead of the buffer bounds).
 *   bf16: y = bf16(fp32(alpha[e]) * x), one fp32 multiply then ties-to-even.
 *   fp8:  the codes are copied and y_scales = fp32(recv_scales * alpha[e]).
 *   recv_x/recv_scales  as written by moe_dispatch; y/y_scales same layout.
 * Rows outside the placed segments are not written.
 */
moe_status moe_expert_scale(const moe_shape *shape, const void *recv_x,
                            const float *recv_scales, const moe_layout *layout,
                            const float *alpha, void *y, float *y_scales,
                            hipStream_t stream);

/*
 * moe_combine -- receiver-side weighted sum ([EFA] Introduction: combine
 * computes the weighted average of the processed tokens; Evaluation: the
 * accumulation happens on the receiving side only).
 *
 *   expert_y      processed rows in the receive layout (bf16, or e4m3 codes).
 *   expert_scales [rows][H/128] fp32 scales for the fp8 payload, else NULL.
 *   layout        only token_row is read.
 *   topk_weights  [T][k] fp32 router weights.
 *   out           [T][H] bf16: out[t] = bf16( sum_j w[t][j] * v_j ), the sum an
 *                 fp32 fused multiply-add chain over j = 0..k-1 starting at 0,
 *                 v_j the bf16 value or fp32(code) * scale (one fp32 multiply);
 *                 pairs with token_row -1 add nothing.
 */
moe_status moe_combine(const moe_shape *shape, const void *expert_y,
                       const float *expert_scales, const moe_layout *layout,
                       const float *topk_weights, void *out,
                       hipStream_t stream);

/*
 * moe_combine_partial_send / moe_combine_partial_recv -- combine with sender-side partial
 * reduction ([EFA] Evaluation: accumulating on the sender transfers less data,
 * with possible precision implications; the pages' own kernels accumulate on
 * the receiver only, which is moe_combine).
 *
 *   Let M = min(k, N).  For token t, the distinct ranks of its placed pairs
 *   (token_row >= 0, valid id) in ascending order r_0 < r_1 < ... < r_{m-1}
 *   own partial slots 0..m-1.
 *   send: partial [T][M][H] bf16 -- slot i = bf16(fp32 fused multiply-add
 *         chain over the pairs on rank r_i, in slot order, from 0; fp8 values
 *         are fp32(code) * scale); partial_rank [T][M] int32 -- r_i, or -1
 *         for slots i >= m, whose partial rows are not written.  Reads
 *         layout->token_row, topk_ids [T][k] and topk_weights [T][k].
 *   recv: out [T][H] bf16 = bf16(fp32 sum of the slots with partial_rank >= 0,
 *         in slot order, from 0).
 * With N == 1 the pair equals moe_combine.  Errors as moe_combine.
 */
moe_status moe_combine_partial_send(const moe_shape *shape, const void *expert_y,
                            const float *expert_scales, const moe_layout *layout,
                            const int32_t *topk_ids, const float *topk_weights,
                            void *partial, int32_t *partial_rank, hipStream_t stream);
moe_status moe_combine_partial_recv(const moe_shape *shape, const void *partial,
                            const int32_t *partial_rank, void *out, hipStream_t stream);

/* Static text for a status code.  Host function. */
const char *moe_status_string(moe_status status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_DISPATCH_H */
