// capi.hip -- the C ABI of libmoe_dispatch.so: argument checks, then launches
// on the caller's stream.  No allocation, no synchronisation, no state.
#include <string.h>

#include "moe_dispatch.h"
#include "launch.h"

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Validates a shape; on success fills L and the receive row count.
moe_status check_shape(const moe_shape* s, int* L, int64_t* rows) {
  if (!s) return MOE_ERR_INVALID_ARG;
  if (s->num_tokens < 0 || s->hidden <= 0 || s->num_experts < 1 || s->top_k < 1 ||
      s->num_ranks < 1 || s->rank_capacity < 0)
    return MOE_ERR_INVALID_ARG;
  if (s->payload != MOE_PAYLOAD_BF16 && s->payload != MOE_PAYLOAD_FP8_E4M3_B128)
    return MOE_ERR_INVALID_ARG;
  if (s->top_k > s->num_experts) return MOE_ERR_INVALID_ARG;
  if (s->num_experts % s->num_ranks != 0) return MOE_ERR_INVALID_ARG;
  if (s->num_experts > MOE_MAX_EXPERTS || s->top_k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
  if (s->payload == MOE_PAYLOAD_BF16 && s->hidden % 8 != 0) return MOE_ERR_INVALID_ARG;
  if (s->payload == MOE_PAYLOAD_FP8_E4M3_B128 && s->hidden % 128 != 0) return MOE_ERR_INVALID_ARG;
  const int64_t pairs = (int64_t)s->num_tokens * s->top_k;
  const int64_t r = s->rank_capacity > 0 ? (int64_t)s->num_ranks * s->rank_capacity : pairs;
  if (pairs > INT32_MAX || r > INT32_MAX) return MOE_ERR_UNSUPPORTED;  // rows are int32
  *L = s->num_experts / s->num_ranks;
  *rows = r;
  return MOE_OK;
}

// token_row may be NULL only when there are no tokens (an empty array).
moe_status check_layout(const moe_layout* lay, int32_t T) {
  if (!lay || !lay->expert_counts || !lay->expert_offsets || !lay->rank_counts ||
      !lay->rank_offsets || !lay->status || (T > 0 && !lay->token_row))
    return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

moe_status from_hip(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace

extern "C" {

int64_t moe_recv_rows(const moe_shape* shape) {
  int L;
  int64_t rows;
  if (check_shape(shape, &L, &rows) != MOE_OK) return -1;
  return rows;
}

size_t moe_dispatch_workspace_size(const moe_shape* shape) {
  int L;
  int64_t rows;
  if (check_shape(shape, &L, &rows) != MOE_OK) return 0;
  return moe::dispatch_workspace_bytes(shape->num_tokens, shape->top_k, shape->num_experts);
}

moe_status moe_route_topk(const float* logits, const float* bias, int32_t T, int32_t E,
                          int32_t k, int32_t score, int32_t* topk_ids, float* topk_weights,
                          hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || k > E) return MOE_ERR_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOP_K) return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * E > INT32_MAX * (int64_t)64) return MOE_ERR_UNSUPPORTED;
  return from_hip(moe::launch_route_topk(logits, bias, T, E, k, score, 1, 1, topk_ids,
                                         topk_weights, stream));
}

moe_status moe_route_topk_grouped(const float* logits, const float* bias, int32_t T, int32_t E,
                                  int32_t k, int32_t score, int32_t n_groups,
                                  int32_t topk_groups, int32_t* topk_ids, float* topk_weights,
                                  hipStream_t stream) {
  if (T < 0 || E < 1 || k < 1 || n_groups < 1 || topk_groups < 1 || topk_groups > n_groups)
    return MOE_ERR_INVALID_ARG;
  if (E % n_groups != 0 || k > topk_groups * (E / n_groups)) return MOE_ERR_INVALID_ARG;
  if (score != MOE_SCORE_SOFTMAX && score != MOE_SCORE_SIGMOID) return MOE_ERR_INVALID_ARG;
  if (E > MOE_MAX_EXPERTS || k > MOE_MAX_TOP_K || n_groups > MOE_MAX_GROUPS)
    return MOE_ERR_UNSUPPORTED;
  if (T > 0 && (!logits || !topk_ids || !topk_weights)) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_route_topk(logits, bias, T, E, k, score, n_groups, topk_groups,
                                         topk_ids, topk_weights, stream));
}

namespace {

// moe_dispatch, and with S > 0 the per-source metadata of moe_dispatch_sources
// written by the scatter launch of the multi-kernel path (the caller has
// checked that every chunk lies inside one source).
moe_status dispatch_impl(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                         void* recv_x, float* recv_scales, const moe_layout* layout,
                         void* workspace, size_t workspace_bytes, hipStream_t stream, int S,
                         int chunks_per_source, int32_t* source_counts,
                         int32_t* source_offsets) {
  int L;
  int64_t rows;
  moe_status st = check_shape(shape, &L, &rows);
  if (st != MOE_OK) return st;
  if ((st = check_layout(layout, shape->num_tokens)) != MOE_OK) return st;
  const bool fp8 = shape->payload == MOE_PAYLOAD_FP8_E4M3_B128;
  if (shape->num_tokens > 0) {
    if (!x || !topk_ids || !recv_x) return MOE_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(recv_x)) return MOE_ERR_INVALID_ARG;
    if (fp8 && !recv_scales) return MOE_ERR_INVALID_ARG;
  }
  const size_t need = moe::dispatch_workspace_bytes(shape->num_tokens, shape->top_k,
                                                    shape->num_experts);
  if (need > 0 && (!workspace || workspace_bytes < need || !aligned16(workspace)))
    return MOE_ERR_INVALID_ARG;

  moe::DispatchParams p{};
  p.x = x;
  p.ids = topk_ids;
  p.recv = recv_x;
  p.recv_scales = recv_scales;
  p.expert_counts = layout->expert_counts;
  p.expert_offsets = layout->expert_offsets;
  p.rank_counts = layout->rank_counts;
  p.rank_offsets = layout->rank_offsets;
  p.token_row = layout->token_row;
  p.row_src = layout->row_src;
  p.status = layout->status;
  p.workspace = workspace;
  p.T = shape->num_tokens;
  p.H = shape->hidden;
  p.E = shape->num_experts;
  p.k = shape->top_k;
  p.N = shape->num_ranks;
  p.L = L;
  p.C = shape->rank_capacity;
  p.payload = fp8 ? 1 : 0;
  p.src_S = S;
  p.src_cps = chunks_per_source;
  p.src_counts = source_counts;
  p.src_offsets = source_offsets;
  return from_hip(moe::launch_dispatch(p, stream));
}

}  // namespace

moe_status moe_dispatch(const moe_shape* shape, const void* x, const int32_t* topk_ids,
                        void* recv_x, float* recv_scales, const moe_layout* layout,
                        void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return dispatch_impl(shape, x, topk_ids, recv_x, recv_scales, layout, workspace,
                       workspace_bytes, stream, 0, 0, nullptr, nullptr);
}

moe_status moe_dispatch_sources(const moe_shape* shape, int32_t num_sources, const void* x,
                                const int32_t* topk_ids, void* recv_x, float* recv_scales,
                                const moe_layout* layout, int32_t* source_counts,
                                int32_t* source_offsets, void* workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  if (!shape || num_sources < 1) return MOE_ERR_INVALID_ARG;
  const int64_t total = (int64_t)num_sources * shape->num_tokens;
  if (total > INT32_MAX) return MOE_ERR_UNSUPPORTED;
  moe_shape world = *shape;
  world.num_tokens = (int32_t)total;
  int L;
  int64_t rows;
  moe_status st = check_shape(&world, &L, &rows);
  if (st != MOE_OK) return st;
  if (!source_counts || !source_offsets) return MOE_ERR_INVALID_ARG;
  if (moe::dispatch_bases_per_source(num_sources, shape->num_tokens, shape->top_k))
    return dispatch_impl(&world, x, topk_ids, recv_x, recv_scales, layout, workspace,
                         workspace_bytes, stream, num_sources,
                         shape->num_tokens * shape->top_k / moe::kChunkPairs, source_counts,
                         source_offsets);
  st = moe_dispatch(&world, x, topk_ids, recv_x, recv_scales, layout, workspace, workspace_bytes,
                    stream);
  if (st != MOE_OK) return st;
  return from_hip(moe::launch_source_metadata(topk_ids, num_sources, shape->num_tokens,
                                              shape->top_k, shape->num_experts,
                                              layout->expert_offsets, source_counts,
                                              source_offsets, stream));
}

moe_status moe_expert_scale(const moe_shape* shape, const void* recv_x, const float* recv_scales,
                            const moe_layout* layout, const float* alpha, void* y,
                            float* y_scales, hipStream_t stream) {
  int L;
  int64_t rows;
  moe_status st = check_shape(shape, &L, &rows);
  if (st != MOE_OK) return st;
  if (!layout || !layout->expert_counts || !layout->expert_offsets) return MOE_ERR_INVALID_ARG;
  const bool fp8 = shape->payload == MOE_PAYLOAD_FP8_E4M3_B128;
  if (!alpha) return MOE_ERR_INVALID_ARG;
  if (rows == 0) return MOE_OK;  // nothing can be placed
  if (!recv_x || !y || !aligned16(recv_x) || !aligned16(y)) return MOE_ERR_INVALID_ARG;
  if (fp8 && (!recv_scales || !y_scales)) return MOE_ERR_INVALID_ARG;
  return from_hip(moe::launch_expert_scale(recv_x, recv_scales, layout->expert_counts,
                                           layout->expert_offsets, alpha, y, y_scales,
                                           shape->num_experts, L, shape->rank_capacity,
                                           shape->hidden, fp8 ? 1 : 0, stream));
}

moe_status moe_combine(const moe_shape* shape, const void* expert_y, const float* expert_scales,
                       const moe_layout* layout, const float* topk_weights, void* out,
                       hipStream_t stream) {
  int L;
  int64_t rows;
  moe_status st = check_shape(shape, &L, &rows);
  if (st != MOE_OK) return st;
  const bool fp8 = shape->payload == MOE_PAYLOAD_FP8_E4M3_B128;
  if (shape->num_tokens > 0) {
    if (!layout || !layout->token_row || !expert_y || !topk_weights || !out)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(expert_y) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
    if (fp8 && !expert_scales) return MOE_ERR_INVALID_ARG;
  }
  return from_hip(moe::launch_combine(expert_y, expert_scales,
                                      layout ? layout->token_row : nullptr, topk_weights, out,
                                      shape->num_tokens, shape->hidden, shape->top_k,
                                      fp8 ? 1 : 0, stream));
}

moe_status moe_combine_partial_send(const moe_shape* shape, const void* expert_y,
                            const float* expert_scales, const moe_layout* layout,
                            const int32_t* topk_ids, const float* topk_weights, void* partial,
                            int32_t* partial_rank, hipStream_t stream) {
  int L;
  int64_t rows;
  moe_status st = check_shape(shape, &L, &rows);
  if (st != MOE_OK) return st;
  const bool fp8 = shape->payload == MOE_PAYLOAD_FP8_E4M3_B128;
  if (shape->num_tokens > 0) {
    if (!layout || !layout->token_row || !expert_y || !topk_ids || !topk_weights || !partial ||
        !partial_rank)
      return MOE_ERR_INVALID_ARG;
    if (!aligned16(expert_y) || !aligned16(partial)) return MOE_ERR_INVALID_ARG;
    if (fp8 && !expert_scales) return MOE_ERR_INVALID_ARG;
  }
  return from_hip(moe::launch_combine_send(
      expert_y, expert_scales, layout ? layout->token_row : nullptr, topk_ids, topk_weights,
      partial, partial_rank, shape->num_tokens, shape->hidden, shape->top_k,
      shape->num_experts, shape->num_ranks, fp8 ? 1 : 0, stream));
}

moe_status moe_combine_partial_recv(const moe_shape* shape, const void* partial,
                            const int32_t* partial_rank, void* out, hipStream_t stream) {
  int L;
  int64_t rows;
  moe_status st = check_shape(shape, &L, &rows);
  if (st != MOE_OK) return st;
  if (shape->num_tokens > 0) {
    if (!partial || !partial_rank || !out) return MOE_ERR_INVALID_ARG;
    if (!aligned16(partial) || !aligned16(out)) return MOE_ERR_INVALID_ARG;
  }
  const int M = shape->top_k < shape->num_ranks ? shape->top_k : shape->num_ranks;
  return from_hip(moe::launch_combine_recv(partial, partial_rank, out, shape->num_tokens,
                                           shape->hidden, M, stream));
}

namespace {

moe_status gemm_io(bool pack, const moe_shape* shape, const void* src, const float* src_scales,
                   const moe_layout* layout, void* dst, float* dst_scales, int32_t* gemm_offsets,
                   hipStream_t stream) {
  int L;
  int64_t rows;
  moe_status st = check_shape(shape, &L, &rows);
  if (st != MOE_OK) return st;
  const bool fp8 = shape->payload == MOE_PAYLOAD_FP8_E4M3_B128;
  if (!layout || !layout->expert_counts || !layout->expert_offsets || (pack && !gemm_offsets))
    return MOE_ERR_INVALID_ARG;
  const int64_t pairs = (int64_t)shape->num_tokens * shape->top_k;
  if (pairs > 0) {
    if (!src || !dst || !aligned16(src) || !aligned16(dst)) return MOE_ERR_INVALID_ARG;
    if (fp8 && (!src_scales || !dst_scales)) return MOE_ERR_INVALID_ARG;
  }
  return from_hip(moe::launch_gemm_io(pack, src, src_scales, dst, dst_scales,
                                      layout->expert_counts, layout->expert_offsets, gemm_offsets,
                                      (int)pairs, shape->num_experts, L, shape->rank_capacity,
                                      shape->hidden, fp8 ? 1 : 0, stream));
}

}  // namespace

moe_status moe_dispatch_recv(const moe_shape* shape, const void* recv_x, const float* recv_scales,
                             const moe_layout* layout, void* gemm_x, float* gemm_scales,
                             int32_t* gemm_offsets, hipStream_t stream) {
  return gemm_io(true, shape, recv_x, recv_scales, layout, gemm_x, gemm_scales, gemm_offsets,
                 stream);
}

moe_status moe_combine_send(const moe_shape* shape, const void* gemm_y, const float* gemm_scales,
                            const moe_layout* layout, void* expert_y, float* expert_scales,
                            hipStream_t stream) {
  // the dense offsets are rebuilt on the device from the layout's counts
  return gemm_io(false, shape, gemm_y, gemm_scales, layout, expert_y, expert_scales, nullptr,
                 stream);
}

const char* moe_status_string(moe_status status) {
  // A C caller may pass any int; in C++ a value outside the enumerators is
  // not a valid moe_status, so the bits are read as an int first.
  int code;
  static_assert(sizeof(code) == sizeof(status), "moe_status is int-sized");
  memcpy(&code, &status, sizeof(code));
  switch (code) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG: null pointer, bad size or misaligned buffer";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED: outside the library's limits";
    case MOE_ERR_HIP: return "MOE_ERR_HIP: a kernel launch failed";
  }
  return "unknown moe_status";
}

}  // extern "C"
