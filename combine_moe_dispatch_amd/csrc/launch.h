// launch.h -- internal launchers of libmoe_dispatch.so (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Pairs up to which dispatch runs as one fused kernel: each block recounts
// the whole id list from LDS, which stays cheap while it is this short.
constexpr int kSmallMaxPairs = 8192;
// Pairs per chunk of the multi-kernel layout path.
constexpr int kChunkPairs = 1024;

struct DispatchParams {
  const void* x;
  const int32_t* ids;
  void* recv;
  float* recv_scales;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* rank_counts;
  int32_t* rank_offsets;
  int32_t* token_row;
  int32_t* row_src;
  int32_t* status;
  void* workspace;      // multi-kernel path: carved into the three arrays below
  int32_t* local_rank;  // [T*k] rank of a pair among equal experts in its chunk
  int32_t* chunk_hist;  // [nchunks][E] chunk histograms, then chunk bases
  int32_t* chunk_bad;   // [nchunks] chunk saw an id outside [0, E)
  int T, H, E, k, N, L, C;
  int rows;  // receive rows addressed: N*C, or T*k when packed
  int payload;
  int nchunks;
  int col_chunks;     // blocks per token in the scatter
  int vec_per_chunk;  // row units per block (8 columns bf16, 16 columns fp8)
  uint32_t l_magic;   // ceil(2^32 / L) for L >= 2: e / L == umulhi(e, l_magic) for e < 2^16
  uint32_t cc_magic;  // udiv_magic_of(col_chunks)
  // Sources dispatching at once (moe_dispatch_sources) on the multi-kernel
  // path, every chunk inside one source: src_blocks extra blocks at the end of
  // the scatter grid read the per-source metadata off the chunk bases (one
  // wave per expert).  src_blocks == 0 otherwise.
  int src_S;    // number of sources
  int src_cps;  // chunks per source
  int src_blocks;
  int32_t* src_counts;   // [S][E]
  int32_t* src_offsets;  // [E][S]
};

size_t dispatch_workspace_bytes(int T, int k, int E);
hipError_t launch_dispatch(const DispatchParams& p, hipStream_t st);

hipError_t launch_route_topk(const float* logits, const float* bias, int T, int E, int k,
                             int score, int n_groups, int topk_groups, int32_t* ids, float* w,
                             hipStream_t st);

// Multi-kernel dispatch over S sources of T tokens whose chunks each lie
// inside one source; its chunk bases then give the per-source metadata, which
// the scatter launch writes when DispatchParams::src_* are set.
bool dispatch_bases_per_source(int S, int T, int k);

hipError_t launch_source_metadata(const int32_t* ids, int S, int T, int k, int E,
                                  const int32_t* expert_offsets, int32_t* source_counts,
                                  int32_t* source_offsets, hipStream_t st);

hipError_t launch_combine(const void* y, const float* ys, const int32_t* token_row,
                          const float* w, void* out, int T, int H, int k, int payload,
                          hipStream_t st);

hipError_t launch_combine_send(const void* y, const float* ys, const int32_t* token_row,
                               const int32_t* ids, const float* w, void* partial,
                               int32_t* partial_rank, int T, int H, int k, int E, int N,
                               int payload, hipStream_t st);

hipError_t launch_combine_recv(const void* partial, const int32_t* partial_rank, void* out,
                               int T, int H, int M, hipStream_t st);

hipError_t launch_gemm_io(bool pack, const void* src, const float* src_scales, void* dst,
                          float* dst_scales, const int32_t* counts, const int32_t* offsets,
                          int32_t* dense_out, int max_rows, int E, int L, int C, int H,
                          int payload, hipStream_t st);

hipError_t launch_expert_scale(const void* recv, const float* recv_scales,
                               const int32_t* expert_counts, const int32_t* expert_offsets,
                               const float* alpha, void* y, float* y_scales, int E, int L,
                               int C, int H, int payload, hipStream_t st);

}  // namespace moe
