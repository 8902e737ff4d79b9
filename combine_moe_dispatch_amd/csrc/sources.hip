// sources.hip -- every rank of the expert-parallel world dispatching at once.
//
// Before writing, the ranks exchange their per-expert token counts; then each
// knows where its writes go and at which offset it receives each rank's
// tokens ("Enabling trillion-parameter models on AWS EFA", Send and Receive
// Buffers).  With all S source ranks on this GPU, source s's tokens are the
// global tokens s*T .. s*T+T-1, so the receive layout ordered by (rank,
// expert, source, token, slot) is the dispatch layout over all S*T tokens.
// These kernels add the exchanged part: each source's count vector (written
// to HBM, the "exchange") and, per expert, the exclusive scan of the counts
// over sources, i.e. the row where each source's block of that expert begins.
// When the dispatch takes its multi-kernel path with chunks aligned to sources,
// its scatter launch reads both off the chunk bases instead (dispatch.hip).
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kIdsPerThread = 8;  // loads in flight per thread and round

// One block per source: LDS histogram of its T*k ids -> source_counts[s][:].
__global__ void __launch_bounds__(kBlock)
source_counts_kernel(const int32_t* __restrict__ ids, int pairs_per_source, int E,
                     int32_t* __restrict__ source_counts) {
  __shared__ int hist[kMaxExperts];
  const int s = blockIdx.x;
  for (int e = threadIdx.x; e < E; e += kBlock) hist[e] = 0;
  __syncthreads();
  const int32_t* src = ids + (size_t)s * pairs_per_source;
  for (int q0 = 0; q0 < pairs_per_source; q0 += kBlock * kIdsPerThread) {
    int v[kIdsPerThread];
#pragma unroll
    for (int i = 0; i < kIdsPerThread; ++i) {
      const int q = q0 + i * kBlock + threadIdx.x;
      v[i] = q < pairs_per_source ? src[q] : -1;
    }
#pragma unroll
    for (int i = 0; i < kIdsPerThread; ++i)
      if ((unsigned)v[i] < (unsigned)E) atomicAdd(&hist[v[i]], 1);
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kBlock) source_counts[(size_t)s * E + e] = hist[e];
}

// One wave per expert, lanes over sources: source_offsets[e][s] =
// expert_offsets[e] + sum of source_counts[s'][e] over s' < s, 64 sources per
// DPP scan.
constexpr int kWavesPerBlock = kBlock / kWave;

__global__ void __launch_bounds__(kBlock)
source_offsets_kernel(const int32_t* __restrict__ source_counts,
                      const int32_t* __restrict__ expert_offsets, int S, int E,
                      int32_t* __restrict__ source_offsets) {
  const int e = blockIdx.x * kWavesPerBlock + threadIdx.x / kWave;
  if (e >= E) return;  // whole wave
  const int lane = lane_id();
  int run = expert_offsets[e];
  for (int s0 = 0; s0 < S; s0 += kWave) {
    const int s = s0 + lane;
    const int c = s < S ? source_counts[(size_t)s * E + e] : 0;
    const int incl = wave_inclusive_sum_dpp(c);
    if (s < S) source_offsets[(size_t)e * S + s] = run + incl - c;
    run += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
}

}  // namespace

hipError_t launch_source_metadata(const int32_t* ids, int S, int T, int k, int E,
                                  const int32_t* expert_offsets, int32_t* source_counts,
                                  int32_t* source_offsets, hipStream_t st) {
  hipLaunchKernelGGL(source_counts_kernel, dim3(S), dim3(kBlock), 0, st, ids, T * k, E,
                     source_counts);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  hipLaunchKernelGGL(source_offsets_kernel, dim3((E + kWavesPerBlock - 1) / kWavesPerBlock),
                     dim3(kBlock), 0, st, source_counts, expert_offsets, S, E, source_offsets);
  return hipGetLastError();
}

}  // namespace moe
