// gemm_io.hip -- the receive half of dispatch and the send half of combine.
//
// After the transfers land, the receiver shuffles the tokens from its receive
// buffers into the tensor handed to the experts' grouped GEMM; on the way
// back each expert's outputs go to the buffers the combine reads ("Enabling
// trillion-parameter models on AWS EFA", Dispatch and Combine; Send and
// Receive Buffers).  Here the receive regions may have gaps (fixed per-rank
// capacity), so the GEMM input is their dense, gap-free concatenation in
// expert order: expert e's placed rows occupy [dense[e], dense[e+1]), in the
// same (token, slot) order as its segment.  Work is sized from the per-expert
// counts in device memory, not from the buffers' bounds ("Lower Latency and
// Higher Throughput with Multi-Node DeepSeek Deployment", Quantization), so
// the calls need no host round trip and can be captured in a graph.
//
// Each block rebuilds dense[] in LDS (placed count per expert, then a scan),
// block 0 publishes it, and the block moves kRows dense rows: a binary search
// in LDS finds a row's expert, and the rows move as 16-byte streaming
// accesses, every load of a pass issued before its stores (fp8 rows carry
// their H/128 scales along).
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kRows = 4;  // dense rows per block

// dense[0..E]: exclusive scan of the placed rows per expert (a segment may be
// cut short by its rank's capacity).
// Also copies the segment offsets into off[0..E).
__device__ void dense_offsets(const int32_t* counts, const int32_t* offsets, int E, int L, int C,
                              int* dense, int* off, int* wave_tot) {
  const int per = (E + kBlock - 1) / kBlock;  // <= 4
  const int start = threadIdx.x * per;
  int cnt[4], o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {  // all loads first (clamped), one round trip
    const int e = min(start + i, E - 1);
    cnt[i] = counts[e];
    o[i] = offsets[e];
  }
  int placed[4];
  int local = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int e = start + i;
    int p = 0;
    if (i < per && e < E) {
      p = cnt[i];
      if (C > 0) p = max(0, min(p, (e / L) * C + C - o[i]));
      off[e] = o[i];
    }
    placed[i] = p;
    local += p;
  }
  const int incl = wave_inclusive_sum_dpp(local);
  const int w = threadIdx.x / kWave;
  if (lane_id() == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int run = incl - local;
  for (int i = 0; i < w; ++i) run += wave_tot[i];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < per && start + i < E) {
      dense[start + i] = run;
      run += placed[i];
    }
  }
  if (threadIdx.x == kBlock - 1) {
    int tot = 0;
    for (int i = 0; i < kBlock / kWave; ++i) tot += wave_tot[i];
    dense[E] = tot;
  }
  __syncthreads();
}

// Largest e with dense[e] <= i (dense is non-decreasing, dense[0] = 0).
__device__ __forceinline__ int find_expert(const int* dense, int E, int i) {
  int lo = 0, hi = E;  // answer in [lo, hi)
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (dense[mid] <= i)
      lo = mid;
    else
      hi = mid;
  }
  return lo;
}

constexpr int kVecsPerThread = 4;  // 16-byte vectors of one row per thread and pass

// PACK: receive regions -> dense rows; otherwise dense rows -> regions.  The
// block's kRows rows are located first (binary search in LDS), then each pass
// issues every load of those rows before the first store.
template <bool PACK>
__global__ void __launch_bounds__(kBlock)
gemm_io_kernel(const uint8_t* __restrict__ src, const float* __restrict__ src_scales,
               uint8_t* __restrict__ dst, float* __restrict__ dst_scales,
               const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
               int32_t* __restrict__ dense_out, int E, int L, int C, int row_bytes, int nb) {
  __shared__ int s_dense[kMaxExperts + 1];
  __shared__ int s_off[kMaxExperts];
  __shared__ int s_wave[kBlock / kWave];
  dense_offsets(counts, offsets, E, L, C, s_dense, s_off, s_wave);
  if (PACK && blockIdx.x == 0)
    for (int e = threadIdx.x; e <= E; e += kBlock) dense_out[e] = s_dense[e];
  const int total = s_dense[E];
  const int nvec = row_bytes / 16;
  bool ok[kRows];
  size_t from[kRows], to[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int i = blockIdx.x * kRows + r;
    ok[r] = i < total;  // uniform
    const int e = ok[r] ? find_expert(s_dense, E, i) : 0;
    const size_t region_row = (size_t)(s_off[e] + (i - s_dense[e]));
    from[r] = PACK ? region_row : (size_t)i;
    to[r] = PACK ? (size_t)i : region_row;
  }
  for (int v0 = 0; v0 < nvec; v0 += kVecsPerThread * kBlock) {
    uint4 buf[kRows][kVecsPerThread];
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const uint4* s4 = reinterpret_cast<const uint4*>(src + from[r] * row_bytes);
#pragma unroll
      for (int j = 0; j < kVecsPerThread; ++j) {
        const int v = v0 + j * kBlock + threadIdx.x;
        buf[r][j] = ok[r] && v < nvec ? load_stream(&s4[v]) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      uint4* d4 = reinterpret_cast<uint4*>(dst + to[r] * row_bytes);
#pragma unroll
      for (int j = 0; j < kVecsPerThread; ++j) {
        const int v = v0 + j * kBlock + threadIdx.x;
        if (ok[r] && v < nvec) store_stream(&d4[v], buf[r][j]);
      }
    }
  }
  if (src_scales) {
    for (int b0 = 0; b0 < nb; b0 += kBlock) {
      float sc[kRows];
      const int b = b0 + threadIdx.x;
#pragma unroll
      for (int r = 0; r < kRows; ++r) sc[r] = ok[r] && b < nb ? src_scales[from[r] * nb + b] : 0.0f;
#pragma unroll
      for (int r = 0; r < kRows; ++r)
        if (ok[r] && b < nb) dst_scales[to[r] * nb + b] = sc[r];
    }
  }
}

}  // namespace

hipError_t launch_gemm_io(bool pack, const void* src, const float* src_scales, void* dst,
                          float* dst_scales, const int32_t* counts, const int32_t* offsets,
                          int32_t* dense_out, int max_rows, int E, int L, int C, int H,
                          int payload, hipStream_t st) {
  const int row_bytes = payload == 0 ? 2 * H : H;
  const int nb = payload == 0 ? 0 : H / kFp8Block;
  const unsigned blocks = (unsigned)max(1, (max_rows + kRows - 1) / kRows);
  const uint8_t* s = reinterpret_cast<const uint8_t*>(src);
  uint8_t* d = reinterpret_cast<uint8_t*>(dst);
  if (pack)
    hipLaunchKernelGGL((gemm_io_kernel<true>), dim3(blocks), dim3(kBlock), 0, st, s,
                       payload ? src_scales : nullptr, d, dst_scales, counts, offsets, dense_out,
                       E, L, C, row_bytes, nb);
  else
    hipLaunchKernelGGL((gemm_io_kernel<false>), dim3(blocks), dim3(kBlock), 0, st, s,
                       payload ? src_scales : nullptr, d, dst_scales, counts, offsets, dense_out,
                       E, L, C, row_bytes, nb);
  return hipGetLastError();
}

}  // namespace moe
