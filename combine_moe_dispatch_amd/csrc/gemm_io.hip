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
// One wave per block, no LDS and no barrier: every wave loads all experts'
// counts and segment offsets (PER consecutive experts per lane, as 16-byte
// loads where E is a multiple of 4), forms the
// dense offsets with a DPP scan, and finds the expert of each of its dense
// rows by a compare in every lane and a ballot.  Wave 0 publishes the dense
// offsets.  A row then moves as 16-byte streaming accesses, all loads of a
// pass (KV vectors per lane, indices clamped so none is conditional) issued
// before its stores; fp8 rows carry their H/128 scales along.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

// PACK: receive regions -> dense rows; otherwise dense rows -> regions.
// Block b moves dense row b.
template <bool PACK, int PER, int KV>
__global__ void __launch_bounds__(kWave)
gemm_io_kernel(const uint8_t* __restrict__ src, const float* __restrict__ src_scales,
               uint8_t* __restrict__ dst, float* __restrict__ dst_scales,
               const int32_t* __restrict__ counts, const int32_t* __restrict__ offsets,
               int32_t* __restrict__ dense_out, int E, int C, uint32_t l_magic, int row_bytes,
               int nb, int vec4) {
  const int lane = threadIdx.x;
  const int e0 = lane * PER;
  int cnt[PER], off[PER];
  // every load first (clamped): one round trip.  vec4 (E % 4 == 0, both
  // arrays 16-byte aligned): a lane's PER consecutive entries as 16-byte loads
  if (PER % 4 == 0 && vec4) {
    const int4* c4 = reinterpret_cast<const int4*>(counts);
    const int4* o4 = reinterpret_cast<const int4*>(offsets);
#pragma unroll
    for (int i = 0; i < PER / 4; ++i) {
      const int vi = min(lane * (PER / 4) + i, E / 4 - 1);
      const int4 c = c4[vi], o = o4[vi];
      cnt[4 * i] = c.x; cnt[4 * i + 1] = c.y; cnt[4 * i + 2] = c.z; cnt[4 * i + 3] = c.w;
      off[4 * i] = o.x; off[4 * i + 1] = o.y; off[4 * i + 2] = o.z; off[4 * i + 3] = o.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int e = min(e0 + i, E - 1);
      cnt[i] = counts[e];
      off[i] = offsets[e];
    }
  }
  // placed rows per expert: the count, cut at the end of the expert's rank
  // region for fixed capacity (rank = e / L by a multiply-high with
  // ceil(2^32 / L), exact for e * L < 2^32; l_magic = 0 means L = 1)
  int placed[PER];
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const uint32_t e = (uint32_t)(e0 + i);
    int pl = max(cnt[i], 0);
    if (C > 0) {
      const int r = (int)(l_magic ? __umulhi(e, l_magic) : e);
      pl = max(0, min(pl, (r + 1) * C - off[i]));
    }
    placed[i] = (int)e < E ? pl : 0;
    local += placed[i];
  }
  const int incl = wave_inclusive_sum_dpp(local);
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
  int dense[PER];
  {
    int run = incl - local;
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      dense[i] = run;
      run += placed[i];
    }
  }
  if (PACK && blockIdx.x == 0) {
#pragma unroll
    for (int i = 0; i < PER; ++i)
      if (e0 + i < E) dense_out[e0 + i] = dense[i];
    if (lane == 0) dense_out[E] = total;
  }
  const int nvec = row_bytes / 16;
  const int i = blockIdx.x;
  if (i >= total) return;
  // the one expert segment holding dense row i
  int hit = -1;
#pragma unroll
  for (int q = 0; q < PER; ++q)
    if (dense[q] <= i && i < dense[q] + placed[q]) hit = off[q] + (i - dense[q]);
  const uint64_t m = __ballot(hit >= 0);
  if (m == 0) return;  // not reached: i < total lies in some segment
  const int region_row = __builtin_amdgcn_readlane(hit, (int)__builtin_ctzll(m));
  const size_t from = PACK ? (size_t)region_row : (size_t)i;
  const size_t to = PACK ? (size_t)i : (size_t)region_row;
  const uint4* s4 = reinterpret_cast<const uint4*>(src + from * row_bytes);
  uint4* d4 = reinterpret_cast<uint4*>(dst + to * row_bytes);
  for (int v0 = 0; v0 < nvec; v0 += KV * kWave) {
    uint4 buf[KV];
#pragma unroll
    for (int j = 0; j < KV; ++j) buf[j] = load_stream(&s4[min(v0 + j * kWave + lane, nvec - 1)]);
#pragma unroll
    for (int j = 0; j < KV; ++j) {
      const int v = v0 + j * kWave + lane;
      if (v < nvec) store_stream(&d4[v], buf[j]);
    }
  }
  if (src_scales)
    for (int b = lane; b < nb; b += kWave) dst_scales[to * nb + b] = src_scales[from * nb + b];
}

template <bool PACK, int PER>
void launch_kv(int nvec, dim3 grid, hipStream_t st, const uint8_t* s, const float* ss,
               uint8_t* d, float* ds, const int32_t* counts, const int32_t* offsets,
               int32_t* dense_out, int E, int C, uint32_t l_magic, int row_bytes, int nb,
               int vec4) {
  // vectors per lane and pass: enough for a whole row where it fits in 16
  if (nvec <= 4 * kWave)
    hipLaunchKernelGGL((gemm_io_kernel<PACK, PER, 4>), grid, dim3(kWave), 0, st, s, ss, d, ds,
                       counts, offsets, dense_out, E, C, l_magic, row_bytes, nb, vec4);
  else if (nvec <= 8 * kWave)
    hipLaunchKernelGGL((gemm_io_kernel<PACK, PER, 8>), grid, dim3(kWave), 0, st, s, ss, d, ds,
                       counts, offsets, dense_out, E, C, l_magic, row_bytes, nb, vec4);
  else
    hipLaunchKernelGGL((gemm_io_kernel<PACK, PER, 16>), grid, dim3(kWave), 0, st, s, ss, d, ds,
                       counts, offsets, dense_out, E, C, l_magic, row_bytes, nb, vec4);
}

template <bool PACK>
void launch_per(int nvec, dim3 grid, hipStream_t st, const uint8_t* s, const float* ss,
                uint8_t* d, float* ds, const int32_t* counts, const int32_t* offsets,
                int32_t* dense_out, int E, int C, uint32_t l_magic, int row_bytes, int nb,
               int vec4) {
  // experts per lane: E <= 64 * PER
  if (E <= 4 * kWave)
    launch_kv<PACK, 4>(nvec, grid, st, s, ss, d, ds, counts, offsets, dense_out, E, C, l_magic,
                       row_bytes, nb, vec4);
  else if (E <= 8 * kWave)
    launch_kv<PACK, 8>(nvec, grid, st, s, ss, d, ds, counts, offsets, dense_out, E, C, l_magic,
                       row_bytes, nb, vec4);
  else
    launch_kv<PACK, 16>(nvec, grid, st, s, ss, d, ds, counts, offsets, dense_out, E, C, l_magic,
                        row_bytes, nb, vec4);
}

static_assert(kMaxExperts <= 16 * kWave, "the widest kernel holds 16 experts per lane");

}  // namespace

hipError_t launch_gemm_io(bool pack, const void* src, const float* src_scales, void* dst,
                          float* dst_scales, const int32_t* counts, const int32_t* offsets,
                          int32_t* dense_out, int max_rows, int E, int L, int C, int H,
                          int payload, hipStream_t st) {
  const int row_bytes = payload == 0 ? 2 * H : H;
  const int nb = payload == 0 ? 0 : H / kFp8Block;
  // one dense row per wave: every wave loads all E counts and offsets (a few
  // KB, from L2), which costs less than moving several rows one after the
  // other in a wave (measured at 32768 rows: 156 us against 178 with 4)
  const dim3 grid((unsigned)max(1, max_rows));
  const uint32_t l_magic = L >= 2 ? (uint32_t)(((1ull << 32) + L - 1) / L) : 0u;
  const uint8_t* s = reinterpret_cast<const uint8_t*>(src);
  uint8_t* d = reinterpret_cast<uint8_t*>(dst);
  const float* ss = payload ? src_scales : nullptr;
  const int nvec = row_bytes / 16;
  const int vec4 = E % 4 == 0 && ((reinterpret_cast<uintptr_t>(counts) |
                                   reinterpret_cast<uintptr_t>(offsets)) & 15) == 0;
  if (pack)
    launch_per<true>(nvec, grid, st, s, ss, d, dst_scales, counts, offsets, dense_out, E, C,
                     l_magic, row_bytes, nb, vec4);
  else
    launch_per<false>(nvec, grid, st, s, ss, d, dst_scales, counts, offsets, dense_out, E, C,
                      l_magic, row_bytes, nb, vec4);
  return hipGetLastError();
}

}  // namespace moe
