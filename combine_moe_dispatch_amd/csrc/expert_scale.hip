// expert_scale.hip -- per-expert scalar stand-in for the experts' grouped GEMM.
//
// Between dispatch and combine the experts multiply their tokens with their
// weights in a grouped GEMM ("Enabling trillion-parameter models on AWS EFA",
// MoE all-to-all over EFA).  Trained weights are not part of this library, so
// each expert scales its rows by one fp32 scalar.  Like a grouped GEMM under
// graph capture, the kernel sizes its work from the per-expert counts and
// offsets in device memory, not from the buffer bounds ("Lower Latency and
// Higher Throughput with Multi-Node DeepSeek Deployment", Quantization).
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kRowGroups = 8;  // blocks per expert

__device__ __forceinline__ int placed_end(const int32_t* counts, const int32_t* offsets, int e,
                                          int L, int C) {
  int end = offsets[e] + counts[e];
  if (C > 0) end = min(end, (e / L) * C + C);
  return end;
}

__global__ void __launch_bounds__(kBlock)
expert_scale_bf16_kernel(const uint4* recv, const int32_t* counts, const int32_t* offsets,
                         const float* alpha, uint4* y, int E, int L, int C, int H) {
  const int e = blockIdx.x / kRowGroups;
  const int g = blockIdx.x - e * kRowGroups;
  const int begin = offsets[e];
  const int end = placed_end(counts, offsets, e, L, C);
  const float a = alpha[e];
  const int nvec = H / 8;
  for (int row = begin + g; row < end; row += kRowGroups) {
    for (int v = threadIdx.x; v < nvec; v += kBlock) {
      const uint4 x = recv[(size_t)row * nvec + v];
      const uint32_t q[4] = {x.x, x.y, x.z, x.w};
      uint32_t o[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const float lo = a * bf16_lo(q[m]);
        const float hi = a * bf16_hi(q[m]);
        o[m] = pack_bf16x2(lo, hi);
      }
      y[(size_t)row * nvec + v] = make_uint4(o[0], o[1], o[2], o[3]);
    }
  }
}

__global__ void __launch_bounds__(kBlock)
expert_scale_fp8_kernel(const uint4* recv, const float* recv_scales, const int32_t* counts,
                        const int32_t* offsets, const float* alpha, uint4* y, float* y_scales,
                        int E, int L, int C, int H) {
  const int e = blockIdx.x / kRowGroups;
  const int g = blockIdx.x - e * kRowGroups;
  const int begin = offsets[e];
  const int end = placed_end(counts, offsets, e, L, C);
  const float a = alpha[e];
  const int nvec = H / 16;
  const int nb = H / kFp8Block;
  for (int row = begin + g; row < end; row += kRowGroups) {
    for (int v = threadIdx.x; v < nvec; v += kBlock) y[(size_t)row * nvec + v] = recv[(size_t)row * nvec + v];
    for (int b = threadIdx.x; b < nb; b += kBlock)
      y_scales[(size_t)row * nb + b] = recv_scales[(size_t)row * nb + b] * a;
  }
}

}  // namespace

hipError_t launch_expert_scale(const void* recv, const float* recv_scales,
                               const int32_t* expert_counts, const int32_t* expert_offsets,
                               const float* alpha, void* y, float* y_scales, int E, int L,
                               int C, int H, int payload, hipStream_t st) {
  const unsigned blocks = (unsigned)E * kRowGroups;
  if (payload == 0)
    hipLaunchKernelGGL(expert_scale_bf16_kernel, dim3(blocks), dim3(kBlock), 0, st,
                       reinterpret_cast<const uint4*>(recv), expert_counts, expert_offsets,
                       alpha, reinterpret_cast<uint4*>(y), E, L, C, H);
  else
    hipLaunchKernelGGL(expert_scale_fp8_kernel, dim3(blocks), dim3(kBlock), 0, st,
                       reinterpret_cast<const uint4*>(recv), recv_scales, expert_counts,
                       expert_offsets, alpha, reinterpret_cast<uint4*>(y), y_scales, E, L, C, H);
  return hipGetLastError();
}

}  // namespace moe
