// combine.hip -- receiver-side weighted sum of each token's returned rows.
//
// The combine receives the processed rows and forms their router-weighted
// average, accumulating only on the receiving side ("Enabling
// trillion-parameter models on AWS EFA", Introduction, Send and Receive
// Buffers, Evaluation).  A block owns one (token, column chunk); the token's
// k rows and weights are staged once in LDS, each thread issues its k 16-byte
// gathers together (8 at a time) and folds them with fp32 fused multiply-adds
// in slot order from zero, then rounds to bf16 (nearest even) and stores 16
// bytes.  With the fp8 payload a thread owns 16 columns: one 16-byte gather of
// codes per row, each code decoded exactly to fp32 and multiplied by its
// block's fp32 scale.  This is a bandwidth-bound gather-reduce: no MFMA.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kGroup = 8;  // gathers in flight per thread

struct CombineParams {
  const void* y;
  const float* ys;
  const int32_t* token_row;
  const float* w;
  void* out;
  int T, H, k;
  int col_chunks;
  int vec_per_chunk;
};

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

__global__ void __launch_bounds__(kBlock) combine_bf16_kernel(CombineParams p) {
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int t = blockIdx.x / p.col_chunks;
  const int cc = blockIdx.x - t * p.col_chunks;
  if (threadIdx.x < p.k) {
    s_row[threadIdx.x] = p.token_row[(size_t)t * p.k + threadIdx.x];
    s_w[threadIdx.x] = p.w[(size_t)t * p.k + threadIdx.x];
  }
  __syncthreads();
  const int nvec = p.H / 8;
  const int v = cc * p.vec_per_chunk + threadIdx.x;
  const int v1 = min(cc * p.vec_per_chunk + p.vec_per_chunk, nvec);
  if (v >= v1) return;
  const uint4* y = reinterpret_cast<const uint4*>(p.y);
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.0f;
  for (int j0 = 0; j0 < p.k; j0 += kGroup) {
    uint4 yv[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int j = j0 + g;
      const int row = j < p.k ? s_row[j] : -1;
      yv[g] = row >= 0 ? y[(size_t)row * nvec + v] : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int j = j0 + g;
      if (j >= p.k || s_row[j] < 0) continue;
      const float wj = s_w[j];
      const uint32_t q[4] = {yv[g].x, yv[g].y, yv[g].z, yv[g].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[2 * m] = fmaf(wj, bf16_lo(q[m]), acc[2 * m]);
        acc[2 * m + 1] = fmaf(wj, bf16_hi(q[m]), acc[2 * m + 1]);
      }
    }
  }
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  reinterpret_cast<uint4*>(p.out)[(size_t)t * nvec + v] = o;
}

// fp8: vectors of 16 codes; 8 vectors share one 128-column scale.
__global__ void __launch_bounds__(kBlock) combine_fp8_kernel(CombineParams p) {
  __shared__ int s_row[kMaxTopK];
  __shared__ float s_w[kMaxTopK];
  const int t = blockIdx.x / p.col_chunks;
  const int cc = blockIdx.x - t * p.col_chunks;
  if (threadIdx.x < p.k) {
    s_row[threadIdx.x] = p.token_row[(size_t)t * p.k + threadIdx.x];
    s_w[threadIdx.x] = p.w[(size_t)t * p.k + threadIdx.x];
  }
  __syncthreads();
  const int nvec = p.H / 16;
  const int nb = p.H / kFp8Block;
  const int v = cc * p.vec_per_chunk + threadIdx.x;
  const int v1 = min(cc * p.vec_per_chunk + p.vec_per_chunk, nvec);
  if (v >= v1) return;
  const uint4* y = reinterpret_cast<const uint4*>(p.y);
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  for (int j0 = 0; j0 < p.k; j0 += kGroup) {
    uint4 yv[kGroup];
    float sc[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int j = j0 + g;
      const int row = j < p.k ? s_row[j] : -1;
      yv[g] = row >= 0 ? y[(size_t)row * nvec + v] : make_uint4(0, 0, 0, 0);
      sc[g] = row >= 0 ? p.ys[(size_t)row * nb + v / 8] : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const int j = j0 + g;
      if (j >= p.k || s_row[j] < 0) continue;
      const float wj = s_w[j];
      const uint32_t q[4] = {yv[g].x, yv[g].y, yv[g].z, yv[g].w};
#pragma unroll
      for (int m = 0; m < 16; ++m) {
        const float val = e4m3_to_f32((q[m / 4] >> (8 * (m % 4))) & 0xffu) * sc[g];
        acc[m] = fmaf(wj, val, acc[m]);
      }
    }
  }
  uint4* out = reinterpret_cast<uint4*>(p.out) + (size_t)t * (p.H / 8) + 2 * (size_t)v;
  uint4 o0, o1;
  o0.x = pack_bf16x2(acc[0], acc[1]);
  o0.y = pack_bf16x2(acc[2], acc[3]);
  o0.z = pack_bf16x2(acc[4], acc[5]);
  o0.w = pack_bf16x2(acc[6], acc[7]);
  o1.x = pack_bf16x2(acc[8], acc[9]);
  o1.y = pack_bf16x2(acc[10], acc[11]);
  o1.z = pack_bf16x2(acc[12], acc[13]);
  o1.w = pack_bf16x2(acc[14], acc[15]);
  out[0] = o0;
  out[1] = o1;
}

}  // namespace

hipError_t launch_combine(const void* y, const float* ys, const int32_t* token_row,
                          const float* w, void* out, int T, int H, int k, int payload,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  CombineParams p{y, ys, token_row, w, out, T, H, k, 0, 0};
  const int nvec = payload == 0 ? H / 8 : H / 16;
  p.col_chunks = (nvec + kBlock - 1) / kBlock;
  p.vec_per_chunk = (nvec + p.col_chunks - 1) / p.col_chunks;
  const unsigned blocks = (unsigned)T * (unsigned)p.col_chunks;
  if (payload == 0)
    hipLaunchKernelGGL(combine_bf16_kernel, dim3(blocks), dim3(kBlock), 0, st, p);
  else
    hipLaunchKernelGGL(combine_fp8_kernel, dim3(blocks), dim3(kBlock), 0, st, p);
  return hipGetLastError();
}

}  // namespace moe
