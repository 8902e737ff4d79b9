// route_topk.hip -- top-k router selection, one wavefront per token.
//
// The router picks the experts each token goes to ("Enabling
// trillion-parameter models on AWS EFA", Introduction) and hands the top-k
// indices and scores to the dispatch ("Lower Latency and Higher Throughput
// with Multi-Node DeepSeek Deployment", MoE Router).  Each lane holds
// ceil(E/64) biased logits (coalesced: value i of lane l is expert i*64 + l);
// k rounds of a 64-lane (value, index) arg-max pick the experts in descending
// order, equal values going to the lower expert id.  Lanes 0..k-1 then form
// the weights in fp32 and normalise them to sum to one.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kRouteWaves = 4;  // tokens per 256-thread block

__device__ __forceinline__ bool better(float av, int ai, float bv, int bi) {
  return av > bv || (av == bv && ai < bi);
}

template <int VPL>
__global__ void __launch_bounds__(kRouteWaves * kWave)
route_topk_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                  int T, int E, int k, int score, int32_t* __restrict__ ids,
                  float* __restrict__ weights) {
  const int lane = lane_id();
  const int t = blockIdx.x * kRouteWaves + (threadIdx.x / kWave);
  if (t >= T) return;
  const float* row = logits + (size_t)t * E;

  float v[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int e = i * kWave + lane;
    if (e < E) {
      float l = row[e];
      if (bias) l = l + bias[e];
      v[i] = l;
    } else {
      v[i] = -INFINITY;
    }
  }
  uint32_t taken = 0;  // bit i: value i of this lane was chosen (or is padding)
#pragma unroll
  for (int i = 0; i < VPL; ++i)
    if (i * kWave + lane >= E) taken |= 1u << i;

  float my_val = 0.0f;  // lane j keeps the biased logit of slot j
  int my_id = 0;
  for (int j = 0; j < k; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int e = i * kWave + lane;
      if (!(taken & (1u << i)) && better(v[i], e, bv, bi)) {
        bv = v[i];
        bi = e;
      }
    }
#pragma unroll
    for (int d = kWave / 2; d > 0; d >>= 1) {
      const float ov = __shfl_xor(bv, d, kWave);
      const int oi = __shfl_xor(bi, d, kWave);
      if (better(ov, oi, bv, bi)) {
        bv = ov;
        bi = oi;
      }
    }
    if ((bi & (kWave - 1)) == lane) taken |= 1u << (bi / kWave);
    if (lane == j) {
      my_val = bv;
      my_id = bi;
    }
  }

  float s = 0.0f;
  const float top = __shfl(my_val, 0, kWave);
  if (lane < k) {
    if (score == 1)
      s = 1.0f / (1.0f + expf(-my_val));
    else
      s = expf(my_val - top);
  }
  const float sum = wave_sum_f(s);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = s / sum;
  }
}

template <int VPL>
hipError_t launch_vpl(const float* logits, const float* bias, int T, int E, int k,
                      int score, int32_t* ids, float* w, hipStream_t st) {
  const int blocks = (T + kRouteWaves - 1) / kRouteWaves;
  hipLaunchKernelGGL(route_topk_kernel<VPL>, dim3(blocks), dim3(kRouteWaves * kWave), 0, st,
                     logits, bias, T, E, k, score, ids, w);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route_topk(const float* logits, const float* bias, int T, int E, int k,
                             int score, int32_t* ids, float* w, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int vpl = (E + kWave - 1) / kWave;
  if (vpl <= 1) return launch_vpl<1>(logits, bias, T, E, k, score, ids, w, st);
  if (vpl <= 2) return launch_vpl<2>(logits, bias, T, E, k, score, ids, w, st);
  if (vpl <= 4) return launch_vpl<4>(logits, bias, T, E, k, score, ids, w, st);
  if (vpl <= 6) return launch_vpl<6>(logits, bias, T, E, k, score, ids, w, st);
  if (vpl <= 8) return launch_vpl<8>(logits, bias, T, E, k, score, ids, w, st);
  return launch_vpl<16>(logits, bias, T, E, k, score, ids, w, st);
}

}  // namespace moe
