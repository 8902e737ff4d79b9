// route_topk.hip -- top-k router selection, one wavefront per token.
//
// The router picks the experts each token goes to ("Enabling
// trillion-parameter models on AWS EFA", Introduction) and hands the top-k
// indices and scores to the dispatch ("Lower Latency and Higher Throughput
// with Multi-Node DeepSeek Deployment", MoE Router).
//
// Each lane holds ceil(E/64) biased logits (coalesced: value i of lane l is
// expert i*64 + l), packs each with its id into one 64-bit key whose unsigned
// order is (value descending, id ascending), and sorts its keys once, best
// first.  Each of the k rounds then takes every lane's head and finds the
// wave's largest key in two parts: the largest high word (the value) by a DPP
// butterfly inside each 16-lane row and two DPP row broadcasts across the
// rows (one max instruction per step), then a ballot of the heads holding it;
// only when several do, the same reduction over their low words picks the
// lowest id.  The owning lane pops its head.  Equal values go to the lower
// expert id, so slots come out in descending order.  Lanes 0..k-1 then form
// the weights in fp32 and normalise them to one.
//
// Group-limited routing (same page, MoE Router: plain top-k is the case where
// the kept groups are all experts): each group's score is the sum of its two
// largest biased logits.  Where the groups fall on whole lanes (a lane then
// holds ceil(E/64) consecutive experts, and a group a power-of-two block of
// up to 16 lanes), every lane takes its own top two and DPP steps merge them
// inside the group; otherwise the wave stages its logits in LDS and lane g
// scans group g.  A group is kept when fewer than topk_groups groups beat it
// (larger score, or equal score and lower id), counted with one 64-bit key
// compare per group; the experts of the other groups drop out before the
// top-k rounds.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

// Tokens (waves) per block: one-wave blocks spread a short token list over
// more compute units (DeepSeek-V3 decode 3.25 -> 3.02 us); four-wave blocks
// are faster past a few thousand tokens (skewed prefill 5.16 against 5.31 us).
constexpr int kRouteWavesLarge = 4;
constexpr int kOneWaveMaxTokens = 2048;
constexpr int kNone = 0x7fffffff;

#ifdef MOE_PHASE_STAMPS
// the router's trace buffer (tracing library only)
__device__ uint64_t* g_trace;
__device__ uint32_t g_trace_slots;
#endif

// (value, id) as one 64-bit key whose unsigned order is the selection order:
// the high word maps the fp32 value to an order-preserving unsigned (sign bit
// flipped for non-negative values, all bits for negative ones; -0 is taken
// as +0 first, as the float comparison does), the low word is the bitwise
// complement of the id, so of two equal values the lower id has the larger
// key.  An absent entry is key 0, below every real one.
__device__ __forceinline__ uint64_t route_key(float v, int id) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)id;
}
__device__ __forceinline__ float route_key_value(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}
__device__ __forceinline__ int route_key_id(uint64_t key) { return (int)~(uint32_t)key; }

// Largest 32-bit value over the wave (all 64 lanes active), returned
// uniform.  Four butterfly steps leave every lane of a 16-lane row with the
// row's largest; the row broadcasts then fold row 0 into row 1 and row 2 into
// row 3 (lane 15 of the row before), and row 1 into rows 2-3 (lane 31), so
// lane 63 holds the wave's largest (max is idempotent, so overlapping folds
// do no harm).  Each step is one max instruction reading its first operand
// through DPP, written out because the compiler's form of it is a DPP move
// followed by the max; two wait states go before every step (a DPP read of a
// register the previous instruction wrote) and after the last.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  asm volatile(
      "s_nop 1\n"
      "v_max_u32_dpp %0, %0, %0 quad_perm:[1,0,3,2] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_u32_dpp %0, %0, %0 quad_perm:[2,3,0,1] row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_u32_dpp %0, %0, %0 row_half_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_u32_dpp %0, %0, %0 row_mirror row_mask:0xf bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_u32_dpp %0, %0, %0 row_bcast:15 row_mask:0xa bank_mask:0xf\n"
      "s_nop 1\n"
      "v_max_u32_dpp %0, %0, %0 row_bcast:31 row_mask:0xc bank_mask:0xf\n"
      "s_nop 1\n"
      : "+v"(v));
  return __builtin_amdgcn_readlane(v, 63);
}

// Keep the two largest values seen (equal values fill both).
__device__ __forceinline__ void top2_take(float l, float& m1, float& m2) {
  const bool above1 = l > m1;
  const bool above2 = l > m2;
  m2 = above1 ? m1 : (above2 ? l : m2);
  m1 = above1 ? l : m1;
}

// Sum of s over lanes 0..31 (all other lanes hold 0), the same value in
// every lane: a DPP row-shift inclusive sum inside each 16-lane row, then the
// totals of rows 0 and 1 read with readlane.
__device__ __forceinline__ float slot_sum(float s) {
  float x = s;
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));
  const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 15));
  const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 31));
  return r0 + r1;
}

// Merge this lane's top two (m1 >= m2) with those of the lane a DPP pattern
// names: the two largest of the four values, counted with multiplicity.
template <int CTRL>
__device__ __forceinline__ void top2_merge(float& m1, float& m2) {
  const float o1 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m1), CTRL, 0xf, 0xf, false));
  const float o2 = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(m2), CTRL, 0xf, 0xf, false));
  const float lo = fminf(m1, o1);
  m1 = fmaxf(m1, o1);
  m2 = fmaxf(lo, fmaxf(m2, o2));
}

// LDS hand-off inside one wavefront (no block barrier: waves exit early).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int VPL, bool GROUPED, int WAVES>
__global__ void __launch_bounds__(WAVES * kWave)
route_topk_kernel(const float* __restrict__ logits, const float* __restrict__ bias, int T,
                  int E, int k, int score, int n_groups_lpg, int topk_groups,
                  int32_t* __restrict__ ids, float* __restrict__ weights) {
  // n_groups (at most 64) in the low 16 bits; lanes per group in the high
  // bits, 0 when the groups do not fall on whole lanes (measured faster on the
  // Kimi-K2 shape than a separate argument)
  const int n_groups = n_groups_lpg & 0xffff;
  const int lpg = n_groups_lpg >> 16;
  __shared__ __align__(16) float s_logit[GROUPED ? WAVES : 1][GROUPED ? kMaxExperts : 1];
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int t = blockIdx.x * WAVES + wave;
  // fetched with T: everything the first loads and the group step need
  if constexpr (GROUPED)
    MOE_ARGS_UP_FRONT("s"(logits), "s"(bias), "s"(n_groups_lpg), "s"(topk_groups));
  else
    MOE_ARGS_UP_FRONT("s"(logits), "s"(bias));
  if (t >= T) return;
  MOE_STAMP(t_entry);
  const float* row = logits + (size_t)t * E;

  // Group-limited routing on whole lanes (lpg > 0, set by the host): lane l
  // holds the epl = ceil(E/64) consecutive experts from l*epl, and group g is
  // the lpg aligned lanes from g*lpg (a power of two up to 16).  Otherwise
  // (and for plain top-k) value i of lane l is expert i*64 + l.
  const bool contig = GROUPED && lpg > 0;
  const int epl = (int)((unsigned)(E + kWave - 1) >> 6);

  // every load is unconditional (index clamped, value masked below) and all
  // are issued before the first is used: one memory round trip
  int eid[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) eid[i] = contig ? lane * epl + i : i * kWave + lane;
  float v[VPL], bv_[VPL];
  int id[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) v[i] = row[min(eid[i], E - 1)];
  if (bias) {
#pragma unroll
    for (int i = 0; i < VPL; ++i) bv_[i] = bias[min(eid[i], E - 1)];
  } else {
#pragma unroll
    for (int i = 0; i < VPL; ++i) bv_[i] = 0.0f;
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const bool in = eid[i] < E && (!contig || i < epl);
    v[i] = in ? (bias ? v[i] + bv_[i] : v[i]) : -INFINITY;
    id[i] = in ? eid[i] : kNone;
  }
  if (GROUPED) {
    // group score = sum of the group's two largest biased logits
    const int gsz = contig ? lpg * epl : E / n_groups;
    float gv = -INFINITY;
    int lanes_per_group = 1;
    if (contig) {
      // the lane's own top two, then DPP merges inside the group's lanes;
      // every lane of the group ends with the group's pair
      float m1 = -INFINITY, m2 = -INFINITY;
#pragma unroll
      for (int i = 0; i < VPL; ++i) top2_take(v[i], m1, m2);
      if (lpg >= 2) top2_merge<0xB1>(m1, m2);   // lane ^ 1
      if (lpg >= 4) top2_merge<0x4E>(m1, m2);   // lane ^ 2
      if (lpg >= 8) top2_merge<0x141>(m1, m2);  // mirrored quad
      if (lpg >= 16) top2_merge<0x140>(m1, m2); // mirrored half-row
      gv = gsz > 1 ? m1 + m2 : m1;
      lanes_per_group = lpg;
    } else {
      // lane g scans group g in the wave's LDS copy of its biased logits
      float* sl = s_logit[wave];
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (i * kWave + lane < E) sl[i * kWave + lane] = v[i];
      wave_lds_sync();
      if (lane < n_groups) {
        float m1 = -INFINITY, m2 = -INFINITY;
        if ((gsz & 3) == 0) {
          // 16-byte LDS reads, 4 in flight per round
          const float4* g4 = reinterpret_cast<const float4*>(sl + lane * gsz);
          for (int c0 = 0; c0 < gsz / 4; c0 += 4) {
            float q[16];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float4 f = c0 + c < gsz / 4
                                   ? g4[c0 + c]
                                   : make_float4(-INFINITY, -INFINITY, -INFINITY, -INFINITY);
              q[4 * c] = f.x;
              q[4 * c + 1] = f.y;
              q[4 * c + 2] = f.z;
              q[4 * c + 3] = f.w;
            }
#pragma unroll
            for (int c = 0; c < 16; ++c) top2_take(q[c], m1, m2);
          }
        } else {
          for (int e = lane * gsz; e < lane * gsz + gsz; ++e) top2_take(sl[e], m1, m2);
        }
        gv = gsz > 1 ? m1 + m2 : m1;
      }
    }
    // a group is kept when fewer than topk_groups groups beat it (larger
    // score, or an equal score and a lower group id): one 64-bit key compare
    // against each group's score, read from the group's first lane
    const int my_g = lane >> (__ffs(lanes_per_group) - 1);
    const uint64_t gkey = my_g < n_groups ? route_key(gv, my_g) : 0ull;
    int beaten_by = 0;
    for (int h = 0; h < n_groups; ++h) {
      const int src = h * lanes_per_group;
      const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)gkey, src);
      const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(gkey >> 32), src);
      beaten_by += (((uint64_t)hi << 32) | lo) > gkey ? 1 : 0;
    }
    const bool keep = my_g < n_groups && beaten_by < topk_groups;
    if (contig) {
      // all of a lane's experts are in its own group
      if (!keep) {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          v[i] = -INFINITY;
          id[i] = kNone;
        }
      }
    } else {
      const uint64_t kept = __ballot(keep);  // bit g: group g (lane g) kept
      if ((gsz & (gsz - 1)) == 0) {  // power-of-two groups: a shift, not a division
        const int sh = __ffs(gsz) - 1;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          if (id[i] != kNone && !((kept >> (id[i] >> sh)) & 1ull)) {
            v[i] = -INFINITY;
            id[i] = kNone;
          }
        }
      } else {
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
          if (id[i] != kNone && !((kept >> (id[i] / gsz)) & 1ull)) {
            v[i] = -INFINITY;
            id[i] = kNone;
          }
        }
      }
    }
  }
  // this lane's entries as keys, sorted best first (insertion network)
  MOE_TRACE_WAIT();  // tracing only: the logits have arrived
  MOE_STAMP(t_loaded);
  uint64_t key[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) key[i] = id[i] == kNone ? 0ull : route_key(v[i], id[i]);
#pragma unroll
  for (int a = 1; a < VPL; ++a) {
#pragma unroll
    for (int b = a; b > 0; --b) {
      const uint64_t hi = key[b] > key[b - 1] ? key[b] : key[b - 1];
      const uint64_t lo = key[b] > key[b - 1] ? key[b - 1] : key[b];
      key[b - 1] = hi;
      key[b] = lo;
    }
  }

  uint32_t khi[VPL], klo[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    khi[i] = (uint32_t)(key[i] >> 32);
    klo[i] = (uint32_t)key[i];
  }
  MOE_STAMP(t_sorted);
  uint64_t my_key = 0;  // lane j keeps the key of slot j
  for (int j = 0; j < k; ++j) {
    // the largest value first; only when several heads share it, the
    // largest low word (lowest id) among them
    const uint32_t m = wave_max_u32(khi[0]);
    const uint64_t tied = __ballot(khi[0] == m);
    int win;
    if (__popcll(tied) == 1) {
      win = __ffsll((unsigned long long)tied) - 1;
    } else {
      const uint32_t ml = wave_max_u32(khi[0] == m ? klo[0] : 0u);
      win = __ffsll((unsigned long long)__ballot(khi[0] == m && klo[0] == ml)) - 1;
    }
    const uint32_t wl = __builtin_amdgcn_readlane(klo[0], win);
    if (lane == win) {  // this lane owned the winner: pop its head
#pragma unroll
      for (int i = 0; i + 1 < VPL; ++i) {
        khi[i] = khi[i + 1];
        klo[i] = klo[i + 1];
      }
      khi[VPL - 1] = 0u;
      klo[VPL - 1] = 0u;
    }
    if (lane == j) my_key = ((uint64_t)m << 32) | wl;
  }
  MOE_STAMP(t_selected);
  const float my_val = route_key_value(my_key);
  const int my_id = route_key_id(my_key);

  float s = 0.0f;
  const float top = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_val), 0));
  if (lane < k) {
    if (score == 1)
      s = 1.0f / (1.0f + expf(-my_val));
    else
      s = expf(my_val - top);
  }
  // sum over lanes 0..k-1 (k <= 32: rows 0 and 1) in slot order within each
  // DPP row, then the two row sums
  const float sum = slot_sum(s);
  if (lane < k) {
    ids[(size_t)t * k + lane] = my_id;
    weights[(size_t)t * k + lane] = s / sum;
  }
#ifdef MOE_PHASE_STAMPS
  MOE_STAMP(t_stored);
  MOE_TRACE_WAIT();
  MOE_STAMP(t_done);
  trace_record(g_trace, g_trace_slots, (uint32_t)t, t_entry, t_loaded, t_sorted, t_selected,
               t_stored, t_done);
#endif
}

template <int VPL, int WAVES>
hipError_t launch_waves(const float* logits, const float* bias, int T, int E, int k,
                        int score, int n_groups, int topk_groups, int32_t* ids, float* w,
                        hipStream_t st) {
  const int blocks = (T + WAVES - 1) / WAVES;
  if (n_groups > 1 && topk_groups < n_groups) {
    // lanes per group when the groups fall on whole lanes, else 0
    const int gsz = E / n_groups;
    const int epl = (E + kWave - 1) / kWave;
    const int lpg = gsz % epl == 0 ? gsz / epl : 0;
    const bool on_lanes = lpg > 0 && lpg <= 16 && (lpg & (lpg - 1)) == 0;
    hipLaunchKernelGGL((route_topk_kernel<VPL, true, WAVES>), dim3(blocks),
                       dim3(WAVES * kWave), 0, st, logits, bias, T, E, k, score,
                       n_groups | ((on_lanes ? lpg : 0) << 16), topk_groups, ids, w);
  } else {
    hipLaunchKernelGGL((route_topk_kernel<VPL, false, WAVES>), dim3(blocks),
                       dim3(WAVES * kWave), 0, st, logits, bias, T, E, k, score, 1, 1, ids, w);
  }
  return hipGetLastError();
}

template <int VPL>
hipError_t launch_vpl(const float* logits, const float* bias, int T, int E, int k,
                      int score, int n_groups, int topk_groups, int32_t* ids, float* w,
                      hipStream_t st) {
  if (T <= kOneWaveMaxTokens)
    return launch_waves<VPL, 1>(logits, bias, T, E, k, score, n_groups, topk_groups, ids, w, st);
  return launch_waves<VPL, kRouteWavesLarge>(logits, bias, T, E, k, score, n_groups,
                                             topk_groups, ids, w, st);
}

}  // namespace

hipError_t launch_route_topk(const float* logits, const float* bias, int T, int E, int k,
                             int score, int n_groups, int topk_groups, int32_t* ids, float* w,
                             hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int vpl = (E + kWave - 1) / kWave;
#define MOE_ROUTE_ARGS logits, bias, T, E, k, score, n_groups, topk_groups, ids, w, st
  if (vpl <= 1) return launch_vpl<1>(MOE_ROUTE_ARGS);
  if (vpl <= 2) return launch_vpl<2>(MOE_ROUTE_ARGS);
  if (vpl <= 4) return launch_vpl<4>(MOE_ROUTE_ARGS);
  if (vpl <= 6) return launch_vpl<6>(MOE_ROUTE_ARGS);
  if (vpl <= 8) return launch_vpl<8>(MOE_ROUTE_ARGS);
  return launch_vpl<16>(MOE_ROUTE_ARGS);
#undef MOE_ROUTE_ARGS
}

}  // namespace moe

#ifdef MOE_PHASE_STAMPS
// Tracing library only: the buffer the router writes its phase records to
// (slots records of kTraceWords words, one per token), or null to stop.
// Returns 0 or the HIP error code.
extern "C" int moe_trace_set_route(void* buf, uint32_t slots) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_trace), &buf, sizeof(buf));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_trace_slots), &slots, sizeof(slots));
  return (int)e;
}
#endif
