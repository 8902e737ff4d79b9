// combine_partial.hip -- combine with sender-side partial reduction.
//
// The alternative to accumulating only on the receiving side: each
// destination rank first sums a token's rows for its own experts and sends
// one row per (token, rank), which transfers less data at some cost in
// precision ("Enabling trillion-parameter models on AWS EFA", Evaluation).
//
// Stage 1 (send): for token t the distinct ranks of its placed pairs, in
// ascending order, get partial slots 0..m-1 of M = min(k, N).  Slot i holds
// bf16(fp32 fused multiply-add chain over the pairs on that rank, in slot
// order from 0); partial_rank[t][i] names the rank, -1 marks an unused slot.
// Stage 2 (recv): out[t] = bf16(fp32 sum of the used partial rows in slot
// order from 0).
//
// A one-wave block owns (token, 64-vector column chunk).  With k <= 8 the
// slots' rows, ranks and weights are uniform scalar loads and the grouping is
// scalar arithmetic; all k rows are loaded at once and each group is folded
// once, from its first slot, and stored.  With larger k lane j holds slot j's
// row, rank and weight (the grouping is a few readlanes), and rows stream in
// 8 at a time, folded into up to GC group accumulators (more groups take more
// passes).  bf16 rounding is the hardware packed convert.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 64;  // one wavefront per block
constexpr int kGroup = 8;   // row loads in flight per thread

__device__ __forceinline__ float readlane_f(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}

// Lane j < k: slot j's row, rank (-1 if skipped), weight and group (the
// index of its rank among the token's distinct ranks in ascending order);
// returns m, the number of distinct ranks.  Block (t, chunk 0) also writes
// partial_rank[t][:].
__device__ __forceinline__ int slot_groups(const int32_t* __restrict__ token_row,
                                           const int32_t* __restrict__ ids,
                                           const float* __restrict__ w,
                                           int32_t* __restrict__ partial_rank, int t, int cc,
                                           int k, int E, int L, int M, int& my_row,
                                           float& my_w, int& my_group) {
  const int lane = threadIdx.x;
  int my_rank = -1;
  my_row = -1;
  my_w = 0.0f;
  if (lane < k) {
    my_row = token_row[(size_t)t * k + lane];
    const int e = ids[(size_t)t * k + lane];
    my_rank = (my_row >= 0 && (unsigned)e < (unsigned)E) ? e / L : -1;
    my_w = w[(size_t)t * k + lane];
  }
  // first slot of each rank, the number of distinct ranks, and each slot's group
  bool first = my_rank >= 0;
  for (int j = 0; j < k; ++j)
    if (j < lane && __builtin_amdgcn_readlane(my_rank, j) == my_rank) first = false;
  const uint64_t firsts = __ballot(first);
  const int m = popc64(firsts);
  my_group = -1;
  if (my_rank >= 0) {
    my_group = 0;
    for (int j = 0; j < k; ++j)
      if (((firsts >> j) & 1ull) && __builtin_amdgcn_readlane(my_rank, j) < my_rank) ++my_group;
  }
  if (cc == 0 && lane < M) {
    int r = -1;
    for (int j = 0; j < k; ++j)
      if (__builtin_amdgcn_readlane(my_group, j) == lane) r = __builtin_amdgcn_readlane(my_rank, j);
    partial_rank[(size_t)t * M + lane] = r;
  }
  return m;
}

// bf16 partial row store of 8 or 16 fp32 sums (one or two 16-byte vectors).
template <int COLS>
__device__ __forceinline__ void store_partial(uint4* dst, const float* acc) {
#pragma unroll
  for (int h = 0; h < COLS / 8; ++h)
    store_stream(&dst[h], make_uint4(pack_bf16x2(acc[8 * h + 0], acc[8 * h + 1]),
                                     pack_bf16x2(acc[8 * h + 2], acc[8 * h + 3]),
                                     pack_bf16x2(acc[8 * h + 4], acc[8 * h + 5]),
                                     pack_bf16x2(acc[8 * h + 6], acc[8 * h + 7])));
}

// k <= kGroup: the token's rows, ids and weights are wave-uniform, read with
// scalar loads at the start (no vector load has to wait for them), and the
// grouping by rank is scalar arithmetic.  All k rows are then gathered at
// once into registers and each group is folded (its slots in slot order) and
// stored in turn.  A lane owns KV vectors of 8 columns, u and u + 64 (fp8:
// KV = 2, 8-byte code loads), so every 16-byte store instruction of the wave
// covers 1 KB of a partial row without gaps.  fp8 workgroups are renumbered
// so the column chunks of one token share an XCD and the L2 lines of its
// scales.  K = 8 fixes k at compile time; K = 0 takes k <= 8 at run time.
template <bool FP8, int K>
__global__ void __launch_bounds__(kBlock)
combine_send_small_kernel(const void* __restrict__ y, const float* __restrict__ ys,
                          const int32_t* __restrict__ token_row,
                          const int32_t* __restrict__ ids, const float* __restrict__ w,
                          uint4* __restrict__ partial, int32_t* __restrict__ partial_rank,
                          int H, int k_rt, int E, int L, uint32_t l_magic, int M,
                          int col_chunks, uint32_t cc_magic) {
  constexpr int KV = FP8 ? 2 : 1;
  const int k = K > 0 ? K : k_rt;
  const unsigned b = FP8 ? xcd_local_block(blockIdx.x, gridDim.x) : blockIdx.x;
  const int t = (int)udiv_magic(b, (uint32_t)col_chunks, cc_magic);
  const int cc = b - t * col_chunks;
  const int nv = H / 8;  // 8-column vectors per row
  const int nb = H / kFp8Block;
  const int lane = threadIdx.x;
  // slot g: row, rank (-1 if skipped), weight -- uniform values
  // (straight-line: every load is unconditional, slot indices clamped, and
  // nothing below branches on a loaded value, so all of them are issued
  // before the first wait)
  int rj[kGroup], ej[kGroup], rank[kGroup];
  float wj[kGroup];
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    const size_t q = (size_t)t * k + min(g, k - 1);
    rj[g] = token_row[q];
    ej[g] = ids[q];
    wj[g] = w[q];
  }
  // e / L as a multiply-high by ceil(2^32 / L) (exact: e * L < 2^32); with
  // L == 1 the magic is 0 and the rank is e itself
  const uint32_t l_one = L == 1 ? 0xffffffffu : 0u;
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    const uint32_t eu = (uint32_t)ej[g];
    const bool ok = (g < k) & (rj[g] >= 0) & (eu < (uint32_t)E);
    const int rk = (int)(__umulhi(eu, l_magic) | (eu & l_one));
    rank[g] = ok ? rk : -1;
    rj[g] = g < k ? rj[g] : -1;
    wj[g] = g < k ? wj[g] : 0.0f;
  }
  int u[KV];
#pragma unroll
  for (int i = 0; i < KV; ++i) u[i] = cc * kBlock * KV + lane + i * kBlock;
  // no early exit before the gathers: lanes past the row end mask them
  const bool active = u[0] < nv;
  // raw loads of every placed slot's vectors, issued before the grouping
  // arithmetic below so they are in flight meanwhile; each is decoded once,
  // in its group
  uint4 yv[kGroup];      // bf16: 8 values
  uint2 cv[kGroup][KV];  // fp8: 8 codes per vector
  float sc[kGroup][KV];
  if constexpr (FP8) {
    const uint2* y8 = reinterpret_cast<const uint2*>(y);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
#pragma unroll
      for (int i = 0; i < KV; ++i) {
        const bool use = rank[g] >= 0 && u[i] < nv;
        const size_t r = use ? (size_t)rj[g] : 0;
        cv[g][i] = use ? load_stream(&y8[r * nv + u[i]]) : make_uint2(0, 0);
        sc[g][i] = use ? ys[r * nb + u[i] / 16] : 0.0f;  // scales: cached loads
      }
  } else {
    const uint4* y16 = reinterpret_cast<const uint4*>(y);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      yv[g] = active && rank[g] >= 0 ? load_stream(&y16[(size_t)rj[g] * nv + u[0]])
                                    : make_uint4(0, 0, 0, 0);
  }
  // group of slot g = index of its rank among the token's distinct ranks in
  // ascending order
  bool first[kGroup];  // slot g is the first slot of its rank
  int grp[kGroup];
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    bool f = rank[g] >= 0;
#pragma unroll
    for (int g2 = 0; g2 < g; ++g2) f = f & (rank[g2] != rank[g]);
    first[g] = f;
  }
#pragma unroll
  for (int g = 0; g < kGroup; ++g) {
    int below = 0;  // distinct ranks smaller than rank[g]
#pragma unroll
    for (int g2 = 0; g2 < kGroup; ++g2) below += (first[g2] & (rank[g2] < rank[g])) ? 1 : 0;
    grp[g] = rank[g] >= 0 ? below : -1;
  }
  if (cc == 0 && lane < M) {
    int r = -1;
#pragma unroll
    for (int g = 0; g < kGroup; ++g) r = grp[g] == lane ? rank[g] : r;
    partial_rank[(size_t)t * M + lane] = r;
  }
  if (!active) return;
  // wait here for every gather, on every path: the folds below sit behind
  // uniform branches, and without this the compiler places a full vmcnt wait
  // before each of them, which on this GPU also waits for the partial rows
  // already being stored (stores count in vmcnt too)
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  // each group once, from its first slot: that slot and the later slots of
  // the same rank are folded in slot order, then the row is stored
#pragma unroll
  for (int g0 = 0; g0 < kGroup; ++g0) {
    if (!first[g0]) continue;
    float acc[8 * KV];
#pragma unroll
    for (int c = 0; c < 8 * KV; ++c) acc[c] = 0.0f;
#pragma unroll
    for (int g = g0; g < kGroup; ++g) {
      if (g > g0 && rank[g] != rank[g0]) continue;
      float val[8 * KV];
      if constexpr (FP8) {
#pragma unroll
        for (int i = 0; i < KV; ++i) {
          e4m3x4_to_f32(cv[g][i].x, &val[8 * i]);
          e4m3x4_to_f32(cv[g][i].y, &val[8 * i + 4]);
#pragma unroll
          for (int c = 0; c < 8; ++c) val[8 * i + c] = val[8 * i + c] * sc[g][i];
        }
      } else {
        const uint32_t q4[4] = {yv[g].x, yv[g].y, yv[g].z, yv[g].w};
#pragma unroll
        for (int c4 = 0; c4 < 4; ++c4) {
          val[2 * c4] = bf16_lo(q4[c4]);
          val[2 * c4 + 1] = bf16_hi(q4[c4]);
        }
      }
#pragma unroll
      for (int c = 0; c < 8 * KV; ++c) acc[c] = fmaf(wj[g], val[c], acc[c]);
    }
    uint4* dst = partial + ((size_t)t * M + grp[g0]) * nv;
#pragma unroll
    for (int i = 0; i < KV; ++i)
      if (u[i] < nv) store_partial<8>(&dst[u[i]], &acc[8 * i]);
  }
}

template <bool FP8, int GC>
__global__ void __launch_bounds__(kBlock)
combine_send_kernel(const uint4* __restrict__ y, const float* __restrict__ ys,
                    const int32_t* __restrict__ token_row, const int32_t* __restrict__ ids,
                    const float* __restrict__ w, uint4* __restrict__ partial,
                    int32_t* __restrict__ partial_rank, int H, int k, int E, int L, int M,
                    int col_chunks, uint32_t cc_magic) {
  constexpr int kCols = FP8 ? 16 : 8;  // columns per thread
  const int t = (int)udiv_magic(blockIdx.x, (uint32_t)col_chunks, cc_magic);
  const int cc = blockIdx.x - t * col_chunks;
  const int nvec = H / kCols;
  const int lane = threadIdx.x;
  const int v = cc * kBlock + lane;
  int my_row, my_group;
  float my_w;
  const int m = slot_groups(token_row, ids, w, partial_rank, t, cc, k, E, L, M, my_row, my_w,
                            my_group);
  // lanes past the row end stay alive: later slots' values are read from
  // every lane with readlane
  const bool active = v < nvec;
  const int nb = H / kFp8Block;
  for (int g0 = 0; g0 < m; g0 += GC) {
    float acc[GC][kCols];
#pragma unroll
    for (int q = 0; q < GC; ++q)
#pragma unroll
      for (int c = 0; c < kCols; ++c) acc[q][c] = 0.0f;
    for (int j0 = 0; j0 < k; j0 += kGroup) {
      uint4 yv[kGroup];
      float sc[kGroup];
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const int j = j0 + g;
        const int gj = j < k ? __builtin_amdgcn_readlane(my_group, j) : -1;
        const int rj = j < k ? __builtin_amdgcn_readlane(my_row, j) : -1;
        const bool use = active && gj >= g0 && gj < g0 + GC;
        yv[g] = use ? load_stream(&y[(size_t)rj * nvec + v]) : make_uint4(0, 0, 0, 0);
        sc[g] = (FP8 && use) ? ys[(size_t)rj * nb + v / 8] : 0.0f;
      }
#pragma unroll
      for (int g = 0; g < kGroup; ++g) {
        const int j = j0 + g;
        const int gj = j < k ? __builtin_amdgcn_readlane(my_group, j) : -1;
        if (gj < g0 || gj >= g0 + GC) continue;
        float val[kCols];
        const uint32_t q4[4] = {yv[g].x, yv[g].y, yv[g].z, yv[g].w};
        if (FP8) {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) e4m3x4_to_f32(q4[c4], val + 4 * c4);
#pragma unroll
          for (int c = 0; c < kCols; ++c) val[c] = val[c] * sc[g];
        } else {
#pragma unroll
          for (int c4 = 0; c4 < 4; ++c4) {
            val[2 * c4] = bf16_lo(q4[c4]);
            val[2 * c4 + 1] = bf16_hi(q4[c4]);
          }
        }
        const float wj = readlane_f(my_w, j);
#pragma unroll
        for (int q = 0; q < GC; ++q) {
          if (gj != g0 + q) continue;
#pragma unroll
          for (int c = 0; c < kCols; ++c) acc[q][c] = fmaf(wj, val[c], acc[q][c]);
        }
      }
    }
    // partial rows are bf16: H / 8 vectors of 16 bytes each
#pragma unroll
    for (int q = 0; q < GC; ++q) {
      if (!active || g0 + q >= m) continue;
      store_partial<kCols>(partial + ((size_t)t * M + g0 + q) * (H / 8) + (size_t)v * (kCols / 8),
                           acc[q]);
    }
  }
}

// MM > 0: M (partial slots per token) fixed at compile time, so the slot
// ranks are one wide uniform load issued with the kernel arguments; MM == 0:
// M at run time.  No lane exits before the gathers.  DS: the output row is
// stored with device scope instead of non-temporally (large outputs).
template <int MM, bool DS>
__global__ void __launch_bounds__(kBlock)
combine_recv_kernel(const uint4* __restrict__ partial, const int32_t* __restrict__ partial_rank,
                    uint4* __restrict__ out, int H, int M_rt, int col_chunks,
                    uint32_t cc_magic) {
  const int M = MM > 0 ? MM : M_rt;
  const int t = (int)udiv_magic(blockIdx.x, (uint32_t)col_chunks, cc_magic);
  const int cc = blockIdx.x - t * col_chunks;
  const int nvec = H / 8;
  const int v = cc * kBlock + threadIdx.x;
  const bool active = v < nvec;
  const int32_t* pr = partial_rank + (size_t)t * M;
  float acc[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) acc[c] = 0.0f;
  for (int i0 = 0; i0 < M; i0 += kGroup) {
    bool used[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) used[g] = i0 + g < M && pr[i0 + g] >= 0;
    uint4 pv[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      pv[g] = active && used[g] ? load_stream(&partial[((size_t)t * M + i0 + g) * nvec + v])
                                : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      if (!used[g]) continue;
      const uint32_t q4[4] = {pv[g].x, pv[g].y, pv[g].z, pv[g].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        acc[2 * m] = acc[2 * m] + bf16_lo(q4[m]);
        acc[2 * m + 1] = acc[2 * m + 1] + bf16_hi(q4[m]);
      }
    }
  }
  if (!active) return;
  const uint4 o = make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                             pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7]));
  if constexpr (DS)
    store_device_scope(out + (size_t)t * nvec, nvec * 16, v * 16, o);
  else
    store_stream(&out[(size_t)t * nvec + v], o);
}

}  // namespace

hipError_t launch_combine_send(const void* y, const float* ys, const int32_t* token_row,
                               const int32_t* ids, const float* w, void* partial,
                               int32_t* partial_rank, int T, int H, int k, int E, int N,
                               int payload, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int M = min(k, N);
  const int nvec = payload == 0 ? H / 8 : H / 16;
  const int col_chunks = (nvec + kBlock - 1) / kBlock;
  const unsigned blocks = (unsigned)T * (unsigned)col_chunks;
  const int L = E / N;
  if (k <= kGroup) {
    // 64 vectors of 8 columns per block (bf16), 128 (fp8)
    const int chunks = (H / 8 + kBlock * (payload ? 2 : 1) - 1) / (kBlock * (payload ? 2 : 1));
    const unsigned nblk = (unsigned)T * (unsigned)chunks;
    const uint32_t l_magic = L >= 2 ? (uint32_t)(((1ull << 32) + L - 1) / L) : 0u;
#define MOE_SEND_SMALL(FP8, K)                                                              \
  hipLaunchKernelGGL((combine_send_small_kernel<FP8, K>), dim3(nblk), dim3(kBlock), 0, st, y, \
                     ys, token_row, ids, w, reinterpret_cast<uint4*>(partial), partial_rank,  \
                     H, k, E, L, l_magic, M, chunks, udiv_magic_of((uint32_t)chunks))
    if (payload == 0) {
      if (k == kGroup) MOE_SEND_SMALL(false, kGroup); else MOE_SEND_SMALL(false, 0);
    } else {
      if (k == kGroup) MOE_SEND_SMALL(true, kGroup); else MOE_SEND_SMALL(true, 0);
    }
#undef MOE_SEND_SMALL
    return hipGetLastError();
  }
  if (payload == 0)
    hipLaunchKernelGGL((combine_send_kernel<false, 8>), dim3(blocks), dim3(kBlock), 0, st,
                       reinterpret_cast<const uint4*>(y), ys, token_row, ids, w,
                       reinterpret_cast<uint4*>(partial), partial_rank, H, k, E, E / N, M,
                       col_chunks, udiv_magic_of((uint32_t)col_chunks));
  else
    hipLaunchKernelGGL((combine_send_kernel<true, 4>), dim3(blocks), dim3(kBlock), 0, st,
                       reinterpret_cast<const uint4*>(y), ys, token_row, ids, w,
                       reinterpret_cast<uint4*>(partial), partial_rank, H, k, E, E / N, M,
                       col_chunks, udiv_magic_of((uint32_t)col_chunks));
  return hipGetLastError();
}

hipError_t launch_combine_recv(const void* partial, const int32_t* partial_rank, void* out,
                               int T, int H, int M, hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int nvec = H / 8;
  const int col_chunks = (nvec + kBlock - 1) / kBlock;
  const dim3 grid((unsigned)T * (unsigned)col_chunks);
  const uint32_t cc_magic = udiv_magic_of((uint32_t)col_chunks);
  // output of 32 MB or more: device-scope stores (as in the receiver-side
  // combine; 4096-token prefill 74.0 -> 70.5 us, slower at decode sizes)
  const bool ds = (size_t)T * (size_t)H * 2 >= ((size_t)32 << 20);
#define MOE_RECV(MMV, DSV)                                                                 \
  hipLaunchKernelGGL((combine_recv_kernel<MMV, DSV>), grid, dim3(kBlock), 0, st,            \
                     reinterpret_cast<const uint4*>(partial), partial_rank,                \
                     reinterpret_cast<uint4*>(out), H, M, col_chunks, cc_magic)
  if (M == kGroup) {
    if (ds) MOE_RECV(kGroup, true); else MOE_RECV(kGroup, false);
  } else {
    if (ds) MOE_RECV(0, true); else MOE_RECV(0, false);
  }
#undef MOE_RECV
  return hipGetLastError();
}

}  // namespace moe
