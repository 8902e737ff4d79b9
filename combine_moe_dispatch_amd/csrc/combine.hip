// combine.hip -- receiver-side weighted sum of each token's returned rows.
//
// The combine receives the processed rows and forms their router-weighted
// average, accumulating only on the receiving side ("Enabling
// trillion-parameter models on AWS EFA", Introduction, Send and Receive
// Buffers, Evaluation).  A one-wave block owns one (token, 64-vector column
// chunk); the token's k rows and weights are read at uniform addresses (no
// LDS staging, no barrier), each thread issues its k 16-byte gathers together
// (8 at a time, unconditionally, so each row's fold waits for that row only)
// and folds them with fp32 fused multiply-adds in slot order from zero, then
// rounds to bf16 (nearest even, the hardware packed convert)
// and stores 16 bytes.  The gathers carry non-temporal (streaming) hints, and
// so do the stores of outputs below 32 MB (larger ones are stored with device
// scope).  With the fp8 payload a thread owns 16 columns: two 8-byte gathers
// of codes per row, each code decoded exactly to fp32 (the hardware OCP e4m3
// convert) and multiplied by its block's fp32 scale.  This is a
// bandwidth-bound gather-reduce: no MFMA.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 64;  // one wavefront per block
constexpr int kGroup = 8;   // gathers in flight per thread

#ifdef MOE_PHASE_STAMPS
// the combine kernels' trace buffer (tracing library only)
__device__ uint64_t* g_trace;
__device__ uint32_t g_trace_slots;
#endif

// Fold n gathered rows into acc with fp32 fused multiply-adds in slot order.
template <int N>
__device__ __forceinline__ void fold_rows(float (&acc)[8], const uint4 (&yv)[N],
                                          const int (&row)[N], const float (&wj)[N]) {
#pragma unroll
  for (int g = 0; g < N; ++g) {
    if (row[g] < 0) continue;
    const uint32_t q[4] = {yv[g].x, yv[g].y, yv[g].z, yv[g].w};
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      acc[2 * m] = fmaf(wj[g], bf16_lo(q[m]), acc[2 * m]);
      acc[2 * m + 1] = fmaf(wj[g], bf16_hi(q[m]), acc[2 * m + 1]);
    }
  }
}

// K > 0 (at most kGroup): top-k fixed at compile time, so the token's rows
// and weights are read first, as straight-line uniform loads, before anything
// else waits; K == 0: k at run time.  Rows are gathered kGroup at a time.
// DS: the output row is stored with device scope instead of non-temporally
// (chosen for large outputs).  token_major: grid x = token, y = column
// chunk, so the workgroups launched together read the same column chunk of
// many tokens' rows -- chosen when the whole grid is resident at once
// (DeepSeek-V3 decode 4.32 -> 4.22 us); otherwise x = column chunk, y =
// token, so a row's chunks run close together in time (4096-token prefill
// 91.8 -> 83.4 us).
template <int K, bool DS>
__global__ void __launch_bounds__(kBlock)
combine_bf16_kernel(const uint4* __restrict__ y, const int32_t* __restrict__ token_row,
                    const float* __restrict__ w, uint4* __restrict__ out, int H, int k_rt,
                    int token_major) {
  static_assert(K <= kGroup, "compile-time top-k is gathered in one group");
  MOE_STAMP(t_entry);
  MOE_STAMP_DECL(t_issued);
  const int k = K > 0 ? K : k_rt;
  const int t = token_major ? blockIdx.x : blockIdx.y;
  const int nvec = H / 8;
  const int v = (token_major ? blockIdx.y : blockIdx.x) * kBlock + threadIdx.x;
  const int32_t* trow = token_row + (size_t)t * k;
  const float* tw = w + (size_t)t * k;
  // no early exit before the gathers: lanes past the row end gather a
  // clamped column and skip the store, so nothing delays the uniform loads
  // of the token's rows
  const bool active = v < nvec;
  float acc[8];
#pragma unroll
  for (int m = 0; m < 8; ++m) acc[m] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kGroup) {
    int row[kGroup];
    float wj[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      row[g] = j0 + g < k ? trow[j0 + g] : -1;
      wj[g] = j0 + g < k ? tw[j0 + g] : 0.0f;
    }
    // the gathers are unconditional (row and column clamped; a skipped row is
    // left out of the fold), so the fold of each row waits for that row only
    uint4 yv[kGroup];
    const int vc = min(v, nvec - 1);
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      yv[g] = j0 + g < k ? load_stream(&y[(size_t)max(row[g], 0) * nvec + vc])
                         : make_uint4(0, 0, 0, 0);
    MOE_STAMP_SET(t_issued);
    fold_rows<kGroup>(acc, yv, row, wj);
    // every gathered value is consumed on every path, so no load is moved
    // into the fold's per-row branches
#pragma unroll
    for (int g = 0; g < kGroup; ++g)
      if (j0 + g < k) asm volatile("" ::"v"(yv[g].x));
  }
  MOE_STAMP(t_folded);
  if (!active) return;
  uint4 o;
  o.x = pack_bf16x2(acc[0], acc[1]);
  o.y = pack_bf16x2(acc[2], acc[3]);
  o.z = pack_bf16x2(acc[4], acc[5]);
  o.w = pack_bf16x2(acc[6], acc[7]);
  if constexpr (DS)
    store_device_scope(out + (size_t)t * nvec, nvec * 16, v * 16, o);
  else
    store_stream(&out[(size_t)t * nvec + v], o);
#ifdef MOE_PHASE_STAMPS
  MOE_STAMP(t_stored);
  MOE_TRACE_WAIT();
  MOE_STAMP(t_done);
  trace_record(g_trace, g_trace_slots, blockIdx.y * gridDim.x + blockIdx.x, t_entry, t_issued,
               t_folded, t_folded, t_stored, t_done);
#endif
}

// fp8: a lane owns two 8-code vectors, u and u + 64 of its block's 128, so
// that each 16-byte bf16 store instruction of the wave covers 1 KB of the
// output row without gaps (strided stores were measured to write back
// partial lines: 1.67x the output bytes).  16 consecutive vectors share one
// 128-column scale.  Workgroups are renumbered so that the column chunks of
// one token run on one XCD and share the L2 lines of the token's scales.
// K as for the bf16 kernel: K > 0 fixes top-k at compile time.
template <int K>
__global__ void __launch_bounds__(kBlock)
combine_fp8_kernel(const uint2* __restrict__ y, const float* __restrict__ ys,
                   const int32_t* __restrict__ token_row, const float* __restrict__ w,
                   uint4* __restrict__ out, int H, int k_rt, int col_chunks,
                   uint32_t cc_magic) {
  static_assert(K <= kGroup, "compile-time top-k is gathered in one group");
  const int k = K > 0 ? K : k_rt;
  const unsigned b = xcd_local_block(blockIdx.x, gridDim.x);
  const int t = (int)udiv_magic(b, (uint32_t)col_chunks, cc_magic);
  const int cc = b - t * col_chunks;
  const int nv = H / 8;
  const int nb = H / kFp8Block;
  const int u0 = cc * 2 * kBlock + threadIdx.x;
  const int u1 = u0 + kBlock;
  const int32_t* trow = token_row + (size_t)t * k;
  const float* tw = w + (size_t)t * k;
  // no early exit before the gathers (lanes past the row end mask them)
  const bool has0 = u0 < nv;
  const bool has1 = u1 < nv;
  float acc[16];
#pragma unroll
  for (int m = 0; m < 16; ++m) acc[m] = 0.0f;
  for (int j0 = 0; j0 < k; j0 += kGroup) {
    int row[kGroup];
    float wj[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      row[g] = j0 + g < k ? trow[j0 + g] : -1;
      wj[g] = j0 + g < k ? tw[j0 + g] : 0.0f;
    }
    uint2 c0[kGroup], c1[kGroup];
    float s0[kGroup], s1[kGroup];
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      const bool on = row[g] >= 0;
      const size_t r = on ? (size_t)row[g] : 0;
      c0[g] = on && has0 ? load_stream(&y[r * nv + u0]) : make_uint2(0, 0);
      c1[g] = on && has1 ? load_stream(&y[r * nv + u1]) : make_uint2(0, 0);
      s0[g] = on && has0 ? ys[r * nb + u0 / 16] : 0.0f;  // scales: cached loads
      s1[g] = on && has1 ? ys[r * nb + u1 / 16] : 0.0f;
    }
#pragma unroll
    for (int g = 0; g < kGroup; ++g) {
      if (row[g] < 0) continue;
      float dec[16];
      e4m3x4_to_f32(c0[g].x, dec);
      e4m3x4_to_f32(c0[g].y, dec + 4);
      e4m3x4_to_f32(c1[g].x, dec + 8);
      e4m3x4_to_f32(c1[g].y, dec + 12);
#pragma unroll
      for (int m = 0; m < 8; ++m) acc[m] = fmaf(wj[g], dec[m] * s0[g], acc[m]);
#pragma unroll
      for (int m = 8; m < 16; ++m) acc[m] = fmaf(wj[g], dec[m] * s1[g], acc[m]);
    }
  }
  if (!has0) return;
  uint4* o = out + (size_t)t * nv;
  store_stream(&o[u0], make_uint4(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                                  pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])));
  if (has1)
    store_stream(&o[u1], make_uint4(pack_bf16x2(acc[8], acc[9]), pack_bf16x2(acc[10], acc[11]),
                                    pack_bf16x2(acc[12], acc[13]), pack_bf16x2(acc[14], acc[15])));
}

}  // namespace

hipError_t launch_combine(const void* y, const float* ys, const int32_t* token_row,
                          const float* w, void* out, int T, int H, int k, int payload,
                          hipStream_t st) {
  if (T == 0) return hipSuccess;
  const int per_block = payload == 0 ? kBlock : 2 * kBlock;  // vectors of 8 columns
  const int col_chunks = (H / 8 + per_block - 1) / per_block;
  const unsigned blocks = (unsigned)T * (unsigned)col_chunks;
  const uint32_t cc_magic = udiv_magic_of((uint32_t)col_chunks);
  // bf16 output of 32 MB or more: device-scope stores (measured 3 % faster on
  // the 4096-token skewed prefill, slower at decode sizes)
  const bool ds = (size_t)T * (size_t)H * 2 >= ((size_t)32 << 20);
  // token-major block order when every one-wave block of the grid is
  // resident at once (8 waves per SIMD on 256 compute units), else chunk-major;
  // the token count goes in grid x either way when it exceeds y's limit
  const int token_major = (size_t)T * col_chunks <= 8192 || T > 65535 ? 1 : 0;
  const dim3 grid = token_major ? dim3((unsigned)T, (unsigned)col_chunks)
                                : dim3((unsigned)col_chunks, (unsigned)T);
  // compile-time top-k for the common values (the token's rows are then one
  // straight-line uniform load), run-time k otherwise
#define MOE_COMBINE(KK)                                                                   \
  do {                                                                                    \
    if (payload == 0 && ds)                                                               \
      hipLaunchKernelGGL((combine_bf16_kernel<KK, true>),                                  \
                         grid, dim3(kBlock), 0, st,                                         \
                         reinterpret_cast<const uint4*>(y), token_row, w,                 \
                         reinterpret_cast<uint4*>(out), H, k, token_major);                \
    else if (payload == 0)                                                                \
      hipLaunchKernelGGL((combine_bf16_kernel<KK, false>),                                 \
                         grid, dim3(kBlock), 0, st,                                         \
                         reinterpret_cast<const uint4*>(y), token_row, w,                 \
                         reinterpret_cast<uint4*>(out), H, k, token_major);                \
    else                                                                                  \
      hipLaunchKernelGGL(combine_fp8_kernel<KK>, dim3(blocks), dim3(kBlock), 0, st,       \
                         reinterpret_cast<const uint2*>(y), ys, token_row, w,             \
                         reinterpret_cast<uint4*>(out), H, k, col_chunks, cc_magic);      \
  } while (0)
  switch (k) {
    case 1: MOE_COMBINE(1); break;
    case 2: MOE_COMBINE(2); break;
    case 4: MOE_COMBINE(4); break;
    case 6: MOE_COMBINE(6); break;
    case 8: MOE_COMBINE(8); break;
    default: MOE_COMBINE(0); break;
  }
#undef MOE_COMBINE
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_PHASE_STAMPS
// Tracing library only: the buffer the bf16 combine kernel writes its phase
// records to (slots records of kTraceWords words, one per one-wave block in
// grid order), or null to stop.  Returns 0 or the HIP error code.
extern "C" int moe_trace_set_combine(void* buf, uint32_t slots) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_trace), &buf, sizeof(buf));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_trace_slots), &slots, sizeof(slots));
  return (int)e;
}
#endif
