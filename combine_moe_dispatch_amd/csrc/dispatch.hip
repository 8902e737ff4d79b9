// dispatch.hip -- MoE dispatch: count, scan, stable placement and scatter.
//
// What is computed ("Enabling trillion-parameter models on AWS EFA", sections
// Send and Receive Buffers and Dispatch and Combine): per-expert token counts,
// their cumulative sum giving the offset of each contiguous region, and the
// token rows packed into those regions.  Expert e lives on rank e / L.  Inside
// a rank's region the expert segments are ascending, and inside a segment the
// (token, slot) pairs are ascending, so the placement never depends on the
// order in which threads happen to run.
//
// The pages count with shared-memory atomics in a single block and then pack
// send buffers for a network write.  Here the receive regions are in this
// GPU's memory, so the pack is the final store, and the layout is derived
// without any order-dependent atomics:
//   row(t, j) = base(rank) + #{pairs of the rank with a smaller expert}
//               + #{earlier pairs (t', j') < (t, j) with the same expert}.
// (Histograms are built with LDS atomic adds, whose sums do not depend on the
// order the adds land in.)
//
// Two paths:
//  * fused (T*k <= kSmallMaxPairs): one launch.  Block 0 builds the global
//    histogram and scan and writes the metadata; every other block owns one
//    (token, column chunk).  It loads the whole id list (a few ids per
//    thread) and its slice of the token row at once, and builds one LDS
//    histogram holding two counts per expert (all ids; ids before this
//    token).  Lanes 0..k-1 then form their slots' rows: with fixed-capacity
//    regions of few experts per rank, from a direct sum over the rank's
//    counts; otherwise from a DPP scan of 64 chunk sums in every wave.  The
//    block stores its slice of the row k times.
//  * chunked (larger T*k): (1) per chunk of 1024 pairs, a block computes each
//    pair's rank among equal experts inside the chunk (wave ballot matching,
//    no atomics on the placement path) and the chunk's histogram; (2) one
//    block turns the chunk histograms into per-chunk bases and the global
//    metadata; (3) the scatter reads a pair's row from those (for sources
//    dispatching at once with every chunk inside one source, blocks past the
//    scatter's also write the per-source counts and offsets).  Up to 16
//    chunks, (1) and (2) are one launch: each chunk's block also counts the
//    ids of the chunks before it (its bases) and the last block writes the
//    metadata.
//
// Rows move as 16-byte vectors with non-temporal (streaming) hints.  With the
// fp8 payload a lane owns 16 columns and each group of 8 lanes one 128-column
// block: the group reduces its amax with DPP, each lane stores its 16 codes
// as one 16-byte vector, and the group's first lane the block's scale, per
// destination row.
#include "device_common.h"
#include "launch.h"

namespace moe {

namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;
constexpr int kDevCapacity = 1;
constexpr int kDevBadId = 2;
constexpr int kComputeUnits = 256;  // MI355X

#ifdef MOE_PHASE_STAMPS
// the dispatch kernels' trace buffer (tracing library only)
__device__ uint64_t* g_trace;
__device__ uint32_t g_trace_slots;
#endif

// Exclusive scan of n <= kMaxExperts LDS counts into excl[0..n] (excl[n] is
// the total).  All threads of the block must call it.
__device__ void block_exclusive_scan(const int* cnt, int n, int* excl, int* wave_tot) {
  const int per = (n + kBlock - 1) / kBlock;
  const int start = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i)
    if (start + i < n) local += cnt[start + i];
  const int incl = wave_inclusive_sum_dpp(local);
  const int w = threadIdx.x / kWave;
  if (lane_id() == kWave - 1) wave_tot[w] = incl;
  lds_barrier();  // LDS only: global stores still in flight are not waited for
  int run = incl - local;
  for (int i = 0; i < w; ++i) run += wave_tot[i];
  for (int i = 0; i < per; ++i)
    if (start + i < n) {
      excl[start + i] = run;
      run += cnt[start + i];
    }
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int i = 0; i < kWaves; ++i) tot += wave_tot[i];
    excl[n] = tot;
  }
  lds_barrier();
}

// Global metadata from the per-expert counts and their exclusive scan.
__device__ void write_metadata(const DispatchParams& p, const int* cnt, const int* excl,
                               bool bad) {
  for (int e = threadIdx.x; e < p.E; e += kBlock) {
    const int r = p.L == 1 ? e : (int)__umulhi((uint32_t)e, p.l_magic);
    const int first = excl[r * p.L];
    const int base = p.C > 0 ? r * p.C : first;
    p.expert_counts[e] = cnt[e];
    p.expert_offsets[e] = base + excl[e] - first;
  }
  bool over = false;
  for (int r = threadIdx.x; r < p.N; r += kBlock) {
    const int rc = excl[(r + 1) * p.L] - excl[r * p.L];
    p.rank_counts[r] = rc;
    p.rank_offsets[r] = p.C > 0 ? r * p.C : excl[r * p.L];
    if (p.C > 0 && rc > p.C) over = true;
  }
  over = __syncthreads_or(over);
  if (threadIdx.x == 0) *p.status = (bad ? kDevBadId : 0) | (over ? kDevCapacity : 0);
}

// ---------------------------------------------------------------------------
// Scatter of one token's column slice to its k destination rows.  In every
// wave, lane j < k holds the row of slot j (-1 = skipped); the store loop
// reads it with readlane, so no LDS staging or barrier is needed.
// ---------------------------------------------------------------------------
// A thread's unit of a row: 8 columns (one 16-byte bf16 vector) for the bf16
// payload, 16 columns (two bf16 vectors in, one 16-byte vector of codes out)
// for fp8.
template <int PAYLOAD>
struct Unit {
  static constexpr int kXV = PAYLOAD ? 2 : 1;  // 16-byte x vectors per unit
  static constexpr int kCols = 8 * kXV;
};

__host__ __device__ __forceinline__ int units_per_row(const DispatchParams& p) {
  return p.H / (p.payload ? 16 : 8);
}

template <int PAYLOAD, int MAXV>
__device__ __forceinline__ void load_slice(const DispatchParams& p, int t, int u0, int u1,
                                           uint4 (&xv)[MAXV][Unit<PAYLOAD>::kXV]) {
  constexpr int kXV = Unit<PAYLOAD>::kXV;
  const uint4* x = reinterpret_cast<const uint4*>(p.x) + (size_t)t * (p.H / 8);
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int u = u0 + threadIdx.x + i * kBlock;
    const int uc = min(u, u1 - 1);  // clamped: units past u1 are loaded but never stored
#pragma unroll
    for (int c = 0; c < kXV; ++c) xv[i][c] = load_stream(&x[kXV * uc + c]);
  }
}

template <int MAXV>
__device__ __forceinline__ void store_bf16(const DispatchParams& p, int u0, int u1,
                                           const uint4 (&xv)[MAXV][1], int row_lane,
                                           int lane0) {
  const int nvec = p.H / 8;
  uint4* recv = reinterpret_cast<uint4*>(p.recv);
  for (int j = 0; j < p.k; ++j) {
    const int row = __builtin_amdgcn_readlane(row_lane, lane0 + j);
    if (row < 0) continue;
    uint4* dst = recv + (size_t)row * nvec;
#pragma unroll
    for (int i = 0; i < MAXV; ++i) {
      const int u = u0 + threadIdx.x + i * kBlock;
      if (u < u1) store_stream(&dst[u], xv[i][0]);
    }
  }
}

// Max over each group of 8 lanes (half of a DPP row): lane ^ 1, lane ^ 2,
// then the mirrored quad, so every lane ends with its group's max.
__device__ __forceinline__ float lanes8_max(float v) {
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xf, 0xf, false)));
  v = fmaxf(v, __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x141, 0xf, 0xf, false)));
  return v;
}

// fp8: a unit is 16 columns; 8 consecutive lanes hold one 128-column block
// (u0 and u1 are multiples of 8, so a group is all in or all out).  Each
// lane stores its 16 codes as one 16-byte vector, the group's first lane the
// block's scale.
template <int MAXV>
__device__ __forceinline__ void store_fp8(const DispatchParams& p, int u0, int u1,
                                          const uint4 (&xv)[MAXV][2], int row_lane, int lane0) {
  const int nb = p.H / kFp8Block;
  const int nu = p.H / 16;
#pragma unroll
  for (int i = 0; i < MAXV; ++i) {
    const int u = u0 + threadIdx.x + i * kBlock;
    float f[16];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const uint32_t w4[4] = {xv[i][c].x, xv[i][c].y, xv[i][c].z, xv[i][c].w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        f[8 * c + 2 * m] = bf16_lo(w4[m]);
        f[8 * c + 2 * m + 1] = bf16_hi(w4[m]);
      }
    }
    float amax = 0.0f;
#pragma unroll
    for (int m = 0; m < 16; ++m) amax = fmaxf(amax, fabsf(f[m]));
    amax = lanes8_max(amax);
    if (u >= u1) continue;
    const float s = amax / 448.0f;
    uint32_t code[4] = {0, 0, 0, 0};
    if (amax != 0.0f) {
      if (s >= 0x1p-80f && s <= 0x1p80f) {
        // x / s without a division per element: from the correctly rounded
        // reciprocal r, q0 = x * r and one remainder correction
        // q = q0 + r * (x - s * q0) (fused) give the correctly rounded
        // quotient when nothing underflows (Markstein's division), which
        // this range of s guarantees for every |q| that can round to a
        // non-zero code.  |q| <= 448 (1 + 2^-23)^2 here, where the gfx950
        // packed convert rounds to nearest even exactly like f32_to_e4m3
        // (checked for every finite fp32 below 464).
        const float r = 1.0f / s;
        float q[16];
#pragma unroll
        for (int m = 0; m < 16; ++m) {
          const float q0 = f[m] * r;
          // a signed zero is its own quotient; the correction would turn -0
          // into +0 (the remainder is +0, and +0 + -0 rounds to +0)
          q[m] = f[m] == 0.0f ? f[m] : fmaf(fmaf(-s, q0, f[m]), r, q0);
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(q[4 * w], q[4 * w + 1], 0, false);
          code[w] = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(q[4 * w + 2], q[4 * w + 3], lo, true);
        }
      } else {
#pragma unroll
        for (int m = 0; m < 16; ++m) code[m / 4] |= f32_to_e4m3(f[m] / s) << (8 * (m % 4));
      }
    }
    const uint4 cv = make_uint4(code[0], code[1], code[2], code[3]);
    for (int j = 0; j < p.k; ++j) {
      const int row = __builtin_amdgcn_readlane(row_lane, lane0 + j);
      if (row < 0) continue;
      uint4* dst = reinterpret_cast<uint4*>(p.recv) + (size_t)row * nu;
      store_stream(&dst[u], cv);
      // scales are plain stores: a wave writes only 32 bytes of a row's
      // scales, and the L2 merges the pieces of one row into whole lines
      // (measured faster than streaming them)
      if ((threadIdx.x & 7) == 0) p.recv_scales[(size_t)row * nb + u / 8] = s;
    }
  }
}

// The rows of the token's slots j = 0..k-1 are in lanes lane0 + j.
template <int PAYLOAD, int MAXV>
__device__ __forceinline__ void store_slice(const DispatchParams& p, int u0, int u1,
                                            const uint4 (&xv)[MAXV][Unit<PAYLOAD>::kXV],
                                            int row_lane, int lane0 = 0) {
  if constexpr (PAYLOAD == 0)
    store_bf16<MAXV>(p, u0, u1, xv, row_lane, lane0);
  else
    store_fp8<MAXV>(p, u0, u1, xv, row_lane, lane0);
}

// Blocks of column chunk 0, wave 0: lane i publishes the row of pair q0 + i,
// for the block's n pairs.
__device__ __forceinline__ void publish_rows(const DispatchParams& p, int q0, int n, int cc,
                                             int row_lane) {
  if (cc == 0 && (int)threadIdx.x < n) {
    const int q = q0 + threadIdx.x;
    p.token_row[q] = row_lane;
    if (p.row_src && row_lane >= 0) p.row_src[row_lane] = q;
  }
}

// Experts per scan chunk: 64 chunks cover E; a power of two >= 4 so that a
// chunk is read as whole 16-byte LDS vectors.
__device__ __forceinline__ int chunk_size(int E) {
  const int c = (E + kWave - 1) / kWave;
  return c <= 4 ? 4 : (c <= 8 ? 8 : 16);
}

// Sum of the first `upto` entries of chunk `ci` (csz entries, 16-byte aligned).
__device__ __forceinline__ int chunk_sum_below(const int* hist, int ci, int csz, int upto) {
  const int4* c4 = reinterpret_cast<const int4*>(hist + ci * csz);
  int4 q[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) q[i] = (4 * i < csz) ? c4[i] : make_int4(0, 0, 0, 0);
  int s = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s += (4 * i + 0 < upto) ? q[i].x : 0;
    s += (4 * i + 1 < upto) ? q[i].y : 0;
    s += (4 * i + 2 < upto) ? q[i].z : 0;
    s += (4 * i + 3 < upto) ? q[i].w : 0;
  }
  return s;
}

// Rank of expert e (e / L) without a division: e and L are below 2^10 here,
// so the rounded-up reciprocal is exact (e * L < 2^32).
__device__ __forceinline__ int rank_of(const DispatchParams& p, int e) {
  return p.L == 1 ? e : (int)__umulhi((uint32_t)e, p.l_magic);
}

// Ranks of at most this many experts take the direct in-rank prefix.
constexpr int kDirectMaxL = 32;

// Sum of hist[first .. e), first = the rank's first expert, e inside the rank
// (e < first + L <= first + 4 * NV, NV <= kDirectMaxL / 4).  With L % 4 == 0
// the 4 * NV words from first are read as 16-byte vectors, unconditionally and
// all before the first is used (hist holds kDirectMaxL words of padding past
// its last expert).  NV is fixed at compile time from L (2 for L <= 8, 4 for
// L <= 16, else 8), so a rank of few experts reads and sums only its own
// words.  Up to 4 vectors, every word at or past e is masked out; at 8, the
// sum is that of the whole vectors below e's vector plus the words of e's
// vector below e (read once more), one select per vector and three for the
// partial one instead of one per word -- each select is a 4-cycle instruction
// for a 64-lane wave (Kimi-K2 decode, 24 experts per rank: 4.35 -> 4.27 us;
// for 8 experts per rank the extra read cost more than it saved, 4.16 -> 4.21).
typedef int v4i __attribute__((ext_vector_type(4)));

template <int NV>
__device__ __forceinline__ int rank_prefix(const v4i* hist4, int first, int e, int L) {
  static_assert(NV <= kDirectMaxL / 4, "reads stay inside the padding");
  if ((L & 3) == 0) {
    const v4i* h4 = hist4 + (first >> 2);  // first is a multiple of 4 here
    v4i q[NV];
#pragma unroll
    for (int c = 0; c < NV; ++c) q[c] = h4[c];
    if constexpr (NV >= 8) {
      const int n = e - first;   // words of the window below e, 0 .. L - 1
      const int nfull = n >> 2;  // whole vectors below e's vector
      const v4i part = h4[nfull];
      int s = 0;
#pragma unroll
      for (int c = 0; c < NV; ++c) s += c < nfull ? (q[c].x + q[c].y) + (q[c].z + q[c].w) : 0;
      const int r = n & 3;
      return s + (r > 0 ? part.x : 0) + (r > 1 ? part.y : 0) + (r > 2 ? part.z : 0);
    } else {
      const v4i lanes = {0, 1, 2, 3};
      const v4i zero = {0, 0, 0, 0};
      v4i acc = zero;
#pragma unroll
      for (int c = 0; c < NV; ++c) acc += (lanes + (first + 4 * c) < e) ? q[c] : zero;
      return acc.x + acc.y + acc.z + acc.w;
    }
  }
  const int* hist = reinterpret_cast<const int*>(hist4);
  int s = 0;
  for (int x = first; x < e; ++x) s += hist[x];
  return s;
}

// Number of lanes j' < lane (slots of the same token) holding the same
// non-zero key; key 0 marks an invalid slot.  k <= 8: the slots sit in lanes
// 0..7 of the first DPP row, so seven row shifts compare every earlier slot
// (lanes shifted in from outside the row read 0); larger k: a readlane loop.
__device__ __forceinline__ int earlier_same_slots(int key, int lane, int k) {
  int n = 0;
  if (k <= 8) {
#define MOE_SAME_AT(D) \
  n += (int)((key != 0) & (__builtin_amdgcn_update_dpp(0, key, 0x110 + (D), 0xf, 0xf, true) == key))
    MOE_SAME_AT(1);
    MOE_SAME_AT(2);
    MOE_SAME_AT(3);
    MOE_SAME_AT(4);
    MOE_SAME_AT(5);
    MOE_SAME_AT(6);
    MOE_SAME_AT(7);
#undef MOE_SAME_AT
  } else {
    for (int j = 0; j < k; ++j) {
      const int o = __builtin_amdgcn_readlane(key, j);
      n += (j < lane && key != 0 && o == key) ? 1 : 0;
    }
  }
  return n;
}

__device__ __forceinline__ int checked_row(const DispatchParams& p, int row) {
  return (row >= 0 && row < p.rows) ? row : -1;
}

// ---------------------------------------------------------------------------
// Fused single-launch path.
// ---------------------------------------------------------------------------
// IPT = ids per thread (T*k <= IPT * kBlock).  RT = tokens per scatter
// block: a block owns column chunk cc of the run of RT consecutive tokens
// t0 .. t0 + RT - 1 (RT * k <= 64, so lane i of every wave holds pair
// t0 * k + i of the run), and counts the id list once for all of them.  Every
// global load below is unconditional (indices clamped into range, values
// masked afterwards), so the compiler can count loads in flight exactly and
// wait only for the ids before the histograms, not for the x slices issued
// after them.  NVR: the 16-byte vectors rank_prefix reads (at least L / 4 on
// its direct path).
template <int PAYLOAD, int MAXV, int IPT, int NVR, int RT>
__global__ void __launch_bounds__(kBlock) dispatch_fused_kernel(DispatchParams p) {
  // histogram (packed pair in the scatter blocks), padded for rank_prefix
  __shared__ __align__(16) int s_a[kMaxExperts + kDirectMaxL];
  __shared__ int s_b[kMaxExperts + 1];  // block 0: its exclusive scan
  __shared__ int s_wave[kWaves];
  const int P = p.T * p.k;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  // the scatter blocks' arguments come with the first batch of argument
  // loads, not a round trip after the branch below
  MOE_ARGS_UP_FRONT("s"(p.x), "s"(p.col_chunks), "s"(p.cc_magic), "s"(p.vec_per_chunk), "s"(p.H));

  if (blockIdx.x == 0) {
    MOE_STAMP(t_entry0);
    // histogram, scan and the global metadata; all id loads are issued
    // before the first one is used
    int idv[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i) idv[i] = P > 0 ? p.ids[min(tid + i * kBlock, P - 1)] : 0;
    for (int e = tid; e < p.E; e += kBlock) s_a[e] = 0;
    __syncthreads();
    bool bad = false;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (tid + i * kBlock < P) {
        const int e = idv[i];
        if ((unsigned)e < (unsigned)p.E)
          atomicAdd(&s_a[e], 1);
        else
          bad = true;
      }
    }
    bad = __syncthreads_or(bad);
    block_exclusive_scan(s_a, p.E, s_b, s_wave);
    write_metadata(p, s_a, s_b, bad);
#ifdef MOE_PHASE_STAMPS
    MOE_STAMP(t_issued0);
    MOE_TRACE_WAIT();
    MOE_STAMP(t_done0);
    trace_record(g_trace, g_trace_slots, threadIdx.x / kWave, t_entry0, t_entry0, t_entry0,
                 t_entry0, t_issued0, t_done0);
#endif
    return;
  }

  MOE_STAMP(t_entry);
  // issue every load first: the whole id list (a few per thread; these do
  // not depend on the block's tokens), the run's ids and this block's slice
  // of each of the run's token rows
  int idv[IPT];
#pragma unroll
  for (int i = 0; i < IPT; ++i) idv[i] = p.ids[min(tid + i * kBlock, P - 1)];
  const int b = blockIdx.x - 1;
  const int g = (int)udiv_magic((uint32_t)b, (uint32_t)p.col_chunks, p.cc_magic);
  const int cc = b - g * p.col_chunks;
  const int t0 = g * RT;
  const int q0 = t0 * p.k;                 // the run's first pair
  const int npairs = min(RT * p.k, P - q0);  // and its number of pairs
  const int u0 = cc * p.vec_per_chunk;
  const int u1 = min(u0 + p.vec_per_chunk, p.H >> (PAYLOAD ? 4 : 3));
  const int my_e_raw = p.ids[q0 + min(lane, npairs - 1)];
  uint4 xv[RT][MAXV][Unit<PAYLOAD>::kXV];
#pragma unroll
  for (int i = 0; i < RT; ++i) load_slice<PAYLOAD, MAXV>(p, min(t0 + i, p.T - 1), u0, u1, xv[i]);
  const int my_e = lane < npairs ? my_e_raw : -1;  // lane i: expert of pair q0 + i

  // Two histograms in one: s_a[e] counts all ids == e in its low 16 bits and
  // the ids == e at positions before the run's pairs in its high 16 bits
  // (T*k < 2^16, so sums of these words never carry from the low half into
  // the high half: a masked sum is a count).  s_a is cleared up to 64 whole
  // chunks, so chunk reads see zeros past E.
  const int csz = chunk_size(p.E);
  for (int e = tid; e < kWave * csz; e += kBlock) s_a[e] = 0;
  // LDS-only barriers from here on: the slices of x loaded above stay in
  // flight while the histogram is built
  lds_barrier();
  MOE_STAMP(t_clear);
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int q = tid + i * kBlock;
    const int e = idv[i];
    if (q < P && (unsigned)e < (unsigned)p.E) atomicAdd(&s_a[e], q < q0 ? 0x10001 : 1);
  }
  // while the adds land: earlier pairs of the run with the same expert (one
  // token: DPP row shifts over its k slots; a run: ballot matching)
  const bool valid = lane < npairs && (unsigned)my_e < (unsigned)p.E;
  int dup;
  if constexpr (RT == 1) {
    dup = earlier_same_slots(valid ? my_e + 1 : 0, lane, p.k);
  } else {
    const uint32_t key = valid ? (uint32_t)my_e : (uint32_t)p.E;
    dup = popc64(wave_match(key, 32 - __clz(p.E)) & lanes_below());
  }
  lds_barrier();
  MOE_STAMP(t_hist);

  // Lane i, for the expert e of pair q = q0 + i:
  //   B = #ids == e at positions before q (histogram of the pairs before the
  //       run plus the run's earlier pairs);
  //   fixed-capacity regions: the row is r*C + #ids in [first, e) + B, where
  //       first is the first expert of e's rank r -- with L <= kDirectMaxL a
  //       direct sum over the rank's counts;
  //   otherwise every wave scans 64 chunk sums of csz experts with DPP and
  //       reads off A = #valid ids below e (and F = #valid ids below first).
  const int e = valid ? my_e : 0;
  const int r = rank_of(p, e);
  const int first = r * p.L;
  int row = -1;
  if (p.C > 0 && p.L <= kDirectMaxL) {
    // the LDS reads of this path are issued together, after the branch
    const int b_hist = s_a[e] >> 16;
    const int local =
        (rank_prefix<NVR>(reinterpret_cast<const v4i*>(s_a), first, e, p.L) & 0xffff) + b_hist +
        dup;
    if (valid && local < p.C) row = r * p.C + local;
  } else {
    const int b_hist = s_a[e] >> 16;
    // all LDS reads of this phase are independent and issued together
    const int csum = chunk_sum_below(s_a, lane, csz, csz);
    const int a_part = chunk_sum_below(s_a, e / csz, csz, e % csz);
    const int f_part = chunk_sum_below(s_a, first / csz, csz, first % csz);
    const int cexcl = wave_inclusive_sum_dpp(csum) - csum;
    const int A = (__shfl(cexcl, e / csz, kWave) + a_part) & 0xffff;
    const int F = (__shfl(cexcl, first / csz, kWave) + f_part) & 0xffff;
    if (valid) {
      const int B = b_hist + dup;
      if (p.C > 0) {
        const int local = (A - F) + B;
        if (local < p.C) row = r * p.C + local;
      } else {
        row = A + B;
      }
    }
  }
  row = checked_row(p, row);
  MOE_STAMP(t_rows);
  // payload first: the metadata stores come after it, so the wait for the x
  // slices before the payload stores is not also a wait for them
#pragma unroll
  for (int i = 0; i < RT; ++i) {
    if (t0 + i >= p.T) break;
    store_slice<PAYLOAD, MAXV>(p, u0, u1, xv[i], row, i * p.k);
  }
  publish_rows(p, q0, npairs, cc, row);
#ifdef MOE_PHASE_STAMPS
  MOE_STAMP(t_issued);
  MOE_TRACE_WAIT();
  MOE_STAMP(t_done);
  trace_record(g_trace, g_trace_slots, blockIdx.x * kWaves + threadIdx.x / kWave, t_entry,
               t_clear, t_hist, t_rows, t_issued, t_done);
#endif
}

// ---------------------------------------------------------------------------
// Chunked path: ranks inside a chunk and the chunk's counts.
// ---------------------------------------------------------------------------
// The chunk's 1024 pairs form 16 groups of 64 (one wave's pairs per pass), in
// pair order.  Each wave ranks its pairs among equal experts in its group by
// ballot matching and the group's last equal pair records the group count;
// one pass over the groups per expert turns the counts into exclusive
// prefixes and the chunk's count of the expert (stored to count[e], global or
// LDS), so a pair's rank in the chunk is its group's prefix plus its rank in
// the group.  Three barriers; every thread of the block calls it.  Returns
// whether this thread saw an id outside [0, E).
static_assert(kChunkPairs < (1 << 16), "in-chunk prefixes are held in 16 bits");
constexpr int kChunkSubs = kChunkPairs / kBlock;
constexpr int kChunkGroups = kChunkSubs * kWaves;

__device__ __forceinline__ bool rank_chunk(const DispatchParams& p, int c, uint16_t* s_grp,
                                           int32_t* count) {
  const int P = p.T * p.k;
  const int E = p.E;
  const int tid = threadIdx.x;
  const int w = tid / kWave;

  int idv[kChunkSubs];
#pragma unroll
  for (int s = 0; s < kChunkSubs; ++s)
    idv[s] = p.ids[min(c * kChunkPairs + s * kBlock + tid, P - 1)];
  {
    int4* g4 = reinterpret_cast<int4*>(s_grp);
    for (int i = tid; i < kChunkGroups * E / 8; i += kBlock) g4[i] = make_int4(0, 0, 0, 0);
  }
  // LDS-only barriers: they order the histogram exchanges, not the global
  // stores of the ranks (read by a later kernel)
  lds_barrier();

  const int bits = 32 - __clz(E);  // keys 0..E, E marks "no valid id"
  bool bad = false;
  int before[kChunkSubs];
#pragma unroll
  for (int s = 0; s < kChunkSubs; ++s) {
    const int q = c * kChunkPairs + s * kBlock + tid;
    const bool has = q < P;
    const int e = idv[s];
    const bool valid = has && (unsigned)e < (unsigned)E;
    bad |= has && !valid;
    const uint32_t key = valid ? (uint32_t)e : (uint32_t)E;
    const uint64_t peers = wave_match(key, bits);
    before[s] = popc64(peers & lanes_below());
    const int total = popc64(peers);
    if (valid && before[s] == total - 1) s_grp[(s * kWaves + w) * E + e] = (uint16_t)total;
  }
  lds_barrier();
  for (int e = tid; e < E; e += kBlock) {
    int n[kChunkGroups];
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) n[g] = s_grp[g * E + e];
    int run = 0;
#pragma unroll
    for (int g = 0; g < kChunkGroups; ++g) {
      s_grp[g * E + e] = (uint16_t)run;
      run += n[g];
    }
    count[e] = run;
  }
  lds_barrier();
#pragma unroll
  for (int s = 0; s < kChunkSubs; ++s) {
    const int q = c * kChunkPairs + s * kBlock + tid;
    const int e = idv[s];
    if (q < P && (unsigned)e < (unsigned)E)
      p.local_rank[q] = s_grp[(s * kWaves + w) * E + e] + before[s];
  }
  return bad;
}

// Chunked path, kernel 1 of 3: the chunk's ranks and histogram.
__global__ void __launch_bounds__(kBlock) layout_chunk_kernel(DispatchParams p) {
  // [group][expert]: counts <= 64, then prefixes <= kChunkPairs: 16 bits
  __shared__ __align__(16) uint16_t s_grp[kChunkGroups * kMaxExperts];
  const int c = blockIdx.x;
  bool bad = rank_chunk(p, c, s_grp, p.chunk_hist + (size_t)c * p.E);
  bad = __syncthreads_or(bad);
  if (threadIdx.x == 0) p.chunk_bad[c] = bad ? 1 : 0;
}

// Chunked path with at most kBaseCountMaxChunks chunks: one launch in place
// of kernels 1 and 2.  Block c counts the ids of the chunks before it into an
// LDS histogram, which is the chunk's base for each expert, and ranks its own
// chunk; the last block's bases plus its own chunk's counts are the global
// counts, from which it writes the metadata.  Block c reads c chunks of ids
// besides its own (the last block the whole list), 16-byte loads 16 deep per
// thread.  Up to 16 chunks that costs less than the scan launch (DeepSeek-V3
// shape, 1536 tokens: 48.7 -> 46.9 us); at 32 chunks it costs more (4096-token
// prefill: 106.5 -> 108.6 us), as the last block's count grows with the list.
constexpr int kBaseCountMaxChunks = 16;
constexpr int kCountDepth = 16;  // int4 loads in flight per thread

__global__ void __launch_bounds__(kBlock) layout_bases_kernel(DispatchParams p) {
  __shared__ __align__(16) uint16_t s_grp[kChunkGroups * kMaxExperts];
  __shared__ int s_base[kMaxExperts];
  __shared__ int s_own[kMaxExperts];
  __shared__ int s_excl[kMaxExperts + 1];
  __shared__ int s_wave[kWaves];
  const int c = blockIdx.x;
  const int E = p.E;
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kBlock) s_base[e] = 0;
  lds_barrier();

  // the earlier chunks' ids: whole chunks, so every vector is in range
  const int4* ids4 = reinterpret_cast<const int4*>(p.ids);
  const int nvec = c * (kChunkPairs / 4);
  bool bad = false;
  for (int v0 = 0; v0 < nvec; v0 += kCountDepth * kBlock) {
    int4 v[kCountDepth];
#pragma unroll
    for (int d = 0; d < kCountDepth; ++d) v[d] = ids4[min(v0 + d * kBlock + tid, nvec - 1)];
#pragma unroll
    for (int d = 0; d < kCountDepth; ++d) {
      if (v0 + d * kBlock + tid < nvec) {
        const int e4[4] = {v[d].x, v[d].y, v[d].z, v[d].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if ((unsigned)e4[i] < (unsigned)E)
            atomicAdd(&s_base[e4[i]], 1);
          else
            bad = true;
        }
      }
    }
  }
  // rank_chunk's barriers order the adds above before the reads below
  bad |= rank_chunk(p, c, s_grp, s_own);
  const bool last = c == p.nchunks - 1;
  for (int e = tid; e < E; e += kBlock) {
    const int b = s_base[e];
    p.chunk_hist[(size_t)c * E + e] = b;
    if (last) s_base[e] = b + s_own[e];
  }
  if (!last) return;  // whole block
  bad = __syncthreads_or(bad);
  block_exclusive_scan(s_base, E, s_excl, s_wave);
  write_metadata(p, s_base, s_excl, bad);
}

// Chunked path, kernel 2 of 3: per-chunk bases (exclusive over chunks, in place),
// global counts, scan and metadata.  One block; a thread per expert issues
// the loads of 32 chunks at once.
__global__ void __launch_bounds__(kBlock) layout_scan_kernel(DispatchParams p) {
  __shared__ int s_cnt[kMaxExperts];
  __shared__ int s_excl[kMaxExperts + 1];
  __shared__ int s_wave[kWaves];
  constexpr int kBatch = 32;
  const int tid = threadIdx.x;
  for (int e = tid; e < p.E; e += kBlock) {
    int run = 0;
    for (int c0 = 0; c0 < p.nchunks; c0 += kBatch) {
      int h[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        h[i] = p.chunk_hist[(size_t)min(c0 + i, p.nchunks - 1) * p.E + e];
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (c0 + i < p.nchunks) {
          p.chunk_hist[(size_t)(c0 + i) * p.E + e] = run;
          run += h[i];
        }
    }
    s_cnt[e] = run;
  }
  bool bad = false;
  for (int c = tid; c < p.nchunks; c += kBlock) bad |= p.chunk_bad[c] != 0;
  bad = __syncthreads_or(bad);
  block_exclusive_scan(s_cnt, p.E, s_excl, s_wave);
  write_metadata(p, s_cnt, s_excl, bad);
}

// Sources dispatching at once, every chunk inside one source: the base of
// source s's first chunk for expert e counts e's ids in the sources before s,
// so source s's block of expert e begins at expert_offsets[e] plus that base
// and holds the difference to the next source's base (the expert's total
// after the last source).  One wave per expert, lanes over sources.
__device__ __forceinline__ void source_metadata_from_bases(const DispatchParams& p, unsigned b) {
  const int e = (int)b * kWaves + (int)threadIdx.x / kWave;
  if (e >= p.E) return;  // whole wave
  const int lane = lane_id();
  const int off = p.expert_offsets[e];
  const int total = p.expert_counts[e];
  const size_t stride = (size_t)p.src_cps * p.E;
  for (int s0 = 0; s0 < p.src_S; s0 += kWave) {
    const int s = s0 + lane;
    const int b0 = s < p.src_S ? p.chunk_hist[(size_t)s * stride + e] : 0;
    const int b1 = s + 1 < p.src_S ? p.chunk_hist[(size_t)(s + 1) * stride + e] : total;
    if (s < p.src_S) {
      p.src_offsets[(size_t)e * p.src_S + s] = off + b0;
      p.src_counts[(size_t)s * p.E + e] = b1 - b0;
    }
  }
}

// Chunked path, last kernel: rows from the chunk bases, then the scatter (and,
// for sources dispatching at once, the per-source metadata in the blocks past
// the scatter's).
template <int PAYLOAD, int MAXV>
__global__ void __launch_bounds__(kBlock) dispatch_scatter_kernel(DispatchParams p) {
  const unsigned scatter_blocks = (unsigned)p.T * (unsigned)p.col_chunks;
  if (blockIdx.x >= scatter_blocks) {
    source_metadata_from_bases(p, blockIdx.x - scatter_blocks);
    return;
  }
  const int t = (int)udiv_magic(blockIdx.x, (uint32_t)p.col_chunks, p.cc_magic);
  const int cc = blockIdx.x - t * p.col_chunks;
  const int u0 = cc * p.vec_per_chunk;
  const int u1 = min(u0 + p.vec_per_chunk, p.H >> (PAYLOAD ? 4 : 3));
  const int lane = lane_id();
  // Loads in dependency order, all unconditional (indices clamped, values
  // masked), so each wait covers only what it needs: the slot's id and
  // in-chunk rank; then, from the id, the chunk base and the expert offset;
  // then the x slice, which stays in flight while the row is formed.
  const int q = t * p.k + min(lane, p.k - 1);
  const int e = p.ids[q];
  const int lr = p.local_rank[q];
  const bool valid = lane < p.k && (unsigned)e < (unsigned)p.E;
  const int ec = valid ? e : 0;
  const int base = p.chunk_hist[(size_t)(q / kChunkPairs) * p.E + ec];
  const int eoff = p.expert_offsets[ec];
  uint4 xv[MAXV][Unit<PAYLOAD>::kXV];
  load_slice<PAYLOAD, MAXV>(p, t, u0, u1, xv);
  int row = -1;
  if (valid) {
    const int pos = base + lr;
    if (p.C > 0) {
      const int r = e / p.L;
      const int local = eoff - r * p.C + pos;
      if (local < p.C) row = r * p.C + local;
    } else {
      row = eoff + pos;
    }
  }
  row = checked_row(p, row);
  // payload first: the metadata stores come after it, so the wait for the x
  // slice before the payload stores is not also a wait for them
  store_slice<PAYLOAD, MAXV>(p, u0, u1, xv, row);
  publish_rows(p, t * p.k, p.k, cc, row);
}

static_assert(kSmallMaxPairs <= 32 * kBlock, "the fused path loads at most 32 ids per thread");
static_assert(kSmallMaxPairs < (1 << 16), "packed histogram halves hold counts up to T*k");

// Runs of tokens per scatter block, only where each block recounts 32 ids per
// thread (T*k > 4096) and a block per (token, column chunk) would put six or
// more blocks on each compute unit: there the recount outweighs what fewer
// blocks lose in stores in flight, as long as about two blocks per compute
// unit remain.  Measured at the DeepSeek-V3 shape (k = 8, two column chunks):
// 768 tokens 21.9 -> 19.9 us and 1024 tokens 29.2 -> 25.5 us with runs of 2
// and 4, the fp8 payload at 1024 tokens 21.2 -> 16.1 us; at 513 and 600 tokens
// (four and five blocks per compute unit) runs of two measured 2 % slower, and
// with 16 ids per thread or fewer runs were slower throughout (fp8 payload at
// 512 tokens 8.17 -> 8.83 us).
constexpr int kRunsFromBlocks = 6 * kComputeUnits;
constexpr int kFusedBlocks = 2 * kComputeUnits;

// Tokens per scatter block: 1 below kRunsFromBlocks, else the most (1, 2 or
// 4, with RT * k <= 64) that leave at least kFusedBlocks scatter blocks.
int fused_run(const DispatchParams& p) {
  if ((long)p.T * p.col_chunks < kRunsFromBlocks) return 1;
  int rt = 1;
  while (rt < 4 && 2 * rt * p.k <= kWave &&
         (long)((p.T + 2 * rt - 1) / (2 * rt)) * p.col_chunks >= kFusedBlocks)
    rt *= 2;
  return rt;
}

template <int PAYLOAD, int MAXV, int IPT, int NVR>
void launch_fused_ipt(const DispatchParams& p, hipStream_t st) {
  if constexpr (IPT < 32) {
    const unsigned blocks = 1u + (unsigned)p.T * (unsigned)p.col_chunks;
    hipLaunchKernelGGL((dispatch_fused_kernel<PAYLOAD, MAXV, IPT, NVR, 1>), dim3(blocks),
                       dim3(kBlock), 0, st, p);
  } else {  // runs are built only for 32 ids per thread
    const int rt = fused_run(p);
    const unsigned blocks =
        1u + (unsigned)((p.T + rt - 1) / rt) * (unsigned)p.col_chunks;
    if (rt == 1)
      hipLaunchKernelGGL((dispatch_fused_kernel<PAYLOAD, MAXV, IPT, NVR, 1>), dim3(blocks),
                         dim3(kBlock), 0, st, p);
    else if (rt == 2)
      hipLaunchKernelGGL((dispatch_fused_kernel<PAYLOAD, MAXV, IPT, NVR, 2>), dim3(blocks),
                         dim3(kBlock), 0, st, p);
    else
      hipLaunchKernelGGL((dispatch_fused_kernel<PAYLOAD, MAXV, IPT, NVR, 4>), dim3(blocks),
                         dim3(kBlock), 0, st, p);
  }
}

template <int PAYLOAD, int MAXV, int NVR>
void launch_fused(const DispatchParams& p, hipStream_t st) {
  const long P = (long)p.T * p.k;
  if (P <= kBlock * 4)
    launch_fused_ipt<PAYLOAD, MAXV, 4, NVR>(p, st);
  else if (P <= kBlock * 8)
    launch_fused_ipt<PAYLOAD, MAXV, 8, NVR>(p, st);
  else if (P <= kBlock * 16)
    launch_fused_ipt<PAYLOAD, MAXV, 16, NVR>(p, st);
  else
    launch_fused_ipt<PAYLOAD, MAXV, 32, NVR>(p, st);
}

template <int PAYLOAD, int MAXV>
hipError_t launch_paths(const DispatchParams& p, hipStream_t st) {
  const long P = (long)p.T * p.k;
  if (P <= kSmallMaxPairs) {
    if (p.L <= 8)
      launch_fused<PAYLOAD, MAXV, 2>(p, st);
    else if (p.L <= 16)
      launch_fused<PAYLOAD, MAXV, 4>(p, st);
    else
      launch_fused<PAYLOAD, MAXV, kDirectMaxL / 4>(p, st);
    return hipGetLastError();
  }
  hipError_t err;
  if (p.nchunks <= kBaseCountMaxChunks && (reinterpret_cast<uintptr_t>(p.ids) & 15) == 0) {
    hipLaunchKernelGGL(layout_bases_kernel, dim3(p.nchunks), dim3(kBlock), 0, st, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  } else {
    hipLaunchKernelGGL(layout_chunk_kernel, dim3(p.nchunks), dim3(kBlock), 0, st, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(layout_scan_kernel, dim3(1), dim3(kBlock), 0, st, p);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
  }
  hipLaunchKernelGGL((dispatch_scatter_kernel<PAYLOAD, MAXV>),
                     dim3((unsigned)p.T * (unsigned)p.col_chunks + (unsigned)p.src_blocks),
                     dim3(kBlock), 0, st, p);
  return hipGetLastError();
}

template <int PAYLOAD>
hipError_t launch_payload(const DispatchParams& p, hipStream_t st) {
  const int maxv = (p.vec_per_chunk + kBlock - 1) / kBlock;
  // column chunks hold at most two units per thread, and fp8 chunks one
  // (launch_dispatch)
  if (maxv <= 1) return launch_paths<PAYLOAD, 1>(p, st);
  if constexpr (PAYLOAD == 0)
    if (maxv <= 2) return launch_paths<PAYLOAD, 2>(p, st);
  return hipErrorInvalidValue;
}

size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

}  // namespace

bool dispatch_bases_per_source(int S, int T, int k) {
  const long P = (long)S * T * k;
  return S > 1 && P > kSmallMaxPairs && ((long)T * k) % kChunkPairs == 0;
}

size_t dispatch_workspace_bytes(int T, int k, int E) {
  const size_t P = (size_t)T * (size_t)k;
  if (P <= (size_t)kSmallMaxPairs) return 0;
  const size_t nch = (P + kChunkPairs - 1) / kChunkPairs;
  return align256(4 * P) + align256(4 * nch * (size_t)E) + align256(4 * nch);
}

hipError_t launch_dispatch(const DispatchParams& in, hipStream_t st) {
  DispatchParams p = in;
  const int nunits = units_per_row(p);
  const size_t P = (size_t)p.T * p.k;
  // Column chunks of whole units (8 columns bf16, 16 fp8), balanced; a
  // multiple of 128 columns, so an fp8 scale block never straddles two
  // blocks.  fp8 units (each quantised on its own) and the chunked path: at
  // most one unit per thread.  bf16 on the fused path, where every block
  // recounts all T*k ids: up to two units per thread, so fewer blocks
  // recount, but no fewer chunks than it takes to give each of the 256
  // compute units a block.
  const int align = kFp8Block / (p.payload ? 16 : 8);
  if (p.payload == 0 && P <= (size_t)kSmallMaxPairs) {
    const int fewest = (nunits + 2 * kBlock - 1) / (2 * kBlock);
    const int most = (nunits + kBlock - 1) / kBlock;
    p.col_chunks = max(fewest, min((kComputeUnits + p.T - 1) / max(p.T, 1), most));
  } else {
    p.col_chunks = (nunits + kBlock - 1) / kBlock;
  }
  int vpc = (nunits + p.col_chunks - 1) / p.col_chunks;
  vpc = (vpc + align - 1) / align * align;
  p.vec_per_chunk = vpc;
  p.col_chunks = (nunits + vpc - 1) / vpc;
  p.cc_magic = udiv_magic_of((uint32_t)p.col_chunks);
  p.nchunks = (int)((P + kChunkPairs - 1) / kChunkPairs);
  p.rows = p.C > 0 ? p.N * p.C : (int)P;
  p.l_magic = p.L >= 2 ? (uint32_t)(((1ull << 32) + (uint64_t)p.L - 1) / (uint64_t)p.L) : 0u;
  if (P > (size_t)kSmallMaxPairs) {
    char* ws = reinterpret_cast<char*>(p.workspace);
    p.local_rank = reinterpret_cast<int32_t*>(ws);
    ws += align256(4 * P);
    p.chunk_hist = reinterpret_cast<int32_t*>(ws);
    ws += align256(4 * (size_t)p.nchunks * p.E);
    p.chunk_bad = reinterpret_cast<int32_t*>(ws);
  }
  // the source metadata comes only with the chunked path's scatter
  p.src_blocks = P > (size_t)kSmallMaxPairs && p.src_S > 1 && p.src_counts && p.src_offsets
                     ? (p.E + kWaves - 1) / kWaves
                     : 0;
  return p.payload == 0 ? launch_payload<0>(p, st) : launch_payload<1>(p, st);
}

}  // namespace moe

#ifdef MOE_PHASE_STAMPS
// Tracing library only: the buffer the one-launch dispatch kernel writes its
// phase records to (slots records of kTraceWords words: wave w of block b at
// b * 4 + w; block 0 is the metadata block), or null to stop.  Returns 0 or
// the HIP error code.
extern "C" int moe_trace_set_dispatch(void* buf, uint32_t slots) {
  hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_trace), &buf, sizeof(buf));
  if (e == hipSuccess) e = hipMemcpyToSymbol(HIP_SYMBOL(moe::g_trace_slots), &slots, sizeof(slots));
  return (int)e;
}
#endif
