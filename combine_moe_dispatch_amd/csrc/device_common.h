// device_common.h -- small device helpers shared by the kernels of
// libmoe_dispatch.so: number-format conversions written from the formats,
// wavefront primitives for wave64, and the launch limits.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;          // CDNA wavefront width
constexpr int kMaxExperts = 1024;  // LDS histograms are sized for this
constexpr int kMaxTopK = 32;
constexpr int kFp8Block = 128;     // columns per fp8 scale

// Two fp32 values to a bf16 pair (lo in bits 15:0; bf16 = 8 exponent bits,
// 7 mantissa bits) with the gfx950 packed convert in one instruction: round
// to nearest even on the bit pattern, NaN quieted (the 0x0040 bit set), which
// equals the integer rounding u + 0x7fff + ((u >> 16) & 1), then >> 16, for
// every one of the 2^32 fp32 patterns (checked exhaustively on the GPU, in
// both halves).
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xffff0000u); }

// OCP e4m3fn code from an fp32 value: round to nearest even, magnitudes at or
// beyond 448 saturate to 448 (code 0x7E), NaN gives 0x7F.
//  - |v| < 2^-6 is subnormal in e4m3: the code is |v| / 2^-9 rounded to an
//    integer (0..8; 8 is the smallest normal, code 0x08).
//  - otherwise keep 3 mantissa bits of the fp32 pattern with RNE on the 20
//    dropped bits and rebias the exponent from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t u = __float_as_uint(v);
  uint32_t sign = (u >> 24) & 0x80u;
  uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  if (a >= 0x43e00000u) return sign | 0x7eu;  // >= 448
  if (a < 0x3c800000u) {                      // < 2^-6
    float m = rintf(__uint_as_float(a) * 512.0f);
    return sign | (uint32_t)m;
  }
  a += 0x7ffffu + ((a >> 20) & 1u);
  uint32_t code = (((a >> 23) - 120u) << 3) | ((a >> 20) & 7u);
  return sign | code;
}

// fp32 values of the four e4m3fn codes packed in w (byte i -> f[i]), with the
// gfx950 packed convert (OCP e4m3fn; exact, since every code is an fp32 value).
__device__ __forceinline__ void e4m3x4_to_f32(uint32_t w, float* f) {
  const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Streaming (non-temporal) 16- and 8-byte global accesses, for data touched
// once: the payload rows of dispatch and combine.  Measured on MI355X they
// shorten both kernels (the caches need not hold or write back the stream).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint4 load_stream(const uint4* p) {
  const u32x4 t = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}
__device__ __forceinline__ void store_stream(uint4* p, uint4 v) {
  const u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x4*>(p));
}
// 16-byte store at byte offset off of [base, base + nbytes) with device
// scope (sc1): the line is written through this XCD's L2 instead of being
// held there until the end-of-kernel write-back.  Measured faster than the
// non-temporal store for outputs of tens of MB, slower for a few MB.
__device__ __forceinline__ void store_device_scope(void* base, int nbytes, int off, uint4 v) {
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(base, (short)0, nbytes, 0x00020000);
  const u32x4 t = {v.x, v.y, v.z, v.w};
  __builtin_amdgcn_raw_buffer_store_b128(t, rs, off, 0, 16 /* sc1 */);
}
__device__ __forceinline__ uint2 load_stream(const uint2* p) {
  const u32x2 t = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(p));
  return make_uint2(t.x, t.y);
}
__device__ __forceinline__ void store_stream(uint2* p, uint2 v) {
  const u32x2 t = {v.x, v.y};
  __builtin_nontemporal_store(t, reinterpret_cast<u32x2*>(p));
}

// Workgroups are handed to the 8 XCDs of the chip in turn (workgroup b runs
// on XCD b % 8), and each XCD has its own L2.  This renumbers the n
// workgroups of a launch so that consecutive logical indices run on the same
// XCD: logical = (workgroups on lower XCDs) + b / 8, a bijection onto [0, n).
// Neighbouring tiles that share cache lines then share one L2.
__device__ __forceinline__ unsigned xcd_local_block(unsigned b, unsigned n) {
  constexpr unsigned kXcds = 8;
  const unsigned x = b % kXcds, q = n / kXcds, r = n % kXcds;
  return x * q + (x < r ? x : r) + b / kXcds;
}

// Block barrier that orders LDS accesses only.  __syncthreads() also waits
// for every global load in flight (a workgroup fence covers global memory);
// this one lets them stay in flight across the barrier.  Use it only where
// no global memory written by one thread is read by another after it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over a wave64 with DPP: Hillis-Steele shifts inside
// each 16-lane row (out-of-row sources read 0), then the row totals are
// carried forward with the row broadcasts of lanes 15 and 31.
__device__ __forceinline__ int wave_inclusive_sum_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15 -> rows 1, 3
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31 -> rows 2, 3
  return x;
}



// Lanes of this wave whose `key` equals this lane's key (a 64-bit mask),
// built one key bit at a time from ballots.  `bits` = number of key bits.
__device__ __forceinline__ uint64_t wave_match(uint32_t key, int bits) {
  uint64_t peers = ~0ull;
  for (int b = 0; b < bits; ++b) {
    uint32_t bit = (key >> b) & 1u;
    uint64_t ones = __ballot(bit);
    peers &= bit ? ones : ~ones;
  }
  return peers & __ballot(1);
}

__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

// s_waitcnt operand that waits for vmcnt == 0 and leaves expcnt (7) and
// lgkmcnt (15) unconstrained (gfx9 encoding: vmcnt in bits 3:0 and 15:14,
// expcnt in 6:4, lgkmcnt in 11:8).
constexpr unsigned kWaitVm0 = 0x0F70;

// Kernel arguments are scalar loads, and the compiler issues them where they
// are first needed: behind an early branch they come one memory round trip
// later.  An empty asm that reads the values from scalar registers before
// the branch makes them part of the first batch of argument loads.
#define MOE_ARGS_UP_FRONT(...) asm volatile("" ::__VA_ARGS__)

// Phase stamps, compiled only into the tracing library (libmoe_trace.so,
// built with -DMOE_PHASE_STAMPS; the product library has none of this): a
// kernel reads the 100 MHz wall clock at named points of its path, and one
// lane per wave writes the wave's record of kTraceWords words to the trace
// buffer its source file holds (set with that file's moe_trace_set_* call),
// at the wave's slot when the slot fits.  MOE_TRACE_WAIT makes the wave wait
// for its own outstanding memory operations, so that a stamp after it marks
// their completion.
constexpr int kTraceWords = 8;
#ifdef MOE_PHASE_STAMPS
#define MOE_STAMP(var) const uint64_t var = __builtin_amdgcn_s_memrealtime()
#define MOE_STAMP_DECL(var) uint64_t var = 0
#define MOE_STAMP_SET(var) var = __builtin_amdgcn_s_memrealtime()
#define MOE_TRACE_WAIT() asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory")
// lane 0 writes (w0..w5, the wave's hardware id) at record `slot`
__device__ __forceinline__ void trace_record(uint64_t* buf, uint32_t slots, uint32_t slot,
                                             uint64_t w0, uint64_t w1, uint64_t w2, uint64_t w3,
                                             uint64_t w4, uint64_t w5) {
  if (buf == nullptr || slot >= slots || (threadIdx.x & (kWave - 1)) != 0) return;
  uint32_t hw;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_HW_ID)" : "=s"(hw));
  uint64_t* r = buf + (size_t)slot * kTraceWords;
  r[0] = w0;
  r[1] = w1;
  r[2] = w2;
  r[3] = w3;
  r[4] = w4;
  r[5] = w5;
  r[6] = hw;
  r[7] = 1;  // record written
}
#else
#define MOE_STAMP(var)
#define MOE_STAMP_DECL(var)
#define MOE_STAMP_SET(var)
#define MOE_TRACE_WAIT()
#endif

// n / d without a division, for any n < 2^32 and d >= 1: with
// m = floor((2^32 - 1) / d), umulhi(n, m) is floor(n / d) or one less (the
// product undershoots n / d by less than n / 2^32 < 1), and one remainder
// check corrects it.  Uniform operands keep it to a few scalar instructions.
__host__ __device__ __forceinline__ uint32_t udiv_magic_of(uint32_t d) {
  return 0xffffffffu / d;
}
__device__ __forceinline__ uint32_t udiv_magic(uint32_t n, uint32_t d, uint32_t m) {
  const uint32_t q = __umulhi(n, m);
  return q + (n - q * d >= d ? 1u : 0u);
}

__device__ __forceinline__ uint64_t lanes_below() {
  const int lane = lane_id();
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

}  // namespace moe
