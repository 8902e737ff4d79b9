// ceiling.hip -- plain streaming kernels that measure what this GPU's memory
// system sustains at a given size: read, write and copy of a buffer, and a read
// and a write of given sizes in one kernel, with the same 16-byte
// non-temporal accesses the dispatch and combine kernels use, an
// empty launch, the dispatch's own row copy with its rows handed to it, and
// the combine's row gathers without the weighted sum.  They are the measured
// floor the MoE kernels' times are compared with (libmoe_ceiling.so,
// used by the benchmark only; not part of the dispatch/combine interface).
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Grid-stride read of n 16-byte vectors; the xor of everything read is kept
// alive by a store that practically never happens (a fixed magic value).
__global__ void __launch_bounds__(256)
stream_read_kernel(const u32x4* __restrict__ p, size_t n, unsigned* __restrict__ sink) {
  u32x4 acc = {0, 0, 0, 0};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride)
    acc ^= __builtin_nontemporal_load(&p[i]);
  const unsigned r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9e3779b9u) sink[blockIdx.x] = r;
}

__global__ void __launch_bounds__(256)
stream_write_kernel(u32x4* __restrict__ p, size_t n, unsigned v) {
  const u32x4 val = {v, v, v, v};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(val, &p[i]);
}

// Grid-stride read of nr 16-byte vectors and write of nw in the same loop (a
// constant stored), with the same non-temporal accesses: what a kernel that
// only moved the bytes a dispatch (reads x, writes the rows) or a combine
// (reads the rows, writes the output) moves would take.  The xor of what is
// read is kept alive as in stream_read_kernel.
__global__ void __launch_bounds__(256)
stream_read_write_kernel(const u32x4* __restrict__ src, size_t nr, u32x4* __restrict__ dst,
                         size_t nw, unsigned* __restrict__ sink) {
  u32x4 acc = {0, 0, 0, 0};
  const u32x4 val = {7u, 7u, 7u, 7u};
  const size_t n = nr > nw ? nr : nw;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride) {
    if (i < nr) acc ^= __builtin_nontemporal_load(&src[i]);
    if (i < nw) __builtin_nontemporal_store(val, &dst[i]);
  }
  const unsigned r = acc.x ^ acc.y ^ acc.z ^ acc.w;
  if (r == 0x9e3779b9u) sink[blockIdx.x] = r;
}

// Block b writes vectors [b*4096, b*4096 + 4096): 16 per thread, each
// instruction of the block covering 4 KB, through a buffer descriptor for the
// block's range with the given cache policy (2 = non-temporal, 0 = default,
// 16 = system-coherent write-through).  At some sizes this pattern and policy
// beat the grid-stride loop, so the floor takes the best of both.
template <int POLICY>
__global__ void __launch_bounds__(256)
blocked_write_kernel(u32x4* __restrict__ p, size_t n, unsigned v) {
  const u32x4 val = {v, v, v, v};
  const size_t base = (size_t)blockIdx.x * 4096;
  const int count = (int)min((size_t)4096, n - base);
  const __amdgpu_buffer_rsrc_t rs =
      __builtin_amdgcn_make_buffer_rsrc(p + base, (short)0, count * 16, 0x00020000);
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int i = j * 256 + (int)threadIdx.x;
    if (i < count) __builtin_amdgcn_raw_buffer_store_b128(val, rs, i * 16, 0, POLICY);
  }
}

__global__ void __launch_bounds__(256)
stream_copy_kernel(const u32x4* __restrict__ s, u32x4* __restrict__ d, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(&s[i]), &d[i]);
}

// The dispatch's data movement with its rows handed to it: block b owns
// (token b / col_chunks, column chunk b % col_chunks) of vpc 16-byte vectors,
// at most two per thread, and stores its slice of x row t (a constant when x
// is null) to the k rows listed for t in rows (row t*k + j when rows is
// null), with the dispatch's 16-byte non-temporal loads and stores.  Rows
// outside [0, rows_total) are skipped.  What a dispatch that did not have to
// derive its rows would take, one part at a time.
__global__ void __launch_bounds__(256)
rows_copy_kernel(const u32x4* __restrict__ x, const int* __restrict__ rows,
                 u32x4* __restrict__ dst, int k, int nvec, int col_chunks, int vpc,
                 int rows_total) {
  const int t = (int)blockIdx.x / col_chunks;
  const int cc = (int)blockIdx.x - t * col_chunks;
  const int u0 = cc * vpc;
  const int u1 = min(u0 + vpc, nvec);
  const int slot = min((int)(threadIdx.x & 63), k - 1);
  const int row_lane = rows ? rows[(size_t)t * k + slot] : t * k + slot;
  u32x4 xv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int u = u0 + (int)threadIdx.x + i * 256;
    if (x)
      xv[i] = __builtin_nontemporal_load(&x[(size_t)t * nvec + min(u, u1 - 1)]);
    else
      xv[i] = (u32x4){(unsigned)t, (unsigned)u, 0u, 0u};
  }
  for (int j = 0; j < k; ++j) {
    const int row = __builtin_amdgcn_readlane(row_lane, j);
    if (row < 0 || row >= rows_total) continue;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int u = u0 + (int)threadIdx.x + i * 256;
      if (u < u1) __builtin_nontemporal_store(xv[i], &dst[(size_t)row * nvec + u]);
    }
  }
}

// The combine's data movement without its arithmetic: one-wave blocks over
// (token, 64-vector column chunk), each lane gathering the 16-byte vector of
// its column from the token's k rows -- rows[t*k + j] when rows is given
// (read at uniform addresses, as the combine reads its rows), row t*k + j
// otherwise -- with the combine's non-temporal loads and stores, and storing
// their xor to row t of out.  The loads are unconditional (rows outside
// [0, rows_total) read row 0 and are left out of the xor), eight at a time.
// token_major: grid x = token, y = column chunk; otherwise the reverse.
__global__ void __launch_bounds__(64)
rows_gather_kernel(const u32x4* __restrict__ y, const int* __restrict__ rows,
                   u32x4* __restrict__ out, int k, int nvec, int rows_total, int token_major) {
  const int t = token_major ? (int)blockIdx.x : (int)blockIdx.y;
  const int v = (token_major ? (int)blockIdx.y : (int)blockIdx.x) * 64 + (int)threadIdx.x;
  const int vc = min(v, nvec - 1);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int j0 = 0; j0 < k; j0 += 8) {
    int r[8];
#pragma unroll
    for (int g = 0; g < 8; ++g)
      r[g] = j0 + g < k ? (rows ? rows[(size_t)t * k + j0 + g] : t * k + j0 + g) : -1;
    u32x4 val[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) {
      const bool on = r[g] >= 0 && r[g] < rows_total;
      val[g] = __builtin_nontemporal_load(&y[(size_t)(on ? r[g] : 0) * nvec + vc]);
      if (!on) val[g] = (u32x4){0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int g = 0; g < 8; ++g) acc ^= val[g];
  }
  if (v < nvec) __builtin_nontemporal_store(acc, &out[(size_t)t * nvec + v]);
}

__global__ void empty_kernel() {}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

}  // namespace

// Each returns 0, or 1 for a bad argument (null or unaligned pointer, blocks
// outside [1, 65535], sink with fewer than `blocks` entries is the caller's
// responsibility), or the HIP error code of the launch.  nvec = number of
// 16-byte vectors.
extern "C" int moe_ceiling_read(const void* p, size_t nvec, void* sink, int blocks,
                                hipStream_t stream) {
  if (!p || !sink || !aligned16(p) || blocks < 1 || blocks > 65535) return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(p), nvec, static_cast<unsigned*>(sink));
  return (int)hipGetLastError();
}

extern "C" int moe_ceiling_write(void* p, size_t nvec, int blocks, hipStream_t stream) {
  if (!p || !aligned16(p) || blocks < 1 || blocks > 65535) return 1;
  hipLaunchKernelGGL(stream_write_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<u32x4*>(p), nvec, 7u);
  return (int)hipGetLastError();
}

// src: nr vectors read, dst: nw vectors written (one of the two counts may be
// 0, not both); sink: `blocks` entries.
extern "C" int moe_ceiling_read_write(const void* src, size_t nr, void* dst, size_t nw,
                                      void* sink, int blocks, hipStream_t stream) {
  if ((nr && (!src || !aligned16(src))) || (nw && (!dst || !aligned16(dst))) ||
      (nr == 0 && nw == 0) || !sink || blocks < 1 || blocks > 65535)
    return 1;
  hipLaunchKernelGGL(stream_read_write_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), nr, static_cast<u32x4*>(dst), nw,
                     static_cast<unsigned*>(sink));
  return (int)hipGetLastError();
}

// policy: 0 = non-temporal, 1 = default, 2 = system-coherent write-through.
extern "C" int moe_ceiling_write_blocked(void* p, size_t nvec, int policy, hipStream_t stream) {
  if (!p || !aligned16(p) || nvec == 0 || policy < 0 || policy > 2) return 1;
  const size_t blocks = (nvec + 4095) / 4096;
  if (blocks > 0x7fffffff) return 1;
  u32x4* q = static_cast<u32x4*>(p);
  const dim3 grid((unsigned)blocks);
  if (policy == 0)
    hipLaunchKernelGGL(blocked_write_kernel<2>, grid, dim3(256), 0, stream, q, nvec, 7u);
  else if (policy == 1)
    hipLaunchKernelGGL(blocked_write_kernel<0>, grid, dim3(256), 0, stream, q, nvec, 7u);
  else
    hipLaunchKernelGGL(blocked_write_kernel<16>, grid, dim3(256), 0, stream, q, nvec, 7u);
  return (int)hipGetLastError();
}

extern "C" int moe_ceiling_copy(const void* src, void* dst, size_t nvec, int blocks,
                                hipStream_t stream) {
  if (!src || !dst || !aligned16(src) || !aligned16(dst) || blocks < 1 || blocks > 65535)
    return 1;
  hipLaunchKernelGGL(stream_copy_kernel, dim3(blocks), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), static_cast<u32x4*>(dst), nvec);
  return (int)hipGetLastError();
}

// x: [T][nvec] 16-byte vectors or null (a constant is stored); rows: [T][k]
// or null (rows t*k + j); dst: [rows_total][nvec].  Blocks T * col_chunks;
// col_chunks * vpc must cover nvec with vpc <= 512 (two vectors per thread).
extern "C" int moe_ceiling_rows_copy(const void* x, const int32_t* rows, void* dst, int T, int k,
                                     int nvec, int col_chunks, int vpc, int rows_total,
                                     hipStream_t stream) {
  if (!dst || !aligned16(dst) || (x && !aligned16(x)) || T < 1 || k < 1 || k > 64 ||
      nvec < 1 || col_chunks < 1 || vpc < 1 || vpc > 512 ||
      (long long)col_chunks * vpc < nvec || rows_total < 1 ||
      (long long)T * col_chunks > 0x7fffffffLL || (!rows && (long long)T * k > rows_total))
    return 1;
  hipLaunchKernelGGL(rows_copy_kernel, dim3((unsigned)(T * col_chunks)), dim3(256), 0, stream,
                     static_cast<const u32x4*>(x), rows, static_cast<u32x4*>(dst), k, nvec,
                     col_chunks, vpc, rows_total);
  return (int)hipGetLastError();
}

// y: [rows_total][nvec] 16-byte vectors; rows: [T][k] or null (rows t*k + j,
// which must then lie below rows_total); out: [T][nvec].  Grid T x
// ceil(nvec / 64) one-wave blocks, token-major up to 8192 blocks (as the
// combine orders them), chunk-major past that.
extern "C" int moe_ceiling_rows_gather(const void* y, const int32_t* rows, void* out, int T, int k,
                                       int nvec, int rows_total, hipStream_t stream) {
  if (!y || !out || !aligned16(y) || !aligned16(out) || T < 1 || T > 65535 || k < 1 ||
      k > 64 || nvec < 1 || rows_total < 1 || (!rows && (long long)T * k > rows_total))
    return 1;
  const int chunks = (nvec + 63) / 64;
  if (chunks > 65535) return 1;
  const int token_major = (long long)T * chunks <= 8192 ? 1 : 0;
  const dim3 grid = token_major ? dim3((unsigned)T, (unsigned)chunks)
                                : dim3((unsigned)chunks, (unsigned)T);
  hipLaunchKernelGGL(rows_gather_kernel, grid, dim3(64), 0, stream, static_cast<const u32x4*>(y),
                     rows, static_cast<u32x4*>(out), k, nvec, rows_total, token_major);
  return (int)hipGetLastError();
}

extern "C" int moe_ceiling_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return (int)hipGetLastError();
}
