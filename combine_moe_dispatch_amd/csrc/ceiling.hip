// ceiling.hip -- plain streaming kernels that measure what this GPU's memory
// system sustains at a given size: read, write and copy of a buffer with the
// same 16-byte non-temporal accesses the dispatch and combine kernels use, and
// an empty launch.  They are the measured floor against which the MoE
// kernels' times are judged (libmoe_ceiling.so, used by the benchmark only;
// not part of the dispatch/combine interface).
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

extern "C" int moe_ceiling_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return (int)hipGetLastError();
}
