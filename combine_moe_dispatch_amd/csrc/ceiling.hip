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
