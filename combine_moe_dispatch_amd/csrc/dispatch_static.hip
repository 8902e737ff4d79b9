// dispatch_static.hip -- moe_dispatch_static: moe_dispatch for callers that
// cannot allocate device memory (code under stream capture, tight serving
// loops, harnesses that forbid allocation).  The multi-kernel layout path's
// scratch (per-pair ranks inside a chunk, per-chunk histograms and flags)
// comes from one file-scope device array per GPU instead of a caller
// workspace; the kernels are those of moe_dispatch.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe_dispatch.h"

// In host code `scratch` is only a stand-in symbol, not a device address: the
// address of the array on the current GPU comes from hipGetSymbolAddress
// (once per device), and only that address is ever handed to a kernel.  Each
// GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_scratch[kMaxDevices];  // device address of `scratch` per GPU, once looked up

// Device address of the current GPU's scratch array.
moe_status scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MOE_ERR_HIP;
  if (dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> guard(g_lock);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_dispatch_static(const moe_shape* shape, const void* x,
                                          const int32_t* topk_ids, void* recv_x,
                                          float* recv_scales, const moe_layout* layout,
                                          hipStream_t stream) {
  // 0 for an invalid shape, which moe_dispatch then rejects
  const size_t need = moe_dispatch_workspace_size(shape);
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  if (need > 0) {
    const moe_status st = scratch_address(&ws);
    if (st != MOE_OK) return st;
  }
  // every scratch entry the layout kernels read is written first in the same
  // call, so nothing needs clearing between calls
  return moe_dispatch(shape, x, topk_ids, recv_x, recv_scales, layout, ws, need, stream);
}
