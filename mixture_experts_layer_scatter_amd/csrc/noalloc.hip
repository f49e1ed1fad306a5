// moe_layer_forward_static: the fused layer for callers that cannot allocate (code under HIP
// graph capture, tight serving loops, harnesses that forbid hipMalloc).  Its scratch memory is
// a device array owned by this library, of kStaticScratchBytes, one copy per device, held until
// the process ends; the call runs moe_layer_forward's launch sequence on it.
//
// The array is a file-scope __device__ variable: in host code its name is only a stand-in, so
// its device address is looked up once per device with hipGetSymbolAddress (with that device
// current) and that address is what the kernels receive.
#include "../../include/moe.h"
#include "common.hpp"

#include <atomic>
#include <mutex>

namespace {

constexpr size_t kStaticScratchBytes = size_t(MOE_STATIC_SCRATCH_MIB) << 20;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

// device address of `scratch` on the current device (null on a HIP error)
void* scratch_ptr() {
  static std::atomic<void*> ptr[moe::kMaxDevices] = {};
  static std::mutex mu;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= moe::kMaxDevices) return nullptr;
  void* p = ptr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(mu);
  p = ptr[dev].load(std::memory_order_relaxed);
  if (!p) {
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    ptr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace

extern "C" {

size_t moe_static_scratch_bytes(void) { return kStaticScratchBytes; }

moe_status_t moe_layer_forward_static(const moe_dims_t* dims, const void* x, const void* wg,
                                      const float* bias, const void* w1, const void* w3,
                                      const void* w2, const void* ws1, const void* ws3,
                                      const void* ws2, void* y, const moe_debug_out_t* dbg,
                                      void* stream) {
  const size_t need = moe_workspace_bytes(dims);
  // dims that fail the checks: moe_layer_forward names the reason before touching anything
  if (need == 0) return moe_layer_forward(dims, x, wg, bias, w1, w3, w2, ws1, ws3, ws2, y, dbg,
                                          nullptr, 0, stream);
  if (need > kStaticScratchBytes) return MOE_ERR_WORKSPACE;
  if (dims->T == 0) return MOE_OK;
  void* ws = scratch_ptr();
  if (!ws) return MOE_ERR_HIP;
  // every kernel of the layer writes the scratch it reads later: nothing needs clearing
  return moe_layer_forward(dims, x, wg, bias, w1, w3, w2, ws1, ws3, ws2, y, dbg, ws,
                           kStaticScratchBytes, stream);
}

}  // extern "C"
