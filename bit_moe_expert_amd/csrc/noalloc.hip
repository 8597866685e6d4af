// Fixed device scratch for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc): moe_forward_layer_noalloc runs
// the layer with its workspace carved from this array instead of a caller-provided buffer.
//
// The array exists once per GPU the library runs on and lives until the process ends. In host
// code its name is only a stand-in, so its device address is looked up once per device (with that
// device current) and every launch uses that address. Calls on one GPU share the array: calls that
// overlap on one GPU (different streams without ordering) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace moe {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_device_ptr(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
