// The built-in workspace of the allocation-free eviction step
// (rkv_evict_step_noalloc): a file-scope device array that the code object
// holds on every GPU it is loaded on, until the process ends, so that a call
// needs no hipMalloc. In host code `scratch` names a host-side stand-in, not
// the device array: its device address is looked up once per device with
// hipGetSymbolAddress, with that device current, and only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "rkv_internal.hpp"

namespace rkv {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::once_flag g_once[kMaxDevices];
void* g_addr[kMaxDevices];
int g_err[kMaxDevices];

}  // namespace

int scratch_workspace(void** ws) {
  int dev = 0;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev]() {
    void* a = nullptr;
    const hipError_t r = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    g_err[dev] = (int)r;
    g_addr[dev] = r == hipSuccess ? a : nullptr;
  });
  if (g_err[dev] != 0) return g_err[dev];
  *ws = g_addr[dev];
  return 0;
}

}  // namespace rkv
