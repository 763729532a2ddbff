// Library-owned scratch for the entry points that allocate nothing: one
// file-scope device array per GPU (each device that loads the library holds
// its own copy until the process ends). Host code never passes the array's
// name to a kernel or a copy: the name is a host-side stand-in, not a device
// address. Its device address comes from hipGetSymbolAddress, looked up once
// per device with that device current, and only that address is used.
#include <mutex>

#include "lq_device.h"

namespace lq {

static __device__ __align__(256) unsigned char scratch[LQ_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace lq
