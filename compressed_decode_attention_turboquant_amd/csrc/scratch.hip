// Device scratch for the entry points that allocate nothing.
//
// One file-scope device array per GPU the library runs on (the runtime keeps
// it until the process ends).  Host code never uses the array's name as an
// address: the first call on a device, with that device current, looks its
// address up with hipGetSymbolAddress and keeps it per device; every later
// use goes through that pointer.
#include <mutex>

#include "hsq_internal.h"

namespace hsq {
namespace {

constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_ptr[kMaxDevices];

}  // namespace

int static_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return check_hip(e, "static scratch: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(HSQ_ERR_UNSUPPORTED, "static scratch: device ordinal above 63");
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return check_hip(e, "static scratch: hipGetSymbolAddress");
    if (!p) return fail(HSQ_ERR_HIP, "static scratch: hipGetSymbolAddress returned null");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return HSQ_OK;
}

}  // namespace hsq
