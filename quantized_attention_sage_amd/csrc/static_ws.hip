// The library-held workspace of sage_attn_static: one file-scope device array
// per GPU, for callers that cannot allocate device memory.
//
// In host code `scratch` names a host-side stand-in, not the device array, so
// host code never passes it to a kernel or a copy: the device address is
// looked up once per device (with that device current) and kept here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sage.h"
#include "sage_internal.h"

namespace {

__device__ __align__(256) unsigned char scratch[SAGE_STATIC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

namespace sage {

hipError_t static_workspace(void** ptr, int* device) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  *device = dev;
  return hipSuccess;
}

}  // namespace sage
