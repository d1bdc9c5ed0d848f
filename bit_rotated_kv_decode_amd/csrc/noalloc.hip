// Library-owned decode workspace for callers that cannot allocate device memory.
//
// oscar_decode_step_noalloc runs the same three launches as oscar_decode_step, with the workspace
// (rotated queries, split partials) taken from `scratch`, a fixed device array of this file.  Each
// GPU the library runs on holds its own copy of the array until the process ends; its address on
// a device is looked up once, with that device current, and kept.  In host code the array's name
// is only a host-side stand-in, so every kernel argument uses the looked-up device address.
#include <mutex>

#include "oscar_internal.h"

namespace oscar {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_on_current_device(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace oscar
