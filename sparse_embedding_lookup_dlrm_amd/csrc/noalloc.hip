// Scratch for the allocation-free backward entry point: one static device
// array per GPU, owned by the library, so that a caller that cannot allocate
// device memory (code under graph capture, a tight serving loop) needs no
// workspace. Each GPU the library runs on holds its own copy until the
// process ends.
#include <mutex>

#include "common.h"

namespace dlrm {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current device's scratch array. The array's name in
// host code is only a stand-in for the symbol, so the address is looked up
// once per device (with that device current) and kept.
hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
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
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace dlrm
