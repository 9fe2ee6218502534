// The library's one static device buffer: scratch space for the entry point
// that allocates nothing (csa2_topk_noalloc), for callers that cannot call
// hipMalloc (code under HIP graph capture, tight serving loops, harnesses that
// forbid allocation).
//
// Every GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends.  In host code the array's name is only a
// host-side stand-in: the device address comes from hipGetSymbolAddress,
// looked up once per device with that device current, and only that address
// is ever handed to kernels.  Calls on one GPU share the array, which keeps
// the last call's contents; calls that overlap on one GPU race.
#include <mutex>

#include "csa2_internal.h"

namespace csa2 {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device, once looked up
}  // namespace

hipError_t static_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace csa2
