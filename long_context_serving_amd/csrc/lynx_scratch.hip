// Library-owned scratch memory for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops, harnesses that
// forbid hipMalloc): a file-scope device array of fixed size, which every
// GPU the library runs on holds until the process ends.
//
// In host code the array's name is a host-side stand-in, not a device
// address, so host code never passes it anywhere: its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and kept, and only that address reaches kernels.
#include <mutex>

#include "lynx_internal.h"

namespace lynx {
namespace {

constexpr size_t kScratchBytes = static_cast<size_t>(LYNX_STATIC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) char scratch[kScratchBytes];

std::mutex g_mutex;
void *g_address[kMaxDevices] = {};

}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

hipError_t scratch_address(void **ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_address[dev] == nullptr) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_address[dev] = p;
  }
  *ptr = g_address[dev];
  return hipSuccess;
}

}  // namespace lynx
