// Library-owned device scratch for rdkv_decode_static, the decode entry point
// that allocates nothing: its split-K partials go to a file-scope device
// array instead of a caller workspace.  The array is part of the code object,
// so every GPU the library runs on holds its own copy, at its own address,
// until the process ends.  Host code never uses the array's name as an
// address (on the host it is only a stand-in); the device address comes from
// hipGetSymbolAddress, once per device, with that device current.
#include <mutex>

#include "rdkv_internal.h"

namespace rdkv {
namespace {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch[kMaxDevices];

}  // namespace

hipError_t static_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace rdkv
