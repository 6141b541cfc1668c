// Library-held scratch for callers that cannot allocate (code under stream capture, serving
// loops, harnesses that forbid hipMalloc): the two-phase chunk forward's workspace lives in
// a file-scope device array instead of caller memory.
//
// Each device that loads the library holds its own copy of `scratch` for the life of the
// process. Host code never uses the array's name as an address (on the host it is only a
// stand-in for the device symbol): the device address is looked up once per device with
// hipGetSymbolAddress and kept in `g_scratch_ptr`.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn2_launch.h"

namespace gdn2 {

constexpr size_t kScratchBytes = size_t(128) << 20;  // 128 MiB per device

// Kept even though no kernel names it: it is reached only through hipGetSymbolAddress.
__attribute__((used)) static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

size_t scratch_capacity() { return kScratchBytes; }

// Device address of this device's scratch array (looked up on the first call per device,
// with that device current). Returns hipSuccess and sets *ptr, or the runtime's error.
hipError_t scratch_for_device(int device, void** ptr) {
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[device] == nullptr) {
    int cur = -1;
    hipError_t e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != device && (e = hipSetDevice(device)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != device) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[device] = p;
  }
  *ptr = g_scratch_ptr[device];
  return hipSuccess;
}

}  // namespace gdn2
