// Library-owned scratch memory of the allocation-free forward entry point
// (ssm_scan_fwd_noalloc in include/ssm_scan.h).
//
// A scan that splits the sequence into pieces keeps each piece's affine
// aggregate (decay product and end state, per (b, d, n)) between its two
// launches. ssm_scan_fwd takes that buffer from the caller; the
// allocation-free variant takes it from `scratch`, a fixed array in device
// memory that every GPU the library runs on holds for the life of the
// process. Host code never uses the array's name as an address: the first
// call on a device, with that device current, asks the runtime for the
// array's address on that device and keeps it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t{16} << 20;  // 16 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex g_mutex;
void* g_scratch[kMaxDevices] = {};

}  // namespace

namespace ssm {

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace ssm
