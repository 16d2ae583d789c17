// The fixed device scratch of sfi_fast_step_packed_noalloc, the fast step for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in
// symbol); it looks up each device's address once, with that device current,
// and uses that address everywhere.
#include <hip/hip_runtime.h>

#include <mutex>

#include "sfi_internal.hpp"

namespace sfi {
namespace {

static __device__ __align__(256) unsigned char scratch[SFI_NOALLOC_SCRATCH_BYTES];

struct DeviceScratch {
  std::mutex mu;
  char* ptr[kMaxDevices] = {};
};

DeviceScratch& device_scratch() {
  static DeviceScratch d;
  return d;
}

}  // namespace

int32_t noalloc_scratch(hipStream_t s, char** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(SFI_ERR_HIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(SFI_ERR_UNSUPPORTED, "device %d beyond %d devices", dev, kMaxDevices);
  DeviceScratch& d = device_scratch();
  std::lock_guard<std::mutex> lk(d.mu);
  if (d.ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(SFI_ERR_HIP, "hipGetSymbolAddress(scratch) on device %d: %s", dev, hipGetErrorString(e));
    // the chunk counters must start at zero (every call leaves them at zero);
    // a fill kernel rather than a memset, so a capturing caller records a
    // kernel node
    e = launch_fill_zero(p, kNoAllocCounterBytes, s);
    if (e != hipSuccess) return fail(SFI_ERR_HIP, "clearing the scratch counters: %s", hipGetErrorString(e));
    d.ptr[dev] = static_cast<char*>(p);
  }
  *out = d.ptr[dev];
  return SFI_OK;
}

}  // namespace sfi
