// Scratch memory of nsa_decode_fwd_noalloc: one file-scope device array per GPU the library runs on.
//
// Callers that cannot allocate device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc) take the decode workspace from this array instead of passing one.
// In host code the name `scratch` is only a host-side stand-in for the symbol; the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with that device current, and
// only that address is ever handed to kernels.  The array lives until the process ends; every call
// on a GPU shares it, so calls that overlap on one GPU race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "common.hpp"

namespace {
constexpr size_t kScratchBytes = (size_t)64 << 20;  // 64 MiB per device
constexpr int kMaxDevices = 64;
}  // namespace

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

size_t noalloc_scratch_bytes() { return kScratchBytes; }

// Device address and size of the current device's scratch array (hipGetSymbolAddress on the first
// call for each device, then the kept address).
hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  *bytes = kScratchBytes;
  return hipSuccess;
}
