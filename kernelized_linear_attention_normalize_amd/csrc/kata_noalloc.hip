// The chunked forward's fixed scratch: the segment-summary workspace of
// kata_chunked_fwd_noalloc lives in a device array owned by the library, so callers that
// cannot allocate device memory (code under HIP graph capture, serving loops, harnesses that
// forbid hipMalloc) can run the associative chunked forward.
//
// Each GPU the library runs on holds its own copy of the array, at its own address, until the
// process ends. Host code never uses the array's name as a device address (on the host it is
// a stand-in symbol): the address is resolved once per device with hipGetSymbolAddress, with
// that device current, and only that pointer reaches kernels. Every call on a device shares
// the device's array; calls that overlap on one GPU race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kata.h"
#include "kata_launch.h"

namespace {

// summaries of the associative scan (fully written by the summary pass before the scan and
// the segment pass read them: nothing in it has to start at zero)
static __device__ __align__(256) unsigned char scratch[KATA_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of scratch per device, null until resolved

}  // namespace

namespace kata {

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
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

}  // namespace kata
