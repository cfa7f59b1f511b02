// Static scratch for the allocation-free segmented prefill
// (gdn_prefill_segmented_noalloc in include/gdn.h).
//
// Some callers cannot allocate device memory: code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc.  For them the window
// offsets and the chunked workspace of a segmented prefill live in one
// file-scope device array of a fixed size, which the code object brings onto
// every device the library runs on and which stays there until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// names a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, taken once per device with that device current, and
// only that address is used.
#include <mutex>

#include "../../include/gdn.h"
#include "gdn_internal.hpp"

namespace gdn {

static __device__ __align__(256) uint8_t scratch[GDN_STATIC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}

}  // namespace gdn
