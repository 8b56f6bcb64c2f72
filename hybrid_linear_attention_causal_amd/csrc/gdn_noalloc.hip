// Device scratch of the allocation-free chunked prefill (gdn_chunk_prefill_noalloc): the
// workspace that gdn_chunk_prefill takes from its caller lives here in a fixed device array
// instead, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope __device__ object: each device the library runs on holds its
// own copy, at its own address, until the process ends.  In host code its name is only a
// host-side stand-in, so the device address is looked up once per device with
// hipGetSymbolAddress (with that device current) and that address is what the launches
// receive.  Every call on one device shares the array; calls that overlap on one device
// (two streams, or two host threads) race on it.  The chunked prefill needs none of it
// cleared: every byte it reads was written earlier in the same call.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn_launch.hpp"

namespace gdn {

static __device__ __align__(256) uint8_t scratch[NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDev = 64;
std::mutex g_mu;
void* g_ptr[kMaxDev];   // device address of scratch on each device, once looked up
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_mu);
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

}  // namespace gdn
