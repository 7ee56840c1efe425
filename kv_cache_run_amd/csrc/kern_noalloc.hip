// Static device scratch of art_decode_noalloc, for callers that cannot
// allocate device memory (HIP graph capture, tight serving loops, harnesses
// that forbid hipMalloc).  One array per device, held until the process ends;
// its device address is looked up once per device with that device current.
#include <hip/hip_runtime.h>

#include <mutex>

#include "art_internal.h"

namespace art {
namespace {

constexpr size_t kScratchBytes = size_t(8) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[64] = {};

}  // namespace

size_t noalloc_scratch_bytes() { return kScratchBytes; }

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace art
