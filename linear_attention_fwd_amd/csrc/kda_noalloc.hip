// kda_noalloc.hip -- device scratch for kda_chunk_fwd_noalloc.
//
// kda_chunk_fwd_noalloc runs the two-kernel prefill of kda_chunk_fwd with its
// workspace (the chunk images and the document order) in this file-scope
// device array instead of caller memory, for callers that cannot allocate.
// Each GPU the library runs on holds its own copy of the array until the
// process ends.  In host code the array's name is only a stand-in: its device
// address is looked up once per device with hipGetSymbolAddress and cached.
#include <mutex>

#include "kda_launch.h"

namespace kda {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *cache[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!cache[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    cache[dev] = p;
  }
  *ptr = cache[dev];
  return hipSuccess;
}

}  // namespace kda
