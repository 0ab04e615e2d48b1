// Link-time stand-ins for the HIP runtime and the kernel launchers, so that the
// host side of libkda (argument validation, planning, workspace layout in
// kda_api.cpp) can be built and run on a CPU under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every launcher records the call and fails, so a
// call that reaches a launch returns KDA_ERR_HIP without touching any memory.
#include <hip/hip_runtime.h>

#include "../../linear_attention_fwd_amd/csrc/kda_launch.h"

int g_launches = 0;

extern "C" {
const char *hipGetErrorString(hipError_t) { return "stubbed HIP runtime"; }
hipError_t hipGetDevice(int *dev) {
  *dev = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int *value, hipDeviceAttribute_t, int) {
  *value = 256;
  return hipSuccess;
}
// Streams live on device 0, except the handle 0x2000, which stands for a
// stream of device 1.
hipError_t hipStreamGetDevice(hipStream_t stream, hipDevice_t *device) {
  *device = (uintptr_t)stream == 0x2000 ? 1 : 0;
  return hipSuccess;
}
}

namespace kda {
static hipError_t launched() {
  ++g_launches;
  return hipErrorInvalidValue;
}
hipError_t launch_fwd(FwdParams, bool, bool, int, bool, hipStream_t) { return launched(); }
hipError_t launch_chunk_prep(const SplitParams &, hipStream_t) { return launched(); }
hipError_t launch_chunk_recurrence(const SplitParams &, hipStream_t) { return launched(); }
hipError_t launch_copy_empty(const int32_t *, int64_t, const float *, float *, int, int,
                             hipStream_t) {
  return launched();
}
hipError_t launch_pair_scan(const float *, const float *, const int32_t *, int, int, int, int64_t,
                            float *, hipStream_t) {
  return launched();
}
hipError_t launch_scan_chains(const ScanChains &, int, hipStream_t) { return launched(); }
hipError_t noalloc_scratch(void **) { return launched(); }
template <typename Tin>
hipError_t launch_decode(float *, const int32_t *, const void *, const void *, const void *,
                         const void *, const void *, const int32_t *, int, const void *,
                         const void *, const void *, const void *, const void *,
                         const DecodeWindowArgs &, bool, const float *, float, int, void *,
                         int32_t *, int, int, int, hipStream_t) {
  return launched();
}
template hipError_t launch_decode<float>(float *, const int32_t *, const void *, const void *,
                                         const void *, const void *, const void *,
                                         const int32_t *, int, const void *, const void *,
                                         const void *, const void *, const void *,
                                         const DecodeWindowArgs &, bool, const float *, float,
                                         int, void *, int32_t *, int, int, int, hipStream_t);
template hipError_t launch_decode<bf16_t>(float *, const int32_t *, const void *, const void *,
                                          const void *, const void *, const void *,
                                          const int32_t *, int, const void *, const void *,
                                          const void *, const void *, const void *,
                                          const DecodeWindowArgs &, bool, const float *, float,
                                          int, void *, int32_t *, int, int, int, hipStream_t);
}  // namespace kda
