// kda_prefill_ext.hip -- the fused prefill kernel (kda_prefill_kernel.h) with the
// unbounded gate and/or raw inputs, in a translation unit of its own.
#include "kda_prefill_kernel.h"

namespace kda {

hipError_t launch_fwd_ext(const FwdParams &p, bool bf16_in, bool f32_compute, bool unb, bool raw,
                          hipStream_t stream) {
  if (bf16_in && f32_compute) {  // raw inputs need fp32 inputs for fp32 arithmetic
    if (raw || !unb) return hipErrorInvalidValue;
    return launch_fwd_t<bf16_t, true, true, false>(p, stream);
  }
  if (bf16_in) {
    if (unb)
      return raw ? launch_fwd_t<bf16_t, false, true, true>(p, stream)
                 : launch_fwd_t<bf16_t, false, true, false>(p, stream);
    return launch_fwd_t<bf16_t, false, false, true>(p, stream);
  }
  if (!f32_compute) return hipErrorInvalidValue;  // fp32 inputs take fp32 arithmetic
  if (unb)
    return raw ? launch_fwd_t<float, true, true, true>(p, stream)
               : launch_fwd_t<float, true, true, false>(p, stream);
  return launch_fwd_t<float, true, false, true>(p, stream);
}

}  // namespace kda
